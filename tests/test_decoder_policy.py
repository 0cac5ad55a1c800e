"""Host-side launch-form choices of SparseDecoder (no GPU work: the buffers
are allocated on the CPU and no kernel is called)."""
from sparse_kv_cache_amd.decode import ONE_LAUNCH_ROWS, SparseDecoder


def _dec(B, H_q=32, H_kv=8, bt_ld=512, num_splits=8, **kw):
    return SparseDecoder(B, H_q, H_kv, 128, 4096, 16, bt_ld, topk_pages=64,
                         num_splits=num_splits, device="cpu", **kw)


def test_one_launch_up_to_the_resident_row_count():
    # score + select + decode + merge in one launch while every block of it
    # fits on the device at once; past that, scoring is a launch of its own
    assert ONE_LAUNCH_ROWS == 512
    d = _dec(16)                                  # 512 query rows
    assert d.fused and d.select_in_decode and d.score_in_decode
    d = _dec(17)                                  # 544
    assert d.fused and d.select_in_decode and not d.score_in_decode
    d = _dec(128)                                 # the high_batch shape
    assert d.fused and d.select_in_decode and not d.score_in_decode


def test_launch_forms_by_splits_rows_and_selection():
    assert not _dec(8, num_splits=16).fused       # more splits than a block's waves
    # ... then the selection runs inside the split decode, rows up to 8192
    assert _dec(8, num_splits=16).select_in_split_decode
    assert _dec(1, H_q=64, num_splits=64, bt_ld=8192).select_in_split_decode
    assert not _dec(1, H_q=64, num_splits=64, bt_ld=8193).select_in_split_decode
    assert not _dec(8).select_in_split_decode     # merged in-block instead
    # whose blocks merge their 16 splits: a head's 64 splits leave 4 partials
    d = _dec(1, H_q=64, num_splits=64)
    assert d.split_blocks and tuple(d.o_blk.shape) == (1, 64, 4, 128)
    assert tuple(d.lse_blk.shape) == (1, 64, 4)
    assert d.partials[0] is d.o_part              # until a decode has run
    assert _dec(8).o_blk is None
    assert not _dec(8, num_splits=16, group_select=True).select_in_split_decode
    assert not _dec(8, bt_ld=5000).select_in_decode
    d = _dec(8, group_select=True)                # one selection per kv head
    assert not d.fused and not d.score_in_decode
    assert d.decode_splits == min(8, 256 // (8 * 8))
    d = _dec(8, bt_ld=4096)
    assert d.score_in_decode                      # scores + selection fit 48 KiB of LDS
