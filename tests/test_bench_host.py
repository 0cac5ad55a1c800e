"""bench.py's host-side logic on the CPU: the refusal of more than one GPU,
the algorithmic byte counts behind roofline.achieved, and the gating of the
committed counter records by kernel name and source hash."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
import bench  # noqa: E402
from sparse_kv_cache_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    # refused before torch or the GPU is touched
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _tiny():
    # one request of 40 tokens: pages of 16, 16 and 8 valid rows; 2 kv heads,
    # 2 query heads each, D = 64
    wl = W.small_case(seed=0, B=1, H_q=4, H_kv=2, D=64, P=16, max_pages=3)
    wl.seq_lens = np.array([40], dtype=np.int32)
    sel = np.full((1, 4, 3), -1, np.int32)
    cnt = np.zeros((1, 4), np.int32)
    sel[0, 0, :2] = [0, 2]; cnt[0, 0] = 2      # kv head 0: {0, 2} and {2}
    sel[0, 1, :1] = [2]; cnt[0, 1] = 1
    sel[0, 2, :1] = [1]; cnt[0, 2] = 1         # kv head 1: {1} twice
    sel[0, 3, :1] = [1]; cnt[0, 3] = 1
    return wl, sel, cnt


def test_unique_kv_bytes_counts_a_shared_page_once_over_its_valid_rows():
    wl, sel, cnt = _tiny()
    kv, pages = bench.unique_kv_bytes(wl, sel, cnt, wl.seq_lens, wl.H_q)
    assert pages == 3                                # (h0, p0), (h0, p2), (h1, p1)
    assert kv == (16 + 8 + 16) * 64 * 2 * 2          # rows x D x bf16 x (K and V)


def test_kernel_bytes_of_the_separate_launches():
    wl, sel, cnt = _tiny()
    kb, pages = bench.kernel_bytes(wl, sel, cnt, wl.seq_lens, 2, False)
    # statistics 8 bytes a dim (bf16 min and max, fp32 mean) for 3 pages x 2
    # kv heads, a score per page and query head, a block id per page, q once
    assert kb["page_score"] == 3 * (2 * 8 * 64 + 4 * 4 + 4) + 4 * 64 * 4
    # the score rows read, the 5 selected indices written
    assert kb["page_topk"] == 3 * 4 * 4 + 5 * 4
    kv = (16 + 8 + 16) * 64 * 2 * 2
    # K/V once, q, the indices, 2 split partials of D + 1 floats per query head
    assert kb["sparse_paged_decode"] == kv + 4 * 64 * 4 + 5 * 4 + 4 * 2 * 65 * 4
    assert kb["lse_merge"] == 4 * 2 * 65 * 4 + 4 * 65 * 4
    fused, _ = bench.kernel_bytes(wl, sel, cnt, wl.seq_lens, 2, False, fused=True)
    assert "lse_merge" not in fused
    assert fused["sparse_paged_decode"] == kv + 4 * 64 * 4 + 5 * 4 + 4 * 65 * 4


def _record(tag):
    text = open(os.path.join(ROOT, "profiles", f"traffic_{tag}.md")).read()
    start = text.find("```json")
    return json.loads(text[start + 7:text.find("```", start + 7)].strip())


def test_counter_records_are_gated_by_kernel_and_source_hash(monkeypatch):
    recs = _record("gqa_ragged")
    # the step's main launch, then the decode timed alone
    assert isinstance(recs, list) and len(recs) == 2
    main, alone = recs
    assert main["kernel"] == "sparse_page_decode"
    assert alone["kernel"] == "sparse_paged_decode_merged"
    monkeypatch.setattr(bench, "decode_source_hash", lambda kind="softmax": main["source_sha1"])
    assert bench.profiled_traffic("gqa_ragged", "softmax", main["kernel"]) == main["traffic"]
    assert bench.profiled_traffic("gqa_ragged", "softmax", alone["kernel"]) == alone["traffic"]
    assert bench.profiled_traffic("gqa_ragged", "softmax") == main["traffic"]
    assert bench.profiled_traffic("gqa_ragged", "softmax", "some_other_kernel") is None
    assert bench.profiled_traffic("no_such_workload") is None
    # a single record (workloads whose step has no separately timed decode)
    one = _record("high_batch")
    assert isinstance(one, dict)
    assert bench.profiled_traffic("high_batch", "softmax", one["kernel"]) == one["traffic"]
    monkeypatch.setattr(bench, "decode_source_hash", lambda kind="softmax": "0" * 40)
    assert bench.profiled_traffic("gqa_ragged", "softmax", main["kernel"]) is None
    assert bench.profiled_traffic("gqa_ragged", "softmax", alone["kernel"]) is None


def test_cpu_baseline_request_copy_gives_the_same_step():
    """The oracle baseline runs each sampled request on a compact copy of its
    own blocks: the step's output must equal the step over the whole pool."""
    import oracle
    wl = W.small_case(seed=5, B=3, H_q=4, H_kv=2, D=64, P=16, max_pages=6,
                      num_blocks=200, topk_pages=3)
    rng = np.random.default_rng(1)
    cache = rng.integers(0x3c00, 0x4100, size=(2, wl.num_blocks, wl.P, wl.H_kv, wl.D),
                         dtype=np.uint16)
    q = rng.standard_normal((wl.B, wl.H_q, wl.D))
    kc = min(max(wl.topk_pages, wl.bos + wl.eos), wl.bt_ld)
    for bb in range(wl.B):
        sl = wl.seq_lens[bb:bb + 1]
        bt = wl.block_table[bb:bb + 1]
        full = oracle.decode_step(q[bb:bb + 1], cache, bt, sl,
                                  oracle.page_stats(cache, bt, sl, wl.P), wl.w_avg,
                                  wl.w_peak, wl.topk_pages, 0.0, wl.bos, wl.eos,
                                  wl.softmax_scale, kc)
        cc, bc = bench.compact_request(wl, cache, wl.seq_lens, bb)
        assert cc.shape[1] == (int(sl[0]) + wl.P - 1) // wl.P
        part = oracle.decode_step(q[bb:bb + 1], cc, bc, sl, oracle.page_stats(cc, bc, sl, wl.P),
                                  wl.w_avg, wl.w_peak, wl.topk_pages, 0.0, wl.bos, wl.eos,
                                  wl.softmax_scale, kc)
        for a, b in zip(full, part):
            assert np.array_equal(np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64),
                                  equal_nan=True)
