"""h2o_accumulate_noalloc (the token-level accumulator step with the
library's fixed scratch buffer) against h2o_accumulate with a caller-owned
scratch: the same hh bytes and score rows, on two calls in a row (the second
smaller, so the fixed buffer still holds the first call's larger contents),
through the C ABI.  Also: a step whose scratch would not fit the fixed buffer
is refused before anything is written, and an empty batch is a no-op."""
import numpy as np
import pytest
import torch

import sparse_kv_cache_amd as skv
from sparse_kv_cache_amd import workloads as W
from parity import bits, dev, say

pytestmark = pytest.mark.gpu


def _compare(wl, step):
    say(f"[gpu] h2o_accumulate_noalloc vs h2o_accumulate: B={wl.B}, tokens "
        f"{int(wl.seq_lens_at(step).max())}, bt_ld {wl.bt_ld}")
    cache = W.make_cache(wl, device="cuda")
    hh0 = W.make_hh(wl, device="cuda")
    # a decayed history on the prompt slots, so the update has bits to keep
    hh0.copy_((torch.rand(hh0.shape, device="cuda") * 0.05).to(torch.bfloat16))
    q = dev(W.make_queries(wl, step))
    bt, sl = dev(wl.block_table), dev(wl.seq_lens_at(step))
    ld = wl.bt_ld
    nan = float("nan")
    sc_ref = torch.full((wl.B, wl.H_kv, ld), nan, device="cuda")
    sc_new = torch.full((wl.B, wl.H_kv, ld), nan, device="cuda")
    hh_ref, hh_new = hh0.clone(), hh0.clone()
    scratch = torch.empty(skv.h2o_scratch_floats(wl.B, wl.H_kv, ld), device="cuda")
    skv.h2o_accumulate(q, cache, bt, sl, hh_ref, sc_ref, scratch, wl.softmax_scale,
                       wl.decay, wl.bos, wl.eos)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    skv.h2o_accumulate_noalloc(q, cache, bt, sl, hh_new, sc_new, wl.softmax_scale,
                               wl.decay, wl.bos, wl.eos)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert np.array_equal(bits(hh_new), bits(hh_ref)), "hh differs"
    assert not np.array_equal(bits(hh_new), bits(hh0)), "the step changed nothing"
    a, b = sc_new.cpu().numpy(), sc_ref.cpu().numpy()
    assert np.array_equal(a, b, equal_nan=True), "score rows differ"
    for r in range(wl.B):
        n = int(wl.seq_lens_at(step)[r])
        assert np.isfinite(a[r, :, :n]).all() and np.isnan(a[r, :, n:]).all()


def test_noalloc_matches_caller_scratch_then_smaller():
    # the token-level workload's own shape first (4 requests, 4097-token rows)
    _compare(W.h2o_token(), 0)
    # then a smaller step: 3 requests of ragged length, shorter rows, other
    # window (the fixed buffer still holds the larger call's values)
    wl = W.h2o_token(seed=11, steps=8, prompt=700, B=3)
    wl.seq_lens = np.array([700, 313, 65], dtype=np.int32)
    wl.bos, wl.eos = 4, 8
    _compare(wl, 5)


def test_noalloc_refuses_a_step_beyond_its_buffer():
    say("[gpu] h2o_accumulate_noalloc: oversize step refused")
    H_kv, ld = 8, 262144            # 8 * 262144 logits alone fill the buffer
    assert skv.h2o_scratch_floats(1, H_kv, ld) > skv.NOALLOC_SCRATCH_FLOATS
    cache = torch.zeros((2, 4, 1, H_kv, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((1, ld), dtype=torch.int32, device="cuda")
    sl = torch.ones((1,), dtype=torch.int32, device="cuda")
    hh = torch.full((4, H_kv), 3.0, dtype=torch.bfloat16, device="cuda")
    sc = torch.full((1, H_kv, ld), float("nan"), device="cuda")
    q = torch.zeros((1, 32, 128), device="cuda")
    with pytest.raises(skv.SparseKVError) as e:
        skv.h2o_accumulate_noalloc(q, cache, bt, sl, hh, sc, 0.1)
    assert e.value.code == -22 and "fixed buffer" in str(e.value)
    torch.cuda.synchronize()
    assert (hh.float() == 3.0).all() and torch.isnan(sc).all()


def test_noalloc_empty_batch_is_a_no_op():
    say("[gpu] h2o_accumulate_noalloc: empty batch")
    cache = torch.zeros((2, 4, 1, 8, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((0, 16), dtype=torch.int32, device="cuda")
    sl = torch.zeros((0,), dtype=torch.int32, device="cuda")
    hh = torch.full((4, 8), 3.0, dtype=torch.bfloat16, device="cuda")
    sc = torch.zeros((0, 8, 16), device="cuda")
    q = torch.zeros((0, 32, 128), device="cuda")
    skv.h2o_accumulate_noalloc(q, cache, bt, sl, hh, sc, 0.1)
    torch.cuda.synchronize()
    assert (hh.float() == 3.0).all()
