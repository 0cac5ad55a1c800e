"""The binding refuses tensors of the wrong shape before any launch.

Every case builds a consistent set of small device tensors and calls the
wrapper against a stub library that only records calls: the consistent set
must reach the library.  Then ONE tensor is replaced by one of the wrong
shape: the wrapper must raise ValueError and the stub must not be reached, so
nothing can have been enqueued.  No kernel runs in this file.  (The tensors
live on the GPU because the wrappers refuse host tensors before they look at
shapes.)"""
import math

import pytest
import torch

import sparse_kv_cache_amd as skv
from parity import say

pytestmark = pytest.mark.gpu

B, H_Q, H_KV, D, P, NB, LD, K_CAP, NS = 2, 8, 2, 64, 16, 16, 8, 4, 2
# splits of the block-merged split decode: more than one block of them
NS_BLK = 40


def _buffers():
    f32, i32, bf = torch.float32, torch.int32, torch.bfloat16
    z = lambda shape, dt=f32: torch.zeros(shape, dtype=dt, device="cuda")
    nblk = skv.sparse_select_decode_split_blocks_count(NS_BLK, P)
    assert 1 < nblk < NS_BLK
    t = dict(
        q=z((B, H_Q, D)), kv=z((2, NB, P, H_KV, D), bf),
        kmin=z((NB, H_KV, D), bf), kmax=z((NB, H_KV, D), bf), kmean=z((NB, H_KV, D)),
        kvar=z((NB, H_KV, D)), bt=z((B, LD), i32), sl=torch.full((B,), 16, dtype=i32,
                                                                 device="cuda"),
        scores=z((B, H_Q, LD)), gscores=z((B, H_KV, LD)),
        sel_idx=z((B, H_Q, K_CAP), i32), sel_cnt=z((B, H_Q), i32),
        sel_blk=z((B, H_Q, K_CAP), i32), o_part=z((B, H_Q, NS, D)),
        lse_part=z((B, H_Q, NS)), o_blk=z((B, H_Q, nblk, D)), lse_blk=z((B, H_Q, nblk)),
        out=z((B, H_Q, D)), lse=z((B, H_Q)),
        tau=z((B, H_Q)), hh=z((NB * P, H_KV), bf), scratch=z((4096,)),
        mu=z((B, H_Q, LD)), var=z((B, H_Q, LD)), est=z((B, H_Q, LD)),
        knew=z((B, H_KV, D), bf),
        gsel_idx=z((B, H_KV, K_CAP), i32), gsel_cnt=z((B, H_KV), i32),
        gsel_blk=z((B, H_KV, K_CAP), i32),
    )
    return t


def _calls(t):
    s = 0.125
    return {
        "page_score": lambda: skv.page_score(t["q"], t["kmin"], t["kmax"], t["kmean"],
                                             t["bt"], t["sl"], P, 1.0, 1.0, t["scores"]),
        "page_score_ex": lambda: skv.page_score_ex(t["q"], t["kmin"], t["kmax"], t["kmean"],
                                                   t["bt"], t["sl"], P, 1.0, 1.0,
                                                   t["scores"]),
        "page_score_group": lambda: skv.page_score_group(t["q"], t["kmin"], t["kmax"],
                                                         t["kmean"], t["bt"], t["sl"], P,
                                                         1.0, 1.0, t["gscores"]),
        "page_topk": lambda: skv.page_topk(t["scores"], t["sl"], P, 2, t["sel_idx"],
                                           t["sel_cnt"]),
        "page_topk_blk": lambda: skv.page_topk_blk(t["scores"], t["sl"], P, 2, t["sel_idx"],
                                                   t["sel_cnt"], t["bt"], t["sel_blk"]),
        "sparse_paged_decode": lambda: skv.sparse_paged_decode(
            t["q"], t["kv"], t["bt"], t["sl"], t["sel_idx"], t["sel_cnt"], s, t["o_part"],
            t["lse_part"]),
        "sparse_paged_decode_ex": lambda: skv.sparse_paged_decode_ex(
            t["q"], t["kv"], t["bt"], t["sl"], t["sel_idx"], t["sel_cnt"], s, t["o_part"],
            t["lse_part"], sel_blk=t["sel_blk"]),
        "sparse_paged_decode_merged": lambda: skv.sparse_paged_decode_merged(
            t["q"], t["kv"], t["bt"], t["sl"], t["sel_idx"], t["sel_cnt"], s, NS, t["out"],
            t["lse"], o_part=t["o_part"], lse_part=t["lse_part"], sel_blk=t["sel_blk"]),
        "sparse_select_decode": lambda: skv.sparse_select_decode(
            t["scores"], t["q"], t["kv"], t["bt"], t["sl"], 2, K_CAP, s, NS, t["out"],
            t["lse"], sel_idx=t["sel_idx"], sel_cnt=t["sel_cnt"], sel_blk=t["sel_blk"]),
        "sparse_page_decode": lambda: skv.sparse_page_decode(
            t["q"], t["kv"], t["kmin"], t["kmax"], t["kmean"], t["bt"], t["sl"], 1.0, 1.0, 2,
            K_CAP, s, NS, t["out"], t["lse"], scores=t["scores"], sel_idx=t["sel_idx"],
            sel_cnt=t["sel_cnt"], sel_blk=t["sel_blk"]),
        "lse_merge": lambda: skv.lse_merge(t["o_part"], t["lse_part"], t["out"], t["lse"]),
        "h2o_accumulate": lambda: skv.h2o_accumulate(
            t["q"], t["kv"], t["bt"], t["sl"], t["hh"], t["gscores"], t["scratch"], s),
        "entmax15_paged_decode": lambda: skv.entmax15_paged_decode(
            t["q"], t["kv"], t["bt"], t["sl"], t["sel_idx"], t["sel_cnt"], s, t["o_part"],
            t["lse_part"], t["scratch"]),
        "entmax15_paged_decode_merged": lambda: skv.entmax15_paged_decode_merged(
            t["q"], t["kv"], t["bt"], t["sl"], t["sel_idx"], t["sel_cnt"], s, t["out"],
            lse_out=t["lse"], tau_out=t["tau"]),
        "gauss_moments": lambda: skv.gauss_moments(t["q"], t["kmean"], t["kvar"], t["bt"],
                                                   t["sl"], P, s, t["mu"], t["var"]),
        "gauss_select": lambda: skv.gauss_select(t["mu"], t["var"], t["sl"], P, t["bt"], False,
                                                 K_CAP, t["est"], t["sel_idx"], t["sel_cnt"],
                                                 tau=t["tau"], sel_blk=t["sel_blk"]),
        "pagestats_update": lambda: skv.pagestats_update(t["kv"], t["kmin"], t["kmax"],
                                                         t["kmean"], t["bt"], t["sl"],
                                                         t["knew"], t["knew"]),
        "sparse_select_decode_split": lambda: skv.sparse_select_decode_split(
            t["scores"], t["q"], t["kv"], t["bt"], t["sl"], 2, K_CAP, s, t["o_part"],
            t["lse_part"], sel_idx=t["sel_idx"], sel_cnt=t["sel_cnt"], sel_blk=t["sel_blk"]),
        "sparse_select_decode_split_blocks": lambda: skv.sparse_select_decode_split_blocks(
            t["scores"], t["q"], t["kv"], t["bt"], t["sl"], 2, K_CAP, s, NS_BLK, t["o_blk"],
            t["lse_blk"], sel_idx=t["sel_idx"], sel_cnt=t["sel_cnt"], sel_blk=t["sel_blk"]),
        "sparse_select_decode_group": lambda: skv.sparse_select_decode_group(
            t["gscores"], t["q"], t["kv"], t["bt"], t["sl"], 2, K_CAP, s, t["o_part"],
            t["lse_part"], sel_idx=t["gsel_idx"], sel_cnt=t["gsel_cnt"],
            sel_blk=t["gsel_blk"]),
        "h2o_select_decode": lambda: skv.h2o_select_decode(
            t["q"], t["kv"], t["bt"], t["sl"], t["hh"], t["scratch"], s, 2, K_CAP,
            t["o_part"], t["lse_part"], scores=t["gscores"], sel_idx=t["gsel_idx"],
            sel_cnt=t["gsel_cnt"], sel_blk=t["gsel_blk"], k_new=t["knew"], v_new=t["knew"]),
    }


# (entry point, tensor replaced, wrong shape)
CASES = [
    ("page_score", "sl", (B + 1,)), ("page_score", "bt", (B + 1, LD)),
    ("page_score", "kmax", (NB, H_KV, 2 * D)), ("page_score", "kmean", (NB + 1, H_KV, D)),
    ("page_score", "scores", (B, H_KV, LD)),
    ("page_score_ex", "kmin", (NB, H_KV, 2 * D)),
    ("page_score_group", "gscores", (B, H_Q, LD)), ("page_score_group", "sl", (B - 1,)),
    ("page_topk", "sl", (B + 1,)), ("page_topk", "sel_cnt", (B, H_Q + 1)),
    ("page_topk", "sel_idx", (B + 1, H_Q, K_CAP)),
    ("page_topk_blk", "sel_blk", (B, H_Q, K_CAP + 1)), ("page_topk_blk", "bt", (B + 1, LD)),
    ("sparse_paged_decode", "o_part", (B, H_Q, NS, D + 8)),
    ("sparse_paged_decode", "lse_part", (B, H_Q, NS + 1)),
    ("sparse_paged_decode", "sel_cnt", (B, H_Q - 1)),
    ("sparse_paged_decode", "sel_idx", (B, 3, K_CAP)),
    ("sparse_paged_decode", "sl", (B + 1,)), ("sparse_paged_decode", "bt", (B - 1, LD)),
    ("sparse_paged_decode", "kv", (2, NB, P, H_KV, 2 * D)),
    ("sparse_paged_decode_ex", "sel_blk", (B, H_Q, K_CAP - 1)),
    ("sparse_paged_decode_merged", "out", (B, H_Q, D - 8)),
    ("sparse_paged_decode_merged", "lse", (B, H_Q + 1)),
    ("sparse_paged_decode_merged", "sel_blk", (B, H_Q, K_CAP + 2)),
    ("sparse_paged_decode_merged", "lse_part", (B, H_Q, NS - 1)),
    ("sparse_paged_decode_merged", "sel_cnt", (B + 1, H_Q)),
    ("sparse_select_decode", "out", (B, H_Q, 2 * D)),
    ("sparse_select_decode", "lse", (B + 1, H_Q)),
    ("sparse_select_decode", "sel_cnt", (B, H_KV)),
    ("sparse_select_decode", "sl", (B + 2,)),
    ("sparse_select_decode", "scores", (B, H_KV, LD)),
    ("sparse_page_decode", "kmin", (NB - 1, H_KV, D)),
    ("sparse_page_decode", "kmean", (NB, H_KV, D // 2)),
    ("sparse_page_decode", "out", (B, H_Q - 1, D)),
    ("sparse_page_decode", "sel_blk", (B, H_Q, K_CAP - 1)),
    ("sparse_page_decode", "scores", (B, H_Q, LD + 1)),
    ("lse_merge", "lse_part", (B, H_Q, NS + 1)), ("lse_merge", "out", (B, H_Q, D + 1)),
    ("lse_merge", "lse", (B, H_Q - 1)),
    ("h2o_accumulate", "sl", (B + 1,)), ("h2o_accumulate", "gscores", (B, H_Q, LD)),
    ("h2o_accumulate", "hh", (NB * P + 1, H_KV)), ("h2o_accumulate", "bt", (B + 1, LD)),
    ("entmax15_paged_decode", "o_part", (B + 1, H_Q, NS, D)),
    ("entmax15_paged_decode", "sel_cnt", (B, H_Q + 2)),
    ("entmax15_paged_decode_merged", "tau", (B, H_Q + 1)),
    ("entmax15_paged_decode_merged", "out", (B + 1, H_Q, D)),
    ("gauss_moments", "kvar", (NB, H_KV + 1, D)), ("gauss_moments", "sl", (B - 1,)),
    ("gauss_select", "tau", (B, H_Q - 1)), ("gauss_select", "sel_idx", (B, H_Q, K_CAP + 1)),
    ("gauss_select", "sel_blk", (B, H_Q, K_CAP - 1)), ("gauss_select", "bt", (B + 1, LD)),
    ("pagestats_update", "knew", (B, H_KV, D + 8)), ("pagestats_update", "bt", (B + 1, LD)),
    ("sparse_select_decode_split", "scores", (B, H_KV, LD)),
    ("sparse_select_decode_split", "o_part", (B, H_Q, NS, D + 8)),
    ("sparse_select_decode_split", "sel_idx", (B, H_KV, K_CAP)),
    ("sparse_select_decode_split", "sl", (B + 1,)),
    ("sparse_select_decode_split_blocks", "o_blk", (B, H_Q, NS_BLK, D)),
    ("sparse_select_decode_split_blocks", "lse_blk", (B, H_Q - 1, 1)),
    ("sparse_select_decode_split_blocks", "scores", (B, H_KV, LD)),
    ("sparse_select_decode_group", "gscores", (B, H_Q, LD)),
    ("sparse_select_decode_group", "gsel_cnt", (B, H_Q)),
    ("sparse_select_decode_group", "lse_part", (B, H_Q, NS + 1)),
    ("h2o_select_decode", "knew", (B, H_KV + 1, D)),
    ("h2o_select_decode", "hh", (NB * P - 1, H_KV)),
    ("h2o_select_decode", "gsel_idx", (B, H_Q, K_CAP)),
    ("h2o_select_decode", "gscores", (B + 1, H_KV, LD)),
]


class _StubLibrary:
    """Stands in for libsparsekv.so: records the entry points called, returns 0.
    Size queries, which only do host arithmetic, go to the real library."""

    QUERIES = ("sparse_select_decode_split_blocks_count",)

    def __init__(self, real):
        self.calls = []
        self.real = real

    def __getattr__(self, name):
        if name in self.QUERIES:
            return getattr(self.real, name)

        def entry(*args):
            self.calls.append(name)
            return 0
        return entry


@pytest.fixture
def stub(monkeypatch):
    lib = _StubLibrary(skv.load_library())
    monkeypatch.setattr(skv, "_lib", lib)
    return lib


@pytest.mark.parametrize("fn,name,shape", CASES,
                         ids=[f"{f}-{n}" for f, n, _ in CASES])
def test_wrong_shape_is_refused_before_launch(stub, fn, name, shape):
    t = _buffers()
    _calls(t)[fn]()
    assert stub.calls == [fn], "the consistent arguments must reach the library"
    stub.calls.clear()
    good = t[name]
    t[name] = torch.zeros(shape, dtype=good.dtype, device="cuda")
    with pytest.raises(ValueError):
        _calls(t)[fn]()
    assert stub.calls == [], f"{fn} reached the library with a wrong {name}"


def test_every_wrapper_is_covered(stub):
    say("[gpu] shape-check table")
    calls = _calls(_buffers())
    assert {f for f, _, _ in CASES} == set(calls)
    assert math.prod((B, H_Q)) > 0
