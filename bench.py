#!/usr/bin/env python3
"""Decode-step throughput of page-scored sparse attention on one MI355X.

One step = one pass of the whole hot path over the batch:
  page level (default gqa_ragged, also mha_tiny / long_context):
      page_score -> page_topk -> sparse_paged_decode -> lse_merge
      (with one selection per query head and at most 8 splits the merge runs
      inside the decode launch: sparse_paged_decode_merged; with more splits
      the selection runs inside the split decode, whose blocks also merge
      their splits, sparse_select_decode_split_blocks, and lse_merge follows)
      (statistics built once beforehand, timed separately)
  high_batch: pagestats_update (append + refresh) -> the four above
  h2o_token:  pagestats_update (append + reset) -> h2o_accumulate ->
      page_topk -> sparse_paged_decode -> lse_merge
      (as h2o_select_decode, the append and the accumulator's logits in one
      launch, the update, selection and decode in another, then lse_merge)

Inputs are seeded synthetic tensors already resident in HBM.  To measure
HBM rather than the 256 MB memory-side cache, the timed steps rotate over R
replicas of the workload (separate caches, statistics and buffers, like the
layers of a model), so each step's data was last touched R-1 steps earlier.
The timed steps are one HIP graph replay (exactly K steps), bracketed by HIP
events and device synchronisation.

Prints ONE JSON line: steps/s (value), effective HBM GB/s of the step and of
each kernel (algorithmic bytes / kernel time; each kernel is timed alone,
launched back to back over the replicas in a graph, with HIP events on the
launch stream), the roofline entry of the decode kernel, and the float64
oracle timed on a bounded sample on the host cores (cpu_baseline).

The roofline entry also places the decode kernel against two references of
the library that carry no arithmetic, timed the same way in the same run:
the streaming read of the kernel's byte count (stream_ref / stream_frac) and
the gather-only read of the decode's own page-heads (gather_ref /
gather_frac).  Unless --no-long-context (or --workload long_context), the
line also carries a "long_context" record: the long-context workload's step
rate (one request of 131,072 tokens, 64 query heads), its decode kernel's
time, bytes, fraction of peak and ratio to the references (timed alone over
the step's selection where the step fuses it), and the step's main launch
with its counter traffic.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa_ragged",
                    choices=["mha_tiny", "gqa_ragged", "h2o_token", "long_context",
                             "high_batch"])
    ap.add_argument("--replicas", type=int, default=0,
                    help="rotation depth (0 = enough to exceed 1 GiB per cycle)")
    ap.add_argument("--splits", type=int, default=0, help="override num_splits")
    ap.add_argument("--select", default="head", choices=["head", "group", "gauss"],
                    help="page level: top-k per query head, or once per kv head "
                         "from the group's mean score (shared by the group), or the "
                         "Gaussian-aware adaptive selection per query head (attends "
                         "with 1.5-entmax)")
    ap.add_argument("--alibi", action="store_true",
                    help="page level: standard ALiBi slopes 2^(-8(i+1)/H_q) in scoring "
                         "and decode")
    ap.add_argument("--attention", default="softmax", choices=["softmax", "entmax15"],
                    help="page level: softmax, or 1.5-entmax over the same selection")
    ap.add_argument("--h2o-softmax", default="group_mean", choices=["group_mean", "per_head"],
                    help="token level: softmax of the group-mean query, or every query "
                         "head's own softmax averaged over the group")
    ap.add_argument("--no-fuse", action="store_true",
                    help="keep page_topk and lse_merge as their own launches even "
                         "where the decode can select and merge in-block")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long-context", action="store_true",
                    help="skip the long_context sub-record that the default run adds")
    ap.add_argument("--no-graph", action="store_true",
                    help="enqueue kernel by kernel instead of replaying HIP graphs")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--repeats", type=int, default=5,
                    help="extra replays of the timed steps for the p10/p50/p90 spread")
    return ap.parse_args()


# ------------------------------------------------------ algorithmic bytes

def unique_kv_bytes(wl, sel_idx, sel_cnt, seq_lens, H_sel):
    """K+V bytes of every distinct (request, kv head, page) selected, counted
    once, over its valid rows."""
    G_sel = wl.H_q // H_sel if H_sel == wl.H_q else 1
    total = 0
    pages_total = 0
    for b in range(wl.B):
        S = int(seq_lens[b])
        for h in range(wl.H_kv):
            if H_sel == wl.H_q:
                rows = range(h * wl.G, (h + 1) * wl.G)
            else:
                rows = [h]
            u = set()
            for r in rows:
                u.update(sel_idx[b, r, :sel_cnt[b, r]].tolist())
            pages = np.fromiter(u, dtype=np.int64, count=len(u))
            n = np.minimum(wl.P, S - pages * wl.P)
            total += int(n.sum()) * wl.D * 2 * 2
            pages_total += len(u)
    del G_sel
    return total, pages_total


def kernel_bytes(wl, sel_idx, sel_cnt, seq_lens, num_splits, token_level,
                 group_select=False, fused=False, entmax=False, gauss=False,
                 h2o_per_head=False):
    """Algorithmic HBM bytes of each kernel of one step: the bytes the
    operation must move at least (unique selected K/V once, statistics, scores,
    indices, partials)."""
    B, Hq, Hkv, D, P = wl.B, wl.H_q, wl.H_kv, wl.D, wl.P
    N = (seq_lens.astype(np.int64) + P - 1) // P
    H_sel = Hkv if (token_level or group_select) else Hq
    cnt = int(sel_cnt.sum())
    kv, upages = unique_kv_bytes(wl, sel_idx, sel_cnt, seq_lens, H_sel)
    out = {}
    if token_level:
        S = seq_lens.astype(np.int64)
        out["pagestats_update"] = B * Hkv * D * 2 * 2 * 2 + B * Hkv * 2 + B * 8
        # the logit scratch holds one row per kv head (group-mean query) or
        # per query head (per-head reading)
        rows = Hq if h2o_per_head else Hkv
        out["h2o_accumulate"] = int((S * Hkv * D * 2).sum() + (S * Hkv * 2 * 2).sum()
                                    + (S * rows * 4 * 2).sum() + (S * Hkv * 4).sum()
                                    + B * Hq * D * 4 + S.sum() * 4 * 2)
    else:
        if wl.steps > 1:   # append + tail refresh
            out["pagestats_update"] = int(B * Hkv * D * 2 * 2 * 2
                                          + B * Hkv * D * 2 * (P - 1)
                                          + B * Hkv * D * 8)
            if gauss:      # the tail page's rows again, its mean, its variance
                out["pagestats_update"] += int(B * Hkv * D * (2 * P + 8))
        if gauss:
            # mean + variance rows (fp32) once per page-head, q, mu + var out
            out["gauss_moments"] = int((N * (Hkv * 8 * D + Hq * 8)).sum() + B * Hq * D * 4)
        else:
            out["page_score"] = int((N * (Hkv * 8 * D + H_sel * 4 + 4)).sum()
                                    + B * Hq * D * 4)
    if gauss:
        # mu + var in, estimates out, tau-hat, selection (indices and blocks)
        out["gauss_select"] = int((N * Hq * 12).sum() + B * Hq * 4 + cnt * 8 + B * Hq * 4)
    else:
        out["page_topk"] = int((N * H_sel * 4).sum() + cnt * 4)
    if entmax and fused:
        # K of the selected pages once and the merged output; V is read only
        # for 16-row groups in the support, which depends on the data and is
        # left out (the GB/s is a lower bound)
        out["sparse_paged_decode"] = int(kv // 2 + B * Hq * D * 4 + cnt * 4
                                         + B * Hq * (D + 1) * 4)
    elif entmax:
        # as above, plus the logits of the selected rows written and read and
        # the partials
        out["sparse_paged_decode"] = int(kv // 2 + B * Hq * D * 4 + cnt * 4
                                         + 2 * cnt * P * 4
                                         + B * Hq * num_splits * (D + 1) * 4)
        out["lse_merge"] = int(B * Hq * num_splits * (D + 1) * 4 + B * Hq * (D + 1) * 4)
    elif fused:   # merged in-block: the merged output instead of the partials
        out["sparse_paged_decode"] = int(kv + B * Hq * D * 4 + cnt * 4 + B * Hq * (D + 1) * 4)
    else:
        out["sparse_paged_decode"] = int(kv + B * Hq * D * 4 + cnt * 4
                                         + B * Hq * num_splits * (D + 1) * 4)
        out["lse_merge"] = int(B * Hq * num_splits * (D + 1) * 4 + B * Hq * (D + 1) * 4)
    return out, upages


# ------------------------------------------------------ measured traffic

# The sources each decode kernel is built from: a counter record stays valid
# while they hash the same.
DECODE_SOURCES = {
    "softmax": ("sparse_kv_cache_amd/csrc/sparse_decode.hip",
                "sparse_kv_cache_amd/csrc/skv_device.h",
                "sparse_kv_cache_amd/csrc/skv_topk.h"),
    "entmax": ("sparse_kv_cache_amd/csrc/entmax_decode.hip",
               "sparse_kv_cache_amd/csrc/skv_device.h"),
    # h2o_select_decode: the logits pass and the group kernel
    "token": ("sparse_kv_cache_amd/csrc/sparse_decode.hip",
              "sparse_kv_cache_amd/csrc/skv_device.h",
              "sparse_kv_cache_amd/csrc/skv_topk.h",
              "sparse_kv_cache_amd/csrc/h2o.hip"),
}


def decode_source_hash(kind="softmax"):
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha1()
    for f in DECODE_SOURCES[kind]:
        with open(os.path.join(root, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profiled_traffic(tag, kind="softmax", kernel=None):
    """HBM bytes per decode launch from the committed counter summary of this
    workload and mode (FETCH_SIZE + WRITE_SIZE, each scaled by a plain copy's
    reading), or None when there is none, when it was taken for another kernel
    (e.g. the one-launch step's record for the separate decode), or when the
    decode kernel's sources have changed since the counters were taken."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        f"traffic_{tag}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    start = text.find("```json")
    if start < 0:
        return None
    body = text[start + 7:text.find("```", start + 7)].strip()
    recs = json.loads(body)
    if recs is None:
        return None
    # one record (the main launch), or a list: the main launch, then the
    # decode timed alone
    recs = recs if isinstance(recs, list) else [recs]
    if kernel is not None:
        recs = [r for r in recs if r.get("kernel") == kernel]
    if not recs or recs[0].get("source_sha1") != decode_source_hash(kind):
        return None
    return int(recs[0]["traffic"])


# ------------------------------------------------------------ cpu baseline

def compact_request(wl, cache_bits, seq_lens, bb):
    """Request bb's blocks copied out of the cache bits ([2, NB, P, H_kv, D])
    in page order, and its block-table row remapped to them: (cache, bt)."""
    N = min((int(seq_lens[bb]) + wl.P - 1) // wl.P, wl.bt_ld)
    blocks = wl.block_table[bb, :N]
    cache_c = np.ascontiguousarray(cache_bits[:, blocks])
    bt = np.zeros((1, wl.bt_ld), dtype=np.int32)
    bt[0, :N] = np.arange(N, dtype=np.int32)
    return cache_c, bt


def cpu_baseline(wl, cache_bits, q, seq_lens, seconds, token_level, hh_bits=None,
                 gauss=False, slopes=None, k_cap=0, h2o_per_head=False):
    """The float64 oracle on a bounded sample of requests (whole step for
    those requests), scaled to steps/s of the full batch: (i) one thread, then
    (ii) the same request-steps on a pool of threads (the oracle's C calls
    release the GIL), one request-step per thread at a time.  Returns both."""
    import oracle
    oracle.build() if not os.path.exists(os.path.join(
        os.path.dirname(os.path.abspath(oracle.__file__)), "liboracle.so")) else None
    qd = q.double().numpy()
    st_cache = {}
    sl64 = None if slopes is None else np.asarray(slopes, np.float32).astype(np.float64)

    def prepare(bb):
        """Per-request inputs built outside the timed region: the request's
        own blocks copied into a compact cache with its block table remapped
        (the oracle's statistics are sized by the cache it is given, so the
        whole pool would cost gigabytes per request), and its statistics."""
        if token_level or bb in st_cache:
            return
        sl = seq_lens[bb:bb + 1]
        cache_c, bt = compact_request(wl, cache_bits, seq_lens, bb)
        if gauss:
            st = (oracle.page_stats(cache_c, bt, sl, wl.P)[2],
                  oracle.page_var(cache_c, bt, sl, wl.P))
        else:
            st = oracle.page_stats(cache_c, bt, sl, wl.P)
        st_cache[bb] = (cache_c, bt, st)

    def request_step(bb):
        """One request's whole step through the oracle."""
        sl = seq_lens[bb:bb + 1]
        S = int(sl[0])
        if token_level:
            bt = wl.block_table[bb:bb + 1]
        else:
            cache_c, bt, st = st_cache[bb]
        if token_level:
            hh = hh_bits.copy()
            sc = oracle.h2o_step(qd[bb:bb + 1], cache_bits, bt, sl, hh, wl.bos,
                                 wl.eos, wl.softmax_scale, wl.decay,
                                 per_head=h2o_per_head)
            for h in range(wl.H_kv):
                sel = oracle.select(sc[0, h, :S], wl.topk_pages, 0.0, wl.bos, wl.eos)
                for g in range(wl.G):
                    oracle.attend(qd[bb, h * wl.G + g], cache_bits, h, bt[0], S, sel,
                                  wl.softmax_scale)
        elif gauss:
            N = (S + wl.P - 1) // wl.P
            n = np.array([min(wl.P, S - p * wl.P) for p in range(N)], dtype=np.int32)
            mu, var = oracle.gauss_moments(qd[bb:bb + 1], *st, bt, sl, wl.P,
                                           wl.softmax_scale, alibi=sl64)
            for i in range(wl.H_q):
                tau = oracle.gauss_tau(mu[0, i, :N], var[0, i, :N], n, sl64 is not None)
                sel = oracle.gauss_select(mu[0, i, :N], var[0, i, :N], n, tau, wl.bos,
                                          wl.eos, k_cap)
                oracle.attend_entmax15(qd[bb, i], cache_c, i // wl.G, bt[0], S, sel,
                                       wl.softmax_scale,
                                       slope=None if sl64 is None else sl64[i])
        else:
            kc = min(max(wl.topk_pages, int(math.floor(wl.topk_frac * wl.bt_ld)),
                         wl.bos + wl.eos), wl.bt_ld)
            oracle.decode_step(qd[bb:bb + 1], cache_c, bt, sl, st, wl.w_avg,
                               wl.w_peak, wl.topk_pages, wl.topk_frac, wl.bos, wl.eos,
                               wl.softmax_scale, kc)

    # (i) one thread
    rows_done, t_used, b = 0, 0.0, 0
    while t_used < seconds and rows_done < 10_000:
        bb = b % wl.B
        prepare(bb)
        t0 = time.perf_counter()
        request_step(bb)
        t_used += time.perf_counter() - t0
        rows_done += 1
        b += 1
    covered = min(rows_done, wl.B)
    what = ("the token-level step" if token_level else
            "moments+tau-hat+select+entmax attend (statistics prebuilt)" if gauss else
            "score+select+attend (statistics prebuilt)")
    single = {"value": 1.0 / (t_used / rows_done * wl.B), "unit": "steps/s", "cores": 1,
              "kind": "oracle", "host_cpu": host_cpu(),
              "sample": f"{rows_done} request-steps of {what}, {covered} of {wl.B} requests",
              "seconds": round(t_used, 2)}

    # (ii) a pool of threads over the same requests, for about as long
    import concurrent.futures as cf
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    threads = max(1, min(16, avail))
    deadline = time.perf_counter() + max(1.0, seconds / 2)

    def worker(w):
        done, k = 0, w
        while time.perf_counter() < deadline:
            request_step(k % covered)
            done += 1
            k += threads
        return done

    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        total = sum(ex.map(worker, range(threads)))
    wall = time.perf_counter() - t0
    parallel = {"value": total / wall / wl.B, "unit": "steps/s", "cores": threads,
                "kind": "oracle", "host_cpu": host_cpu(),
                "sample": (f"{total} request-steps of {what} on {threads} threads over the "
                           f"same {covered} requests"),
                "seconds": round(wall, 2)}
    return single, parallel


def host_cpu():
    """The host CPU's model name (Linux), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# -------------------------------------------------------------------- main

def unique_page_heads(wl, sel_idx, sel_cnt, seq_lens, H_sel):
    """int32 [n, 3] (block, kv head, valid rows) of every distinct (request,
    kv head, page) the selection reads, in (request, kv head, page) order."""
    out = []
    for b in range(wl.B):
        S = int(seq_lens[b])
        for h in range(wl.H_kv):
            rows = range(h * wl.G, (h + 1) * wl.G) if H_sel == wl.H_q else [h]
            u = set()
            for r in rows:
                u.update(sel_idx[b, r, :sel_cnt[b, r]].tolist())
            for p in sorted(u):
                out.append((int(wl.block_table[b, p]), h, min(wl.P, S - p * wl.P)))
    return np.asarray(out, dtype=np.int32).reshape(-1, 3)


def reference_rates(torch, dev, nbytes, caches=None, items=None, reps=16):
    """The library's bandwidth references, timed like the kernels (a graph of
    back-to-back launches, HIP events around one replay): a streaming read of
    nbytes at rotating offsets of a buffer 16x larger (so the memory-side cache
    cannot serve it), and, given the decode's page-heads, the gather-only read
    of exactly those rows rotating over the replica caches."""
    import sparse_kv_cache_amd as skv
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    out = {}
    n16 = max(16, int(nbytes) // 16 * 16)
    pool = torch.empty(n16 * 16 + (1 << 20), dtype=torch.uint8, device=dev)
    pool.fill_(3)
    views = [pool[(i * n16) % (pool.numel() - n16):][:n16] for i in range(reps)]

    def timed(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                fn(i)
        g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms = timed(lambda i: skv.skv_ref_stream_read(views[i], sink))
    out["stream"] = {"bytes": n16, "us": round(ms * 1000, 2),
                     "GBps": round(n16 / (ms * 1e-3) / 1e9, 1)}
    del pool, views
    if caches is not None and items is not None and len(items):
        it = torch.from_numpy(items).to(dev)
        rows = int(items[:, 2].sum())
        gbytes = rows * caches[0].shape[4] * 2 * 2
        ms = timed(lambda i: skv.skv_ref_gather_read(caches[i % len(caches)], it, sink))
        out["gather"] = {"bytes": gbytes, "page_heads": int(len(items)),
                         "us": round(ms * 1000, 2),
                         "GBps": round(gbytes / (ms * 1e-3) / 1e9, 1)}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by request and kv head with no exchange between GPUs)",
              file=sys.stderr)
        return 2
    import torch
    import sparse_kv_cache_amd  # noqa: F401  (loads lazily; fails loudly if unbuilt)

    sparse_kv_cache_amd.load_library()
    torch.cuda.init()
    result = measure(args, args.workload, cpu=not args.no_cpu_baseline)
    if args.workload != "long_context" and not args.no_long_context:
        import copy
        torch.cuda.empty_cache()
        a2 = copy.copy(args)
        a2.select, a2.alibi, a2.attention, a2.no_fuse, a2.splits = "head", False, "softmax", \
            False, 0
        a2.steps, a2.repeats = min(args.steps, 50), 0
        ns = measure(a2, "long_context", cpu=False)
        rf = ns["roofline"]
        # the decode kernel's own numbers (timed alone where the step fuses
        # it with the selection), then the step's main launch
        da = rf.get("decode_alone")
        if da is not None:
            dec = {"kernel": da["kernel"], "us_per_launch": da["us"],
                   "bytes_per_launch": da["bytes"], "achieved_GBps": da["achieved"],
                   "frac": da["frac"], "gather_frac": da["gather_frac"],
                   "stream_frac": round(da["achieved"] / rf["stream_ref"]["GBps"], 4),
                   "traffic": da.get("traffic")}
        else:
            dec = {"kernel": rf["kernel"], "us_per_launch": rf["us_per_launch"],
                   "bytes_per_launch": rf["bytes_per_launch"], "achieved_GBps": rf["achieved"],
                   "frac": rf["frac"], "gather_frac": rf.get("gather_frac"),
                   "stream_frac": rf.get("stream_frac"), "traffic": rf["traffic"]}
        dec["traffic_ratio"] = (None if dec["traffic"] is None else
                                round(dec["traffic"] / dec["bytes_per_launch"], 3))
        result["long_context"] = {
            "workload": "long_context", "steps_per_s": ns["value"],
            "gpu_ms_per_step": ns["gpu_ms_per_step"], "launches": len(ns["kernels"]),
            "sparse_paged_decode": dec,
            "main_launch": {
                "kernel": rf["kernel"], "us_per_launch": rf["us_per_launch"],
                "bytes_per_launch": rf["bytes_per_launch"], "achieved_GBps": rf["achieved"],
                "frac": rf["frac"], "traffic": rf["traffic"],
                "traffic_ratio": (None if rf["traffic"] is None else
                                  round(rf["traffic"] / rf["bytes_per_launch"], 3))},
            "stream_ref": rf.get("stream_ref"), "gather_ref": rf.get("gather_ref"),
            "kernels": ns["kernels"]}
    print(json.dumps(result), flush=True)
    return 0


def measure(args, workload, cpu=True):
    """One workload's bench record (the dict printed as the JSON line)."""
    import torch
    from sparse_kv_cache_amd import workloads as W
    from sparse_kv_cache_amd.decode import SparseDecoder, alibi_slopes

    dev = torch.device("cuda:0")
    wl = W.WORKLOADS[workload]()
    token_level = wl.name == "h2o_token"
    if args.splits:
        wl.num_splits = args.splits
    t_gen = time.perf_counter()
    cache0 = W.make_cache(wl, device=dev)
    q = W.make_queries(wl, 0, device=dev)
    bt = torch.from_numpy(wl.block_table).to(dev)
    seq_steps = [torch.from_numpy(wl.seq_lens_at(s)).to(dev) for s in range(wl.steps)]
    per_step_mb = {"mha_tiny": 0.3, "gqa_ragged": 120, "h2o_token": 46,
                   "long_context": 190, "high_batch": 4500}[wl.name]
    R = args.replicas or max(1, min(16, math.ceil(1024 / per_step_mb)))
    if wl.name == "high_batch":
        R = 1
    caches = [cache0] + [cache0.clone() for _ in range(R - 1)]
    group = args.select == "group" and not token_level
    gauss = args.select == "gauss" and not token_level
    slopes = alibi_slopes(wl.H_q, dev) if (args.alibi and not token_level) else None
    entmax = (args.attention == "entmax15" or gauss) and not token_level
    decs = [SparseDecoder.for_workload(wl, device=dev, group_select=group,
                                       alibi_slopes=slopes, fuse_merge=not args.no_fuse,
                                       attention="entmax15" if entmax else "softmax",
                                       selection="gauss" if gauss else "topk",
                                       h2o_softmax=args.h2o_softmax)
            for _ in range(R)]
    fused = decs[0].fused or decs[0].entmax_fused
    in_decode = decs[0].select_in_decode
    in_group_decode = decs[0].select_in_group_decode and not gauss and not token_level
    in_split_decode = decs[0].select_in_split_decode
    split_name = ("sparse_select_decode_split_blocks" if decs[0].split_blocks
                  else "sparse_select_decode_split")
    token_fused = decs[0].token_fused
    one_launch = decs[0].score_in_decode
    new_kv = [W.make_new_kv(wl, s, device=dev) for s in range(min(wl.steps, 64))] \
        if wl.steps > 1 else None
    if token_level:
        hh0 = W.make_hh(wl, device=dev)
        for d in decs:
            d.hh.copy_(hh0)
    stats_ms = None
    if not token_level:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for c, d in zip(caches, decs):
            d.rebuild_stats(c, bt, seq_steps[0])
        e1.record()
        torch.cuda.synchronize()
        stats_ms = e0.elapsed_time(e1) / R
    gen_s = time.perf_counter() - t_gen

    # A plain device copy of known size: its duration is the achievable HBM
    # rate on this machine, and under a counter profile its FETCH_SIZE /
    # WRITE_SIZE readings calibrate the counters (256 MiB read + 256 MiB
    # written per launch).
    copy_bytes = 256 << 20
    csrc = torch.empty(copy_bytes, dtype=torch.uint8, device=dev)
    cdst = torch.empty(copy_bytes, dtype=torch.uint8, device=dev)
    csrc.fill_(1)
    copy_ms = []
    for _ in range(3):
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        cdst.copy_(csrc)
        c1.record()
        torch.cuda.synchronize()
        copy_ms.append(c0.elapsed_time(c1))
    copy_gbps = 2 * copy_bytes / (min(copy_ms) * 1e-3) / 1e9
    del csrc, cdst

    if gauss:
        names = (["pagestats_update"] if wl.steps > 1 else []) + \
            ["gauss_moments", "gauss_select", "sparse_paged_decode"] + \
            ([] if fused else ["lse_merge"])
    else:
        # (token_fused: the append runs inside h2o_select_decode's first launch)
        names = (["pagestats_update"] if wl.steps > 1 and not token_fused else []) + \
            (["h2o_select_decode", "lse_merge"] if token_fused else
             (["h2o_accumulate"] if token_level else [] if one_launch else ["page_score"]) +
            (["sparse_page_decode"] if one_launch else ["sparse_select_decode"] if in_decode
             else ["sparse_select_decode_group", "lse_merge"] if in_group_decode
             else [split_name, "lse_merge"] if in_split_decode
             else ["page_topk", "sparse_paged_decode"] + ([] if fused else ["lse_merge"])))

    def enqueue(i, name):
        """Enqueue kernel `name` of step i (replica i % R, sequence step i % steps)."""
        r = i % R
        d, c = decs[r], caches[r]
        s = i % wl.steps
        sl = seq_steps[s]
        if name == "pagestats_update":
            kn, vn = new_kv[s % len(new_kv)]
            d.append(c, bt, sl, kn, vn)
        elif name == "h2o_accumulate":
            d.accumulate(q, c, bt, sl)
        elif name == "h2o_select_decode":
            kn, vn = new_kv[s % len(new_kv)] if new_kv is not None else (None, None)
            d.accumulate_select_attend(q, c, bt, sl, kn, vn)
        elif name == "page_score":
            d.score(q, bt, sl)
        elif name == "page_topk":
            d.select(sl, bt)
        elif name == "gauss_moments":
            d.moments(q, bt, sl)
        elif name == "gauss_select":
            d.select_gauss(sl, bt)
        elif name == "sparse_paged_decode":
            d.attend(q, c, bt, sl)
        elif name == "sparse_select_decode":
            d.select_attend(q, c, bt, sl)
        elif name == "sparse_select_decode_group":
            d.select_attend_group(q, c, bt, sl)
        elif name in ("sparse_select_decode_split", "sparse_select_decode_split_blocks"):
            d.select_attend_split(q, c, bt, sl)
        elif name == "sparse_page_decode":
            d.score_select_attend(q, c, bt, sl)
        else:
            d.merge()

    def run_steps(first, count):
        for i in range(first, first + count):
            for n in names:
                enqueue(i, n)

    def captured(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    # The step sequence is captured into HIP graphs (one launch for the whole
    # warm-up, one for the whole timed region): Python's per-call submission
    # cost would otherwise leave the GPU idle between the short kernels.
    if args.no_graph:
        run_steps(0, args.warmup)
    else:
        g_warm = captured(lambda: run_steps(0, args.warmup)) if args.warmup else None
        g_timed = captured(lambda: run_steps(args.warmup, args.steps))
        if g_warm is not None:
            g_warm.replay()
    torch.cuda.synchronize()

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    if args.no_graph:
        run_steps(args.warmup, args.steps)
    else:
        g_timed.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1) / args.steps
    ms_per_step = wall * 1000.0 / args.steps

    # spread: the timed sequence replayed a few more times (HIP events), for
    # the median and p10 / p90 of the per-step time; value stays the first,
    # barrier-bracketed run above
    spread = []
    if not args.no_graph:
        for _ in range(args.repeats):
            r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            r0.record()
            g_timed.replay()
            r1.record()
            torch.cuda.synchronize()
            spread.append(r0.elapsed_time(r1) / args.steps)

    # algorithmic bytes from the selections of the last timed step's replica
    # (read before the per-kernel graphs below overwrite the buffers)
    last = (args.warmup + args.steps - 1)
    d = decs[last % R]
    sl_last = wl.seq_lens_at(last % wl.steps)
    if token_fused:   # the selection stays on chip: one more step that writes it out
        d.keep_selection = True
        d.accumulate_select_attend(q, caches[last % R], bt, seq_steps[last % wl.steps])
        d.keep_selection = False
        torch.cuda.synchronize()
    elif in_decode or in_group_decode or in_split_decode:   # selection in LDS: recompute it
        if one_launch:
            d.score(q, bt, seq_steps[last % wl.steps])
        d.select(seq_steps[last % wl.steps], bt)
        torch.cuda.synchronize()
    sel_idx = d.sel_idx.cpu().numpy()
    sel_cnt = d.sel_cnt.cpu().numpy()

    # Per-kernel durations: each kernel alone, launched back to back over the
    # replicas inside one graph, timed with HIP events around the replay.
    per_kernel_ms = {}
    base = args.warmup + args.steps
    reps = max(2 * R, 16)
    for n in names:
        g = captured(lambda: [enqueue(base + j, n) for j in range(reps)])
        g.replay()
        k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        k0.record()
        g.replay()
        k1.record()
        torch.cuda.synchronize()
        per_kernel_ms[n] = k0.elapsed_time(k1) / reps
        del g

    # partials per head the step's decode wrote (one per block of splits in
    # the block-merged split decode)
    n_part = decs[0].partials[0].shape[2]
    kb, upages = kernel_bytes(wl, sel_idx, sel_cnt, sl_last, n_part,
                              token_level, group, fused, entmax, gauss,
                              h2o_per_head=decs[0].h2o_per_head)
    if one_launch:
        # the statistics read for scoring (scores and selection stay in LDS)
        # plus the merged decode; q counted once
        n_pages = (sl_last.astype(np.int64) + wl.P - 1) // wl.P
        kb.pop("page_topk")
        kb["sparse_page_decode"] = (kb.pop("page_score") - int((n_pages * wl.H_q * 4).sum())
                                    - wl.B * wl.H_q * wl.D * 4 + kb.pop("sparse_paged_decode"))
    elif in_decode:   # one launch: the top-k's score read plus the merged decode
        kb["sparse_select_decode"] = kb.pop("page_topk") - int(sel_cnt.sum()) * 4 \
            + kb.pop("sparse_paged_decode")
    elif token_fused:   # the accumulator step without its score rows, plus the decode
        S_sum = int(sl_last.astype(np.int64).sum())
        kb["h2o_select_decode"] = (kb.pop("h2o_accumulate") - S_sum * wl.H_kv * 4
                                   + kb.pop("sparse_paged_decode") - int(sel_cnt.sum()) * 4)
        kb.pop("page_topk")
        if "pagestats_update" in kb:   # the append, less its table reads (counted once)
            kb["h2o_select_decode"] += kb.pop("pagestats_update") - wl.B * 8
    elif in_group_decode or in_split_decode:   # the top-k's score read plus the decode
        name = "sparse_select_decode_group" if in_group_decode else split_name
        kb[name] = kb.pop("page_topk") - int(sel_cnt.sum()) * 4 + kb.pop("sparse_paged_decode")
    step_bytes = sum(kb.values())
    kern = {}
    for n in names:
        t = per_kernel_ms[n]
        kern[n] = {"us": round(t * 1000, 2), "bytes": kb[n],
                   "GBps": round(kb[n] / (t * 1e-3) / 1e9, 1) if t > 0 else None}
    dominant = max(names, key=lambda n: per_kernel_ms[n])
    focus = ("sparse_page_decode" if one_launch else
             "sparse_select_decode" if in_decode else
             "sparse_select_decode_group" if in_group_decode else
             split_name if in_split_decode else
             "h2o_select_decode" if token_fused else "sparse_paged_decode")
    a = kb[focus] / (per_kernel_ms[focus] * 1e-3) / 1e9
    # the committed counter summary of this workload and mode
    traffic_tag = (wl.name + ("_group" if group else "")
                   + ("_gauss" if gauss else "_entmax" if entmax else "")
                   + ("_alibi" if slopes is not None else "")
                   + ("_heads" if decs[0].h2o_per_head else ""))
    traffic_kind = "entmax" if entmax else "token" if token_fused else "softmax"
    roofline = {"kernel": focus, "bound": "hbm", "achieved": round(a, 1),
                "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(a / PEAK_HBM_GBPS, 4),
                "traffic": (None if (entmax and not fused) else
                            profiled_traffic(traffic_tag, traffic_kind, focus)),
                # the same rate against a plain device copy measured in this run
                "copy_frac": round(a / copy_gbps, 4) if copy_gbps > 0 else None,
                "bytes_per_launch": kb[focus],
                "us_per_launch": round(per_kernel_ms[focus] * 1000, 2)}
    # against the library's streaming read of the same byte count, and (page
    # size 16) the gather-only read of the decode's own page-heads
    items = None
    if wl.P == 16 and not (entmax and not fused):
        H_sel = wl.H_kv if (group or token_level) else wl.H_q
        items = unique_page_heads(wl, sel_idx, sel_cnt, sl_last, H_sel)
    refs = reference_rates(torch, dev, kb[focus], caches, items)
    roofline["stream_ref"] = refs["stream"]
    roofline["stream_frac"] = round(a / refs["stream"]["GBps"], 4)
    if "gather" in refs:
        roofline["gather_ref"] = refs["gather"]
        roofline["gather_frac"] = round(a / refs["gather"]["GBps"], 4)
    # Where the step's decode runs inside a fused launch (selection, scoring
    # or both in the same kernel), the decode kernel is also timed on its own
    # over the same selection, the same way: its rate is the decode's, not
    # the fused launch's.
    if (focus != "sparse_paged_decode" and wl.steps == 1 and not token_level
            and not gauss and not entmax):
        for r in range(R):
            decs[r].score(q, bt, seq_steps[0])
            decs[r].select(seq_steps[0], bt)
        torch.cuda.synchronize()
        g = captured(lambda: [decs[(base + j) % R].attend(q, caches[(base + j) % R], bt,
                                                          seq_steps[0])
                              for j in range(reps)])
        g.replay()
        k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        k0.record()
        g.replay()
        k1.record()
        torch.cuda.synchronize()
        dms = k0.elapsed_time(k1) / reps
        del g
        kb0, _ = kernel_bytes(wl, sel_idx, sel_cnt, sl_last, decs[0].decode_splits,
                              token_level, group, fused, entmax, gauss)
        da = kb0["sparse_paged_decode"] / (dms * 1e-3) / 1e9
        alone = "sparse_paged_decode_merged" if fused else "sparse_paged_decode"
        roofline["decode_alone"] = {
            "kernel": alone,
            "us": round(dms * 1000, 2), "bytes": kb0["sparse_paged_decode"],
            "achieved": round(da, 1), "frac": round(da / PEAK_HBM_GBPS, 4),
            "gather_frac": (round(da / refs["gather"]["GBps"], 4) if "gather" in refs
                            else None),
            "traffic": profiled_traffic(traffic_tag, traffic_kind, alone)}

    result = {
        "metric": "sparse decode steps/s + effective HBM GB/s (% of peak), GQA 32/8 D=128",
        "value": round(args.steps / (wall), 3),
        "unit": "steps/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "gpu_ms_per_step": round(gpu_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "kv_dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H_q": wl.H_q, "H_kv": wl.H_kv,
                   "D": wl.D, "page_size": wl.P, "topk_pages": wl.topk_pages,
                   "topk_frac": wl.topk_frac, "num_splits": decs[0].decode_splits,
                   "mean_seq_len": float(np.mean(sl_last)), "replicas": R,
                   "selection": ("kv_head" if (group or token_level) else
                                 "gauss_query_head" if gauss else "query_head"),
                   "gauss_tau": (None if not gauss else
                                 "page_mixture" if decs[0].mixture else "single"),
                   "alibi": slopes is not None, "merge_in_decode": fused,
                   "select_in_decode": (in_decode or in_group_decode or in_split_decode
                                        or token_fused),
                   "one_launch_step": one_launch,
                   "attention": "entmax15" if entmax else "softmax",
                   "h2o_softmax": args.h2o_softmax if token_level else None,
                   "parallelism": "single-gpu"},
        "selected_pages_per_head": round(float(sel_cnt.mean()), 2),
        "effective_GBps": round(step_bytes / (gpu_ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(step_bytes / (gpu_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "step_bytes": int(step_bytes), "unique_page_heads": int(upages),
        "kernels": kern, "dominant_kernel": dominant,
        "stats_rebuild_ms": None if stats_ms is None else round(stats_ms, 4),
        "roofline": roofline,
        "copy_GBps": round(copy_gbps, 1),
        "setup_s": round(gen_s, 1),
        "gpu_ms_per_step_spread": (None if not spread else {
            "runs": len(spread),
            "p10": round(float(np.percentile(spread, 10)), 4),
            "p50": round(float(np.percentile(spread, 50)), 4),
            "p90": round(float(np.percentile(spread, 90)), 4)}),
        "env": {"torch": torch.__version__, "hip": torch.version.hip,
                "gpu": torch.cuda.get_device_name(0),
                "host_cpu": host_cpu(), "host_threads": os.cpu_count()},
    }
    if cpu:
        from sparse_kv_cache_amd.workloads import bf16_bits
        cb = bf16_bits(caches[last % R])
        hb = bf16_bits(hh0) if token_level else None
        result["cpu_baseline"], result["cpu_baseline_parallel"] = cpu_baseline(
            wl, cb, q.cpu(), sl_last, args.cpu_seconds, token_level, hb,
            gauss=gauss, slopes=None if slopes is None else slopes.cpu().numpy(),
            k_cap=decs[0].k_cap, h2o_per_head=decs[0].h2o_per_head)
    return result


if __name__ == "__main__":
    sys.exit(main())
