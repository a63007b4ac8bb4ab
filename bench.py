"""Benchmark of top-k sparse attention over a paged KV cache on one MI355X.

One step is one pass of the whole path over one decode batch: indexer logits
over the fp4 index keys of the compressed pool -> exact top-512 -> index build
(window + selected compressed entries through the page tables) -> split-K
sparse attention with its merge.  The default workload is decode at position
32767 with B = 1, r = 4 (64 query heads sharing one KV head, head_dim 512,
128-token window, top-k 512 of 8192 compressed entries), bf16 rows.  All
inputs are resident in HBM before timing; outputs and workspaces are
preallocated, so the timed region only launches kernels.

Prints one JSON line.  `value` is gathered KV bytes per second of whole steps
(640 rows x 1 KiB per sequence per step); the `roofline` object is for the
dominant kernel, timed live with HIP events on the stream it runs on;
`cpu_baseline` is the CPU oracle timed on the host on the same step;
`secondary` holds the other page shapes (prefill S8192, decode B8, e4m3,
indexer at context 131072), each with its own roofline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import sparse_attention_paged_amd as sap  # noqa: E402
import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
METRIC = "sparse attn µs + TFLOP/s (prefill S8192) and gathered GB/s (decode B1/B8), vs roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class DecodeStep:
    """Device-resident inputs, outputs and workspaces of one decode step."""

    def __init__(self, B=1, pos=32767, ratio=4, kv_dtype="bf16", seed=W.SEED_BASE + 2):
        self.case = c = W.decode_case(B=B, pos=pos, ratio=ratio, kv_dtype=kv_dtype, seed=seed)
        d = torch.device("cuda")
        self.B, self.ratio = B, ratio
        self.n_c = math.ceil((pos + 1) / ratio) if ratio > 0 else 0
        g = W.make_generator(seed + 1000)
        self.q = c.q.to(d)
        self.win = c.win_pool.to(d)
        self.cmp = c.cmp_pool.to(d) if c.cmp_pool is not None else None
        self.wsc = c.win_scale.to(d) if c.win_scale is not None else None
        self.csc = c.cmp_scale.to(d) if c.cmp_scale is not None else None
        self.pos, self.seq, self.win_pt = c.pos.to(d), c.seq.to(d), c.win_pt.to(d)
        self.C = c.n_win + c.n_cmp
        if ratio > 0:
            self.cmp_pt = c.cmp_pt.to(d)
            self.keys = W.fp4_key_rows(c.cmp_pool.shape[0], g).to(d)     # index key per compressed row
            self.qi = torch.randn((B, 32, 128), generator=g).to(torch.bfloat16).to(d)
            self.wi = torch.rand((B, 32), generator=g).to(d)
            self.n_vis = torch.full((B,), self.n_c, dtype=torch.int32, device=d)
            self.logits = torch.empty((B, self.n_c), dtype=torch.float32, device=d)
            self.sel = torch.empty((B, c.n_cmp), dtype=torch.int32, device=d)
            nb = sap.topk_workspace_bytes(B, self.n_c, c.n_cmp)
            self.tk_ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=d)
        self.idx = torch.empty((B, self.C), dtype=torch.int32, device=d)
        self.out = torch.empty((B, 64, 512), dtype=torch.float32, device=d)
        nb = sap.sparse_attn_workspace_bytes(B, 64, 512, self.C, 0)
        self.ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=d)
        self.splits = sap.sparse_attn_num_splits(B, 64, 512, self.C, 0)

    def select(self):
        if self.ratio > 0:
            sap.indexer_logits_packed(self.qi, self.wi, self.keys, self.cmp_pt, self.case.page, self.n_c,
                                      n_keys=self.n_vis, out=self.logits)
            sap.topk_sparse_idx(self.logits, self.case.n_cmp, self.pos, self.seq, self.case.n_win, self.win_pt,
                                self.cmp_pt, self.case.page, out=self.idx, workspace=self.tk_ws)
        else:
            sap.build_sparse_idx(self.pos, self.seq, self.case.n_win, self.win_pt, self.case.page, out=self.idx)

    def attend(self):
        sap.sparse_attn_paged(self.q, self.win, self.cmp, self.idx, self.case.n_win, self.case.sm_scale,
                              out=self.out, win_scale=self.wsc, cmp_scale=self.csc, workspace=self.ws)

    def step(self):
        self.select()
        self.attend()

    def row_bytes(self):
        return self.win.shape[1] * self.win.element_size() + (4 if self.wsc is not None else 0)

    def gathered_bytes(self):
        return self.B * self.C * self.row_bytes()

    def attn_alg_bytes(self):
        # q + gathered rows + index list + fp32 output, per launch
        return self.B * (64 * 512 * 2 + self.C * (self.row_bytes() + 4) + 64 * 512 * 4)


# untimed launches before a timed loop of long kernels: the GPU clock ramps
# up over the first tens of milliseconds of sustained load
LONG_WARMUP = 20


def time_loop(fn, iters, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(iters):
        fn()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / iters        # ms


GRAPH_CALLS = 10   # calls captured per graph: spreads the graph launch over several calls


def capture(fn, per=1):
    """A HIP graph of `per` back-to-back calls of fn (the calls enqueue on the
    current stream, which is the capture stream inside the graph context)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per):
            fn()
    torch.cuda.synchronize()
    return g


def time_graph(fn, iters, warmup, per=1):
    """ms per fn call, from HIP events around `iters` replays of a graph of
    `per` calls (no host launch cost inside the timed region)."""
    g = capture(fn, per)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(iters):
        g.replay()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / (iters * per)


def code_sha256(src: str) -> str:
    """sha256 of a C++ source with its // comments and blank lines removed
    (a comment edit does not make the counters stale; a code edit does)."""
    lines = []
    for ln in src.splitlines():
        ln = re.sub(r"//.*$", "", ln).rstrip()
        if ln.strip():
            lines.append(ln)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


ATTN_SOURCES = ("attn.hip", "attn_d512.hip", "attn_common.hpp")


def attn_sources_sha256() -> str:
    """code_sha256 over the attention kernel sources, in a fixed order."""
    here = os.path.dirname(os.path.abspath(__file__))
    parts = []
    for name in ATTN_SOURCES:
        with open(os.path.join(here, "sparse_attention_paged_amd", "csrc", name)) as f:
            parts.append(f.read())
    return code_sha256("\n".join(parts))


def counted_traffic(key):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
    (profiles/attn_traffic_counters.json), or None when the attention sources
    changed since the counters were taken."""
    here = os.path.dirname(os.path.abspath(__file__))
    try:
        with open(os.path.join(here, "profiles", "attn_traffic_counters.json")) as f:
            doc = json.load(f)
        sha = attn_sources_sha256()
    except (OSError, ValueError):
        return None
    if doc.get("attn_code_sha256") != sha or key not in doc:
        return None
    return doc[key]["traffic_bytes"]


def roofline(bound, achieved, peak, unit, traffic=None):
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 5), "traffic": traffic}


# the pages' attention shapes ("perf(kernel): keep 16-byte kv loads ...", All
# shapes): H100 80GB time of the final Triton kernel, as context only
PAGES_H100_US = {
    "prefill_s2048_r4": 2887.86, "prefill_s8192_r4": 11399.31, "prefill_s4096_at28672_r4": 5762.74,
    "prefill_s8192_r128": 3672.89, "prefill_s8192_r0": 2561.59,
    "decode_b1_r4": 16.83, "decode_b1_r128": 15.98, "decode_b1_r0": 13.37,
    "decode_b8_r4": 20.81, "decode_b8_r128": 17.73, "decode_b8_r0": 13.89,
}


def prefill_secondary(iters, kv="bf16"):
    if kv == "e4m3":
        case = W.prefill_case(T=8192, ratio=4, kv_dtype="e4m3", q_scale=2.0 ** -7, seed=W.SEED_BASE + 35)
    else:
        case = W.prefill_case(T=8192, ratio=4)
    d = torch.device("cuda")
    q, win, cmp = case.q.to(d), case.win_pool.to(d), case.cmp_pool.to(d)
    wsc = case.win_scale.to(d) if case.win_scale is not None else None
    csc = case.cmp_scale.to(d) if case.cmp_scale is not None else None
    idx = sap.build_sparse_idx(case.pos.to(d), case.seq.to(d), case.n_win, case.win_pt.to(d), case.page,
                               case.cmp_logical.to(d), case.cmp_pt.to(d))
    out = torch.empty((case.T, 64, 512), dtype=torch.float32, device=d)
    valid = (idx >= 0).sum().item()
    flops = valid * 64 * 512 * 4.0
    ms = time_loop(lambda: sap.sparse_attn_paged(q, win, cmp, idx, case.n_win, case.sm_scale, out=out,
                                                 win_scale=wsc, cmp_scale=csc, num_splits=1), iters, LONG_WARMUP)
    tf = flops / (ms * 1e-3) / 1e12
    key = f"prefill_s8192_r4_{kv}"
    # e4m3 rows are widened to bf16 tiles: the MFMAs are bf16 (P as three bf16 terms triples PV)
    ctx = {"pages_h100_us": PAGES_H100_US["prefill_s8192_r4"]} if kv == "bf16" else {}
    return {"workload": key, "us": round(ms * 1e3, 2), "tflops": round(tf, 2), **ctx,
            "gflop": round(flops / 1e9, 2),
            "roofline": roofline("mfma", tf, BF16_PEAK_TFLOPS, "TFLOP/s", traffic=counted_traffic(key))}


def decode_secondary(B, kv, iters):
    st = DecodeStep(B=B, kv_dtype=kv, seed=W.SEED_BASE + (4 if kv == "e4m3" else 2))
    st.select()
    ms_attn = time_graph(st.attend, iters // GRAPH_CALLS, 1, GRAPH_CALLS)
    ms_step = time_graph(st.step, iters // GRAPH_CALLS, 1, GRAPH_CALLS)
    gb = st.attn_alg_bytes() / (ms_attn * 1e-3) / 1e9
    ctx = {"pages_h100_us": PAGES_H100_US[f"decode_b{B}_r4"]} if kv == "bf16" else {}
    return {"workload": f"decode_b{B}_pos32767_r4_{kv}", "attn_us": round(ms_attn * 1e3, 2), **ctx,
            "step_us": round(ms_step * 1e3, 2),
            "gathered_GBs_attn": round(st.gathered_bytes() / (ms_attn * 1e-3) / 1e9, 1),
            "splits": st.splits, "roofline": roofline("hbm", gb, HBM_PEAK_GBS, "GB/s")}


def pages_shapes_secondary(iters):
    """Attention alone (split-K + merge for decode) at every shape of the
    pages' table, bf16 pools, fp32 output."""
    d = torch.device("cuda")
    res = []
    for name, (T, start, ratio) in (("prefill_s2048_r4", (2048, 0, 4)), ("prefill_s4096_at28672_r4", (4096, 28672, 4)),
                                    ("prefill_s8192_r128", (8192, 0, 128)), ("prefill_s8192_r0", (8192, 0, 0))):
        case = W.prefill_case(T=T, start=start, ratio=ratio)
        q, win = case.q.to(d), case.win_pool.to(d)
        cmp = case.cmp_pool.to(d) if case.n_cmp > 0 else None
        idx = sap.build_sparse_idx(case.pos.to(d), case.seq.to(d), case.n_win, case.win_pt.to(d), case.page,
                                   case.cmp_logical.to(d) if case.n_cmp > 0 else None,
                                   case.cmp_pt.to(d) if case.n_cmp > 0 else None)
        out = torch.empty((case.T, 64, 512), dtype=torch.float32, device=d)
        valid = (idx >= 0).sum().item()
        ms = time_loop(lambda: sap.sparse_attn_paged(q, win, cmp, idx, case.n_win, case.sm_scale, out=out,
                                                     num_splits=1), iters, LONG_WARMUP)
        tf = valid * 64 * 512 * 4.0 / (ms * 1e-3) / 1e12
        res.append({"workload": name, "us": round(ms * 1e3, 2), "tflops": round(tf, 2),
                    "pages_h100_us": PAGES_H100_US[name],
                    "roofline": roofline("mfma", tf, BF16_PEAK_TFLOPS, "TFLOP/s")})
    for B in (1, 8):
        for ratio in (128, 0):
            st = DecodeStep(B=B, ratio=ratio)
            st.select()
            ms = time_graph(st.attend, 100 // GRAPH_CALLS, 1, GRAPH_CALLS)
            name = f"decode_b{B}_r{ratio}"
            res.append({"workload": name + "_pos32767_bf16", "attn_us": round(ms * 1e3, 2),
                        "pages_h100_us": PAGES_H100_US[name], "splits": st.splits,
                        "roofline": roofline("hbm", st.attn_alg_bytes() / (ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s")})
    return res


def indexer_secondary(B, iters):
    case = W.indexer_case(B=B, N=131072)
    d = torch.device("cuda")
    q, w, pool, pt = case.q.to(d), case.w.to(d), case.key_pool.to(d), case.page_table.to(d)
    out = torch.empty((B, case.N), dtype=torch.float32, device=d)
    sel = torch.empty((B, 512), dtype=torch.int32, device=d)
    ws = torch.empty(max(sap.topk_workspace_bytes(B, case.N, 512), 1), dtype=torch.uint8, device=d)
    ms_idx = time_graph(lambda: sap.indexer_logits_packed(q, w, pool, pt, case.page, case.N, out=out),
                        iters // GRAPH_CALLS, 1, GRAPH_CALLS)
    ms_topk = time_graph(lambda: sap.topk_select(out, 512, out=sel, workspace=ws), iters // GRAPH_CALLS, 1,
                         GRAPH_CALLS)
    alg = B * (case.N * 68 + case.N * 4 + 32 * 128 * 2 + 32 * 4)
    gb = alg / (ms_idx * 1e-3) / 1e9
    return {"workload": f"indexer_b{B}_ctx131072", "indexer_us": round(ms_idx * 1e3, 2),
            "topk512_us": round(ms_topk * 1e3, 2), "roofline": roofline("hbm", gb, HBM_PEAK_GBS, "GB/s")}


def indexer_prefill_secondary(length, start, ratio, iters):
    case = W.indexer_prefill_case(lengths=(length,), starts=(start,), ratio=ratio,
                                  seed=W.SEED_BASE + 650 + length + ratio)
    d = torch.device("cuda")
    q, w, pool, pt, ts, nk = (x.to(d) for x in (case.q, case.w, case.key_pool, case.page_table, case.tok_start,
                                                  case.n_keys))
    out = torch.empty((case.T, case.N), dtype=torch.float32, device=d)
    ms = time_graph(lambda: sap.indexer_logits_prefill(q, w, pool, pt, case.page, ts, case.max_tokens, case.N,
                                                       n_keys=nk, out=out), iters, LONG_WARMUP // 2, 2)
    # useful flops: each visible (token, key) pair costs 32 heads x 128 x 2
    tf = float(case.n_keys.to(torch.float64).sum()) * 32 * 128 * 2 / (ms * 1e-3) / 1e12
    return {"workload": f"indexer_prefill_n{length}_start{start}_r{ratio}", "us": round(ms * 1e3, 2),
            "tflops": round(tf, 2), "roofline": roofline("mfma", tf, BF16_PEAK_TFLOPS, "TFLOP/s")}


def indexer_cand_secondary(T, shared, iters):
    case = W.indexer_cand_case(T=T, n_ctx=131072, NC=16384, shared_seq=shared, seed=W.SEED_BASE + 620 + T)
    d = torch.device("cuda")
    q, w, pool, pt, cand, nk = (x.to(d) for x in (case.q, case.w, case.key_pool, case.page_table, case.cand,
                                                    case.n_keys))
    out = torch.empty((case.T, case.NC), dtype=torch.float32, device=d)
    ms = time_graph(lambda: sap.indexer_logits_candidates(q, w, pool, pt, case.page, cand, n_keys=nk, out=out),
                    iters // GRAPH_CALLS, 1, GRAPH_CALLS)
    # per candidate: the 68-byte key row, its index and its logit
    gb = T * case.NC * (68 + 4 + 4) / (ms * 1e-3) / 1e9
    kind = "prefill_n128" if shared else f"decode_b{T}"
    return {"workload": f"indexer_cand_{kind}_ctx131072_nc16384", "us": round(ms * 1e3, 2),
            "roofline": roofline("hbm", gb, HBM_PEAK_GBS, "GB/s")}


def gated_pool_secondary(B, R, D, iters):
    case = W.gated_pool_case(B=B, R=R, D=D, seed=W.SEED_BASE + 700 + B + R + D)
    x, g = case.x.cuda(), case.gate.cuda()
    out = torch.empty((B, D), dtype=torch.float32, device="cuda")
    ms = time_graph(lambda: sap.gated_pool(x, g, out=out), iters // GRAPH_CALLS, 1, GRAPH_CALLS)
    # bf16 rows, fp32 gates in; fp32 pooled rows out
    alg = B * R * D * (2 + 4) + B * D * 4
    return {"workload": f"gated_pool_b{B}_r{R}_d{D}", "us": round(ms * 1e3, 2),
            "roofline": roofline("hbm", alg / (ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s")}


def cpu_baseline(st: DecodeStep, budget_s: float):
    """The oracle on the same decode step, on the host cores."""
    import oracle

    c = st.case
    keys = st.keys.cpu()
    qi, wi = st.qi.cpu(), st.wi.cpu()
    pt = c.cmp_pt
    reps, t0 = 0, time.perf_counter()
    while True:
        logits = oracle.indexer_logits(qi, wi, keys, pt, c.page, None, st.n_c)
        sel = oracle.topk(logits.to(torch.float32), c.n_cmp)
        idx = oracle.build_idx(c.pos, c.seq, c.n_win, c.win_pt, c.page, sel, c.n_cmp, c.cmp_pt)
        oracle.sparse_attn(c.q, c.win_pool, c.cmp_pool, idx, c.n_win, c.sm_scale)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per = el / reps
    return {"value": round(st.gathered_bytes() / per / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": f"{reps} full decode steps (B{st.B}, indexer over {st.n_c} keys, "
                                        f"top-{c.n_cmp}, attention over {st.C} rows), {per * 1e3:.1f} ms each"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(each GPU would run its own sequences with no exchange)", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    log("building decode step inputs (B1, position 32767, r4)")
    st = DecodeStep(B=1, pos=32767, ratio=4)

    log("timing whole steps (graph replays; eager launches for reference)")
    # a graph holds GRAPH_CALLS steps back to back; K = steps (a multiple of it)
    reps = max(1, args.steps // GRAPH_CALLS)
    args.steps = reps * GRAPH_CALLS
    ms_step = time_graph(st.step, reps, max(1, args.warmup // GRAPH_CALLS), GRAPH_CALLS)
    ms_step_eager = time_loop(st.step, args.steps, args.warmup)
    log("timing the attention launches alone")
    ms_attn = time_graph(st.attend, reps, 1, GRAPH_CALLS)
    ms_sel = time_graph(st.select, reps, 1, GRAPH_CALLS)
    value = st.gathered_bytes() / (ms_step * 1e-3) / 1e9
    attn_gbs = st.attn_alg_bytes() / (ms_attn * 1e-3) / 1e9

    res = {
        "metric": METRIC, "value": round(value, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode_b1_pos32767_r4_bf16", "global_batch": 1, "seq_len": 32768, "heads": 64,
                   "head_dim": 512, "window": 128, "topk": 512, "ratio": 4, "parallelism": "single-gpu",
                   "step": "indexer(8192 fp4 keys) + top-512 fused with the index build + split-K attention + merge"},
        "timing": f"HIP-graph replays ({GRAPH_CALLS} steps per graph), HIP events around the timed replays",
        "eager_ms_per_step": round(ms_step_eager, 5),
        "attn_us": round(ms_attn * 1e3, 3), "select_us": round(ms_sel * 1e3, 3), "splits": st.splits,
        "context": {"pages_h100_attn_us": PAGES_H100_US["decode_b1_r4"],
                    "note": "the pages' H100 Triton time for this attention call alone; another machine"},
        "roofline": roofline("hbm", attn_gbs, HBM_PEAK_GBS, "GB/s",
                             traffic=counted_traffic("decode_b1_r4_bf16_attention_pair")),
    }
    res["roofline"]["kernel"] = "sparse attention split-K + merge (per launch pair)"
    res["roofline"]["bytes_per_launch"] = st.attn_alg_bytes()
    if not args.no_secondary:
        sec = []
        log("secondary: prefill S8192 r4")
        sec.append(prefill_secondary(10))
        log("secondary: prefill S8192 r4 e4m3")
        sec.append(prefill_secondary(5, "e4m3"))
        for B, kv in ((8, "bf16"), (8, "e4m3")):
            log(f"secondary: decode B{B} {kv}")
            sec.append(decode_secondary(B, kv, 100))
        for B in (1, 4):
            log(f"secondary: indexer B{B}")
            sec.append(indexer_secondary(B, 100))
        for length, start, ratio in ((2048, 129024, 2), (8192, 0, 2)):
            log(f"secondary: indexer prefill n{length} start{start} r{ratio}")
            sec.append(indexer_prefill_secondary(length, start, ratio, 5))
        for T, shared in ((1, False), (128, True)):
            log(f"secondary: indexer candidates T{T}")
            sec.append(indexer_cand_secondary(T, shared, 100))
        for B, R in ((1, 128), (8, 128), (8, 8)):
            log(f"secondary: gated pool B{B} R{R} D512")
            sec.append(gated_pool_secondary(B, R, 512, 100))
        log("secondary: the pages' other attention shapes")
        sec.extend(pages_shapes_secondary(5))
        res["secondary"] = sec
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on the same decode step")
        res["cpu_baseline"] = cpu_baseline(st, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
