"""Benchmark of top-k sparse attention over a paged KV cache on one MI355X.

One step is one pass of the whole path over one decode batch: indexer logits
over the fp4 index keys of the compressed pool -> exact top-512 fused with the
index build (window + selected compressed entries through the page tables) ->
split-K sparse attention with its merge.  The default workload is decode at
position 32767 with B = 1, r = 4 (64 query heads sharing one KV head,
head_dim 512, 128-token window, top-k 512 of 8192 compressed entries), bf16
rows.  All inputs are resident in HBM before timing; outputs and workspaces
are preallocated, so the timed region only launches kernels.

Prints one JSON line.  `value` is gathered KV bytes per second of whole steps
(640 rows x 1 KiB per sequence per step); the `roofline` object is for the
dominant kernel, timed live with HIP events on the stream it runs on;
`cpu_baseline` is the CPU oracle timed on the host on the same step;
`secondary` holds the pages' other shapes (prefill, decode B8, e4m3, indexer,
top-k, candidates, gated pool), a decode batch sweep, and cold-cache timings.

Two timing regimes:
  warm  HIP-graph replays of several calls back to back (inputs stay in the
        L2 caches and the 256 MiB Infinity Cache between calls);
  cold  each call preceded by a 512 MiB read of another buffer (L2 and the
        Infinity Cache evicted), inside a graph of such pairs; the graph of
        the flushes alone is timed too and subtracted, so every input comes
        from HBM.  HBM fractions are quoted on these.

Profiling mode (for rocprofv3 counter runs, which need a program that launches
only the kernels being measured): `python bench.py --only WORKLOAD --reps N`
runs one workload's calls N times after its setup and prints nothing else.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import re
import statistics
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


def sha256_of(t: torch.Tensor) -> str:
    return hashlib.sha256(t.detach().contiguous().cpu().view(torch.uint8).numpy().tobytes()).hexdigest()


# ------------------------------------------------------------------- timing

# untimed launches before a timed loop of long kernels: the GPU clock ramps
# up over the first tens of milliseconds of sustained load
LONG_WARMUP = 20
GRAPH_CALLS = 10   # calls captured per graph: spreads the graph launch over several calls


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


def time_graph(fn, iters, warmup, per=GRAPH_CALLS):
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


class Flush:
    """Evicts the L2 caches and the 256 MiB Infinity Cache: a read of 512 MiB
    of another buffer (clean lines: a scratch write would leave dirty lines
    whose write-back then lands inside the timed kernel)."""

    def __init__(self):
        self.r = torch.ones((512 << 20) // 4, dtype=torch.float32, device="cuda")
        self.acc = torch.empty((), dtype=torch.float32, device="cuda")

    def __call__(self):
        torch.sum(self.r, dim=0, out=self.acc)


_FLUSH = None


def flusher():
    global _FLUSH
    if _FLUSH is None:
        _FLUSH = Flush()
    return _FLUSH


def time_cold(fn, n=20, reps=9):
    """ms of one call of fn with cold caches: a graph of n (flush, fn) pairs
    against a graph of the n flushes alone, replayed alternately, the
    difference of the medians per call.  (Timing single replays with events
    instead would add the graph launch to every call.)"""
    fl = flusher()

    def pair():
        fl()
        fn()
    graphs = [capture(pair, n), capture(fl, n)]
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    v = [[], []]
    for _ in range(reps):
        for i, g in enumerate(graphs):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            g.replay()
            e1.record(s)
            e1.synchronize()
            v[i].append(e0.elapsed_time(e1))
    return max(statistics.median(v[0]) - statistics.median(v[1]), 0.0) / n


def roofline(bound, achieved, peak, unit, traffic=None, **extra):
    r = {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 5), "traffic": traffic}
    r.update(extra)
    return r


def code_sha256(src: str) -> str:
    """sha256 of a C++ source with its // comments and blank lines removed
    (a comment edit does not make the counters stale; a code edit does)."""
    lines = []
    for ln in src.splitlines():
        ln = re.sub(r"//.*$", "", ln).rstrip()
        if ln.strip():
            lines.append(ln)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def sources_sha256(names) -> str:
    parts = []
    for name in names:
        with open(os.path.join(ROOT, "sparse_attention_paged_amd", "csrc", name)) as f:
            parts.append(f.read())
    return code_sha256("\n".join(parts))


# which kernel sources each counted-traffic entry depends on
TRAFFIC_SOURCES = {
    "attn_dec": ("attn_dec.hip", "attn_common.hpp", "formats.hpp"),
    "attn_d512": ("attn_d512.hip", "attn_common.hpp"),
    "indexer": ("indexer.hip", "formats.hpp"),
}


def counted_traffic(key):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
    (profiles/traffic_counters.json), or None when the kernel sources
    changed since the counters were taken."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic_counters.json")) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        return None
    e = doc.get("entries", {}).get(key)
    if not e:
        return None
    if sources_sha256(TRAFFIC_SOURCES[e["sources"]]) != e["code_sha256"]:
        return None
    return e["traffic_bytes"]


# the pages' attention shapes ("perf(kernel): keep 16-byte kv loads ...", All
# shapes) and indexer shapes ("perf(kernel): read dsv41 indexer key rows as
# int32 words", All shapes): H100 80GB time of the final Triton kernel, as
# context only
PAGES_H100_US = {
    "prefill_s2048_r4": 2887.86, "prefill_s8192_r4": 11399.31, "prefill_s4096_at28672_r4": 5762.74,
    "prefill_s8192_r128": 3672.89, "prefill_s8192_r0": 2561.59,
    "decode_b1_r4": 16.83, "decode_b1_r128": 15.98, "decode_b1_r0": 13.37,
    "decode_b8_r4": 20.81, "decode_b8_r128": 17.73, "decode_b8_r0": 13.89,
    "indexer_b1_n16384": 5.47, "indexer_b4_n16384": 16.39, "indexer_b1_n65536": 16.38,
    "indexer_b1_n131072": 31.37, "cand_b1": 4.51, "cand_b4": 9.17,
}


# ------------------------------------------------------------------ decode

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


class SweepDecode:
    """Decode attention for a batch sweep, generated on the device (seeded):
    B sequences at position 32767, each with its own 32768-row window pool
    and 8192-row compressed pool (r = 4) in 64-row pages under random page
    tables, 512 distinct random compressed entries per token; bf16 rows
    ~N(0, 1), q ~N(0, 1), fp32 output."""

    def __init__(self, B, seed=W.SEED_BASE + 300):
        d = torch.device("cuda")
        gd = torch.Generator(device=d)
        gd.manual_seed(seed + B)
        gc = W.make_generator(seed + B)
        self.B, self.n_win, self.n_cmp, self.page = B, 128, 512, 64
        self.q = torch.randn((B, 64, 512), generator=gd, device=d, dtype=torch.bfloat16)
        self.win = torch.randn((B * 32768, 512), generator=gd, device=d, dtype=torch.bfloat16)
        self.cmp = torch.randn((B * 8192, 512), generator=gd, device=d, dtype=torch.bfloat16)
        win_pt = W.page_table(B, 512, gc).to(d)
        cmp_pt = W.page_table(B, 128, gc).to(d)
        r = torch.rand((B, 8192), generator=gd, device=d)
        sel = torch.topk(r, 512, dim=1, largest=False).indices.to(torch.int32)
        pos = torch.full((B,), 32767, dtype=torch.int32, device=d)
        seq = torch.arange(B, dtype=torch.int32, device=d)
        self.idx = sap.build_sparse_idx(pos, seq, 128, win_pt, 64, sel.contiguous(), cmp_pt)
        self.C = 640
        self.out = torch.empty((B, 64, 512), dtype=torch.float32, device=d)
        nb = sap.sparse_attn_workspace_bytes(B, 64, 512, self.C, 0)
        self.ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=d)
        self.splits = sap.sparse_attn_num_splits(B, 64, 512, self.C, 0)
        self.sm = 1.0 / math.sqrt(512)

    def attend(self):
        sap.sparse_attn_paged(self.q, self.win, self.cmp, self.idx, self.n_win, self.sm, out=self.out,
                              workspace=self.ws)

    def alg_bytes(self):
        return self.B * (64 * 512 * 2 + self.C * (1024 + 4) + 64 * 512 * 4)


def decode_secondary(B, kv, iters):
    st = DecodeStep(B=B, kv_dtype=kv, seed=W.SEED_BASE + (4 if kv == "e4m3" else 2))
    st.select()
    ms_attn = time_graph(st.attend, iters // GRAPH_CALLS, 1)
    ms_step = time_graph(st.step, iters // GRAPH_CALLS, 1)
    ms_cold = time_cold(st.attend)
    ms_step_cold = time_cold(st.step)
    alg = st.attn_alg_bytes()
    ctx = {"pages_h100_us": PAGES_H100_US[f"decode_b{B}_r4"]} if kv == "bf16" else {}
    return {"workload": f"decode_b{B}_pos32767_r4_{kv}", "attn_us": round(ms_attn * 1e3, 2),
            "attn_us_cold": round(ms_cold * 1e3, 2), **ctx,
            "step_us": round(ms_step * 1e3, 2), "step_us_cold": round(ms_step_cold * 1e3, 2),
            "gathered_GBs_attn": round(st.gathered_bytes() / (ms_attn * 1e-3) / 1e9, 1),
            "splits": st.splits, "out_sha256": sha256_of(st.out),
            "roofline": roofline("hbm", alg / (ms_cold * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s",
                                 bytes_per_launch=alg, timing="cold",
                                 frac_warm=round(alg / (ms_attn * 1e-3) / 1e9 / HBM_PEAK_GBS, 5))}


def decode_sweep(batches):
    """Attention alone (split-K + merge, or one pass per token once the batch
    fills the GPU) over a growing batch: where the HBM roof becomes reachable."""
    res = []
    for B in batches:
        log(f"secondary: decode sweep B{B}")
        sw = SweepDecode(B)
        ms = time_graph(sw.attend, 5, 1, per=4)
        ms_cold = time_cold(sw.attend, 10, 5)
        alg = sw.alg_bytes()
        res.append({"workload": f"decode_sweep_b{B}_pos32767_r4_bf16", "attn_us": round(ms * 1e3, 2),
                    "attn_us_cold": round(ms_cold * 1e3, 2), "splits": sw.splits, "alg_MB": round(alg / 1e6, 2),
                    "out_sha256": sha256_of(sw.out),
                    "roofline": roofline("hbm", alg / (ms_cold * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s",
                                         timing="cold",
                                         frac_warm=round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 5))})
        del sw
        torch.cuda.empty_cache()
    return res


def decode_pages_shapes():
    res = []
    for B in (1, 8):
        for ratio in (128, 0):
            st = DecodeStep(B=B, ratio=ratio)
            st.select()
            ms = time_graph(st.attend, 100 // GRAPH_CALLS, 1)
            ms_cold = time_cold(st.attend)
            name = f"decode_b{B}_r{ratio}"
            alg = st.attn_alg_bytes()
            res.append({"workload": name + "_pos32767_bf16", "attn_us": round(ms * 1e3, 2),
                        "attn_us_cold": round(ms_cold * 1e3, 2), "pages_h100_us": PAGES_H100_US[name],
                        "splits": st.splits, "out_sha256": sha256_of(st.out),
                        "roofline": roofline("hbm", alg / (ms_cold * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s",
                                             timing="cold")})
    return res


# ----------------------------------------------------------------- prefill

class Prefill:
    def __init__(self, T=8192, start=0, ratio=4, kv="bf16", out_dtype=torch.float32):
        if kv == "e4m3":
            seed = W.SEED_BASE + (35 if start == 0 else 36)
            case = W.prefill_case(T=T, start=start, ratio=ratio, kv_dtype="e4m3", q_scale=2.0 ** -7, seed=seed)
        else:
            seed = {4: 3, 128: 31, 0: 32}[ratio] if start == 0 and T == 8192 else 33
            case = W.prefill_case(T=T, start=start, ratio=ratio, seed=W.SEED_BASE + seed)
        d = torch.device("cuda")
        self.case = case
        self.q, self.win = case.q.to(d), case.win_pool.to(d)
        self.cmp = case.cmp_pool.to(d) if case.n_cmp > 0 else None
        self.wsc = case.win_scale.to(d) if case.win_scale is not None else None
        self.csc = case.cmp_scale.to(d) if case.cmp_scale is not None else None
        self.idx = sap.build_sparse_idx(case.pos.to(d), case.seq.to(d), case.n_win, case.win_pt.to(d), case.page,
                                        case.cmp_logical.to(d) if case.n_cmp > 0 else None,
                                        case.cmp_pt.to(d) if case.n_cmp > 0 else None)
        self.out = torch.empty((case.T, 64, 512), dtype=out_dtype, device=d)
        self.valid = int((self.idx >= 0).sum().item())
        # HBM bytes the launch cannot avoid: q, out, the index rows and every
        # distinct pool row it references (once)
        v = self.idx[self.idx >= 0].to(torch.int64)
        col = torch.arange(self.idx.shape[1], device=d).expand_as(self.idx)[self.idx >= 0]
        key = torch.where(col < case.n_win, v, v + (1 << 40))
        uniq = int(torch.unique(key).numel())
        rb = 512 * self.win.element_size() + (4 if self.wsc is not None else 0)
        self.hbm_bytes = (self.q.numel() * 2 + self.out.numel() * self.out.element_size() +
                          self.idx.numel() * 4 + uniq * rb)

    def run(self):
        sap.sparse_attn_paged(self.q, self.win, self.cmp, self.idx, self.case.n_win, self.case.sm_scale,
                              out=self.out, win_scale=self.wsc, cmp_scale=self.csc, num_splits=1)


def prefill_line(name, pf: Prefill, iters, traffic_key=None):
    ms = time_loop(pf.run, iters, LONG_WARMUP)
    flops = pf.valid * 64 * 512 * 4.0
    tf = flops / (ms * 1e-3) / 1e12
    gbs = pf.hbm_bytes / (ms * 1e-3) / 1e9
    t_mfma, t_hbm = flops / (BF16_PEAK_TFLOPS * 1e12), pf.hbm_bytes / (HBM_PEAK_GBS * 1e9)
    traffic = counted_traffic(traffic_key) if traffic_key else None
    # the binding roof is the one with the longer ideal time
    if t_mfma >= t_hbm:
        rf = roofline("mfma", tf, BF16_PEAK_TFLOPS, "TFLOP/s", traffic=traffic,
                      frac_hbm=round(gbs / HBM_PEAK_GBS, 5))
    else:
        rf = roofline("hbm", gbs, HBM_PEAK_GBS, "GB/s", traffic=traffic,
                      frac_mfma=round(tf / BF16_PEAK_TFLOPS, 5))
    ctx = {}
    base = name.replace("_bf16out", "").replace("_e4m3", "").replace("_bf16", "")
    if name.endswith("_bf16") and base in PAGES_H100_US:
        ctx = {"pages_h100_us": PAGES_H100_US[base]}
    return {"workload": name, "us": round(ms * 1e3, 2), "tflops": round(tf, 2), **ctx,
            "gflop": round(flops / 1e9, 2), "hbm_GB": round(pf.hbm_bytes / 1e9, 4),
            "out_sha256": sha256_of(pf.out), "roofline": rf}


def prefill_secondary():
    res = []
    for name, kw, iters in (("prefill_s8192_r4_bf16", dict(), 10),
                            ("prefill_s8192_r4_bf16out", dict(out_dtype=torch.bfloat16), 10),
                            ("prefill_s8192_r4_e4m3", dict(kv="e4m3"), 5),
                            ("prefill_s2048_r4_bf16", dict(T=2048), 5),
                            ("prefill_s4096_at28672_r4_bf16", dict(T=4096, start=28672), 5),
                            ("prefill_s8192_r128_bf16", dict(ratio=128), 5),
                            ("prefill_s8192_r0_bf16", dict(ratio=0), 5)):
        log(f"secondary: {name}")
        pf = Prefill(**kw)
        key = name if name == "prefill_s8192_r4_bf16" else None
        res.append(prefill_line(name, pf, iters, traffic_key=key))
        del pf
        torch.cuda.empty_cache()
    return res


# ----------------------------------------------------- indexer and top-k

class Indexer:
    def __init__(self, B, N, seed=None):
        self.case = case = W.indexer_case(B=B, N=N, seed=seed if seed is not None else W.SEED_BASE + 5)
        d = torch.device("cuda")
        self.B, self.N = B, N
        self.q, self.w = case.q.to(d), case.w.to(d)
        self.pool, self.pt = case.key_pool.to(d), case.page_table.to(d)
        self.out = torch.empty((B, N), dtype=torch.float32, device=d)
        self.sel = torch.empty((B, 512), dtype=torch.int32, device=d)
        self.ws = torch.empty(max(sap.topk_workspace_bytes(B, N, 512), 1), dtype=torch.uint8, device=d)

    def logits(self):
        sap.indexer_logits_packed(self.q, self.w, self.pool, self.pt, self.case.page, self.N, out=self.out)

    def topk(self):
        sap.topk_select(self.out, 512, out=self.sel, workspace=self.ws)

    def alg_bytes(self):
        return self.B * (self.N * 68 + self.N * 4 + 32 * 128 * 2 + 32 * 4)


def indexer_secondary(B, N, iters, pages_key=None, topk=False):
    ix = Indexer(B, N)
    ms = time_graph(ix.logits, iters // GRAPH_CALLS, 1)
    ms_cold = time_cold(ix.logits)
    alg = ix.alg_bytes()
    key = f"indexer_b{B}_n{N}"
    res = {"workload": f"indexer_b{B}_n{N}", "indexer_us": round(ms * 1e3, 2),
           "indexer_us_cold": round(ms_cold * 1e3, 2), "logits_sha256": sha256_of(ix.out)}
    if pages_key:
        res["pages_h100_us"] = PAGES_H100_US[pages_key]
    if topk:
        res["topk512_us"] = round(time_graph(ix.topk, iters // GRAPH_CALLS, 1) * 1e3, 2)
        res["topk512_us_cold"] = round(time_cold(ix.topk) * 1e3, 2)
        res["topk_sha256"] = sha256_of(ix.sel)
    res["roofline"] = roofline("hbm", alg / (ms_cold * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s",
                               traffic=counted_traffic(key), bytes_per_launch=alg, timing="cold",
                               frac_warm=round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 5))
    return res


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

    def run():
        sap.indexer_logits_candidates(q, w, pool, pt, case.page, cand, n_keys=nk, out=out)
    ms = time_graph(run, iters // GRAPH_CALLS, 1)
    ms_cold = time_cold(run)
    # per candidate: the 68-byte key row, its index and its logit
    alg = T * case.NC * (68 + 4 + 4)
    kind = "prefill_n128" if shared else f"decode_b{T}"
    ctx = {} if shared else {"pages_h100_us": PAGES_H100_US[f"cand_b{T}"]}
    return {"workload": f"indexer_cand_{kind}_ctx131072_nc16384", "us": round(ms * 1e3, 2),
            "us_cold": round(ms_cold * 1e3, 2), **ctx, "logits_sha256": sha256_of(out),
            "roofline": roofline("hbm", alg / (ms_cold * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", timing="cold")}


def gated_pool_secondary(B, R, D, iters):
    case = W.gated_pool_case(B=B, R=R, D=D, seed=W.SEED_BASE + 700 + B + R + D)
    x, g = case.x.cuda(), case.gate.cuda()
    out = torch.empty((B, D), dtype=torch.float32, device="cuda")

    def run():
        sap.gated_pool(x, g, out=out)
    ms = time_graph(run, iters // GRAPH_CALLS, 1)
    ms_cold = time_cold(run)
    # bf16 rows, fp32 gates in; fp32 pooled rows out
    alg = B * R * D * (2 + 4) + B * D * 4
    return {"workload": f"gated_pool_b{B}_r{R}_d{D}", "us": round(ms * 1e3, 2), "us_cold": round(ms_cold * 1e3, 2),
            "out_sha256": sha256_of(out),
            "roofline": roofline("hbm", alg / (ms_cold * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", timing="cold")}


# ---------------------------------------------------------- CPU baseline

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


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
            "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count(),
            "kind": "oracle", "sample": f"{reps} full decode steps (B{st.B}, indexer over {st.n_c} keys, "
                                        f"top-{c.n_cmp}, attention over {st.C} rows), {per * 1e3:.1f} ms each"}


# ------------------------------------------------------- profiling mode

def only(workload: str, reps: int) -> None:
    """Run one workload's calls `reps` times (for rocprofv3 counter runs)."""
    if workload == "prefill":
        pf = Prefill()
        torch.cuda.synchronize()
        for _ in range(reps):
            pf.run()
    elif workload in ("decode_attn", "decode_step"):
        st = DecodeStep(B=1)
        st.select()
        torch.cuda.synchronize()
        for _ in range(reps):
            st.attend() if workload == "decode_attn" else st.step()
    elif workload in ("indexer_b1", "indexer_b4"):
        ix = Indexer(int(workload[-1]), 131072)
        torch.cuda.synchronize()
        for _ in range(reps):
            ix.logits()
    elif workload == "copy":
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(reps):
            b.copy_(a)
    else:
        raise SystemExit(f"unknown workload {workload}")
    torch.cuda.synchronize()
    log(f"{workload}: {reps} runs done")


# ------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--only", default=None,
                    help="profiling mode: prefill | decode_attn | decode_step | indexer_b1 | indexer_b4 | copy")
    ap.add_argument("--reps", type=int, default=3)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(each GPU would run its own sequences with no exchange)", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.only:
        only(args.only, args.reps)
        return
    log("building decode step inputs (B1, position 32767, r4)")
    st = DecodeStep(B=1, pos=32767, ratio=4)

    log("timing whole steps (graph replays; eager launches for reference)")
    # a graph holds GRAPH_CALLS steps back to back; K = steps (a multiple of it)
    reps = max(1, args.steps // GRAPH_CALLS)
    args.steps = reps * GRAPH_CALLS
    ms_step = time_graph(st.step, reps, max(1, args.warmup // GRAPH_CALLS))
    ms_step_eager = time_loop(st.step, args.steps, args.warmup)
    log("timing the attention launches alone, warm and cold")
    ms_attn = time_graph(st.attend, reps, 1)
    ms_sel = time_graph(st.select, reps, 1)
    ms_step_cold = time_cold(st.step)
    ms_attn_cold = time_cold(st.attend)
    ms_sel_cold = time_cold(st.select)
    value = st.gathered_bytes() / (ms_step * 1e-3) / 1e9
    alg = st.attn_alg_bytes()

    res = {
        "metric": METRIC, "value": round(value, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode_b1_pos32767_r4_bf16", "global_batch": 1, "seq_len": 32768, "heads": 64,
                   "head_dim": 512, "window": 128, "topk": 512, "ratio": 4, "parallelism": "single-gpu",
                   "step": "indexer(8192 fp4 keys) + top-512 fused with the index build + split-K attention + merge"},
        "timing": f"HIP-graph replays ({GRAPH_CALLS} steps per graph), HIP events around the timed replays",
        "eager_ms_per_step": round(ms_step_eager, 5), "cold_ms_per_step": round(ms_step_cold, 5),
        "attn_us": round(ms_attn * 1e3, 3), "attn_us_cold": round(ms_attn_cold * 1e3, 3),
        "select_us": round(ms_sel * 1e3, 3), "select_us_cold": round(ms_sel_cold * 1e3, 3),
        "splits": st.splits, "out_sha256": sha256_of(st.out), "idx_sha256": sha256_of(st.idx),
        "context": {"pages_h100_attn_us": PAGES_H100_US["decode_b1_r4"],
                    "note": "the pages' H100 Triton time for this attention call alone; another machine"},
        "roofline": roofline("hbm", alg / (ms_attn * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s",
                             traffic=counted_traffic("decode_b1_r4_bf16_attention"),
                             kernel="sparse attention for one decode token (all its launches)",
                             bytes_per_launch=alg,
                             achieved_cold=round(alg / (ms_attn_cold * 1e-3) / 1e9, 3),
                             frac_cold=round(alg / (ms_attn_cold * 1e-3) / 1e9 / HBM_PEAK_GBS, 5)),
    }
    if not args.no_secondary:
        sec = []
        for B, kv in ((8, "bf16"), (8, "e4m3")):
            log(f"secondary: decode B{B} {kv}")
            sec.append(decode_secondary(B, kv, 100))
        log("secondary: decode r128 / r0")
        sec.extend(decode_pages_shapes())
        sec.extend(decode_sweep((8, 16, 32, 64, 128, 256)))
        sec.extend(prefill_secondary())
        for B, N, pk, tk in ((1, 131072, "indexer_b1_n131072", True), (4, 131072, None, True),
                             (1, 16384, "indexer_b1_n16384", False), (4, 16384, "indexer_b4_n16384", False),
                             (1, 65536, "indexer_b1_n65536", False)):
            log(f"secondary: indexer B{B} N{N}")
            sec.append(indexer_secondary(B, N, 100, pk, tk))
        for length, start, ratio in ((2048, 129024, 2), (8192, 0, 2)):
            log(f"secondary: indexer prefill n{length} start{start} r{ratio}")
            sec.append(indexer_prefill_secondary(length, start, ratio, 5))
        for T, shared in ((1, False), (4, False), (128, True)):
            log(f"secondary: indexer candidates T{T}")
            sec.append(indexer_cand_secondary(T, shared, 100))
        for B, R in ((1, 128), (8, 128), (8, 8)):
            log(f"secondary: gated pool B{B} R{R} D512")
            sec.append(gated_pool_secondary(B, R, 512, 100))
        res["secondary"] = sec
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on the same decode step")
        res["cpu_baseline"] = cpu_baseline(st, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
