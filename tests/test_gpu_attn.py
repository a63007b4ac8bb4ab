"""GPU parity of the index build and of sparse attention (prefill and split-K
decode, bf16 and e4m3 rows) against the CPU oracle on the same seeded inputs.

Workloads follow the pages' shapes ('perf(kernel): keep 16-byte kv loads in
dsv4 sparse attention and unroll gated pool', Kernel time: 64 heads,
head_dim 512, 128-token window, index top-k 512, r in {4, 128, 0}, decode at
position 32767 with B 1 / 8, prefill S8192 and a 4096 chunk at 28672) and
its edge-case list (Correctness and tests: 20/16/128 heads, windows of 100
and 50, top-k widths that are not tile multiples, zero counts, the ratio-0
alias and pool views with a row offset).  The fp8 case follows 'Perf/kv fp8
read path' (What this changes).
"""
import dataclasses
import hashlib
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_paged_amd as sap
import workloads as W
from gpu_helpers import assert_attn_close, dev, gpu_attn, gpu_idx, need_gpu, say

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------- index build

@pytest.mark.parametrize("kind", ["decode_b8_r4", "prefill_r4", "prefill_r128_at", "decode_b3_r0"])
def test_index_build_bit_exact(kind):
    need_gpu()
    if kind == "decode_b8_r4":
        case = W.decode_case(B=8, ratio=4, H=1, D=64, seed=101)
    elif kind == "prefill_r4":
        case = W.prefill_case(T=1000, ratio=4, H=1, D=64, seed=102)
    elif kind == "prefill_r128_at":
        case = W.prefill_case(T=700, start=28672, ratio=128, H=1, D=64, seed=103)
    else:
        case = W.decode_case(B=3, pos=100, ratio=0, H=1, D=64, seed=104)
    say(f"  index build {case.name}")
    got = gpu_idx(case).cpu()
    ref = oracle.case_idx(case)
    assert torch.equal(got, ref)


# ------------------------------------------------------------------- small case

def test_tiny_case_bf16_copy():
    need_gpu()
    case = W.tiny_case()
    q = case.q.to(torch.bfloat16)
    wp = case.win_pool.to(torch.bfloat16)
    cp = case.cmp_pool.to(torch.bfloat16)
    idx = oracle.case_idx(case)
    ref = oracle.sparse_attn(q, wp, cp, idx, case.n_win, case.sm_scale)
    for splits in (1, 0, 3):
        out = gpu_attn(case, idx=dev(idx), q=q, win_pool=wp, cmp_pool=cp, num_splits=splits)
        assert_attn_close(out, ref, f"tiny splits={splits}")


# ----------------------------------------------------------------------- decode

@pytest.mark.parametrize("B", [1, 8])
@pytest.mark.parametrize("ratio", [4, 128, 0])
def test_decode_bf16(B, ratio):
    need_gpu()
    case = W.decode_case(B=B, ratio=ratio, seed=W.SEED_BASE + 2 + 10 * B + ratio)
    say(f"  {case.name}: n_cmp {case.n_cmp}")
    idx = oracle.case_idx(case)
    ref = oracle.case_attn(case, idx=idx)
    gidx = gpu_idx(case)
    assert torch.equal(gidx.cpu(), idx)
    outs = {}
    for splits in (0, 1, 2, 5):
        outs[splits] = gpu_attn(case, idx=gidx, num_splits=splits)
        assert_attn_close(outs[splits], ref, f"splits={splits} (runs {sap.sparse_attn_num_splits(case.T, 64, 512, idx.shape[1], splits)})")
    # The merge is exact algebra, but each split rounds its softmax weights to
    # bf16 relative to its own running max, so split counts agree with each
    # other only within the same bf16-weight budget as with the oracle.
    for s in (0, 2, 5):
        d = (outs[s] - outs[1]).double()
        rel = (d.norm() / outs[1].double().norm()).item()
        assert d.abs().max().item() <= 1e-2 and rel <= 2e-3, (s, rel)


@pytest.mark.parametrize("B,kv", [(16, "bf16"), (32, "bf16"), (64, "bf16"), (64, "e4m3")])
def test_decode_resident_batches(B, kv):
    """Batches whose automatic plan keeps every decode workgroup resident on
    its own CU: B16 runs 3 splits of 2 rounds, B32 2 splits of 3, B64 one
    split of 5 rounds and no merge (each round's row indices load during the
    round before)."""
    need_gpu()
    case = W.decode_case(B=B, ratio=4, kv_dtype=kv, seed=W.SEED_BASE + 140 + B)
    idx = oracle.case_idx(case)
    ref = oracle.case_attn(case, idx=idx)
    runs = sap.sparse_attn_num_splits(case.T, 64, 512, idx.shape[1], 0)
    say(f"  {case.name}: {runs} splits")
    out = gpu_attn(case, idx=dev(idx), num_splits=0)
    assert_attn_close(out, ref, f"B{B} {kv} auto ({runs} splits)")


def test_decode_fp8_b8():
    need_gpu()
    case = W.decode_case(B=8, ratio=4, kv_dtype="e4m3", seed=W.SEED_BASE + 4)
    idx = oracle.case_idx(case)
    ref = oracle.case_attn(case, idx=idx)
    say(f"  {case.name}: |ref| max {ref.abs().max().item():.1f}")
    for splits in (0, 1):
        out = gpu_attn(case, idx=dev(idx), num_splits=splits)
        assert_attn_close(out, ref, f"fp8 splits={splits}")


# ---------------------------------------------------------------------- prefill

def _sample_tokens(T, n_rand, seed):
    g = torch.Generator().manual_seed(seed)
    fixed = [0, 1, 2, 3, 31, 32, 63, 64, 127, 128, 129, 511, 512, 513, T // 2, T - 2, T - 1]
    fixed = [t for t in fixed if t < T]
    rnd = torch.randint(0, T, (n_rand,), generator=g).tolist()
    return sorted(set(fixed + rnd))


@pytest.mark.parametrize("variant", ["r4_s8192", "r128_s8192", "r0_s8192", "r4_s4096_at28672",
                                     "r4_s8192_e4m3", "r4_s4096_at28672_e4m3"])
def test_prefill_sampled(variant):
    need_gpu()
    if variant == "r4_s8192_e4m3":
        # fp8 KV in prefill: the e4m3 read path with per-row scales (q carries 2^-7)
        case = W.prefill_case(T=8192, ratio=4, kv_dtype="e4m3", q_scale=2.0 ** -7, seed=W.SEED_BASE + 35)
    elif variant == "r4_s4096_at28672_e4m3":
        # a chunk of chunked prefill re-reading an e4m3 prefix
        case = W.prefill_case(T=4096, start=28672, ratio=4, kv_dtype="e4m3", q_scale=2.0 ** -7,
                              seed=W.SEED_BASE + 36)
    elif variant == "r4_s8192":
        case = W.prefill_case(T=8192, ratio=4)
    elif variant == "r128_s8192":
        case = W.prefill_case(T=8192, ratio=128, seed=W.SEED_BASE + 31)
    elif variant == "r0_s8192":
        case = W.prefill_case(T=8192, ratio=0, seed=W.SEED_BASE + 32)
    else:
        case = W.prefill_case(T=4096, start=28672, ratio=4, seed=W.SEED_BASE + 33)
    say(f"  {case.name}: full GPU run, oracle on sampled tokens")
    gidx = gpu_idx(case)
    out = gpu_attn(case, idx=gidx, num_splits=1)
    toks = _sample_tokens(case.T, 24, 7)
    idx = oracle.case_idx(case)
    assert torch.equal(gidx.cpu(), idx)
    ref = oracle.sparse_attn(case.q[toks], case.win_pool, case.cmp_pool, idx[toks], case.n_win, case.sm_scale,
                             case.win_scale, case.cmp_scale)
    assert_attn_close(out[toks], ref, f"{len(toks)} sampled tokens")


def test_prefill_every_workgroup_slot_two_rounds():
    """The prefill launch at head_dim 512 runs 256 persistent workgroups over
    the tokens in rounds of 256 (round r holds tokens 256r .. 256r+255, each
    XCD a block of 32 consecutive tokens): tokens 0 .. 511 put every
    (workgroup, round) slot of the first two rounds against the oracle, and
    the last two rounds (the tokens with the most columns) follow."""
    need_gpu()
    case = W.prefill_case(T=8192, ratio=4)
    gidx = gpu_idx(case)
    out = gpu_attn(case, idx=gidx, num_splits=1)
    idx = oracle.case_idx(case)
    assert torch.equal(gidx.cpu(), idx)
    for lo, hi in ((0, 512), (8192 - 512, 8192)):
        toks = list(range(lo, hi))
        ref = oracle.sparse_attn(case.q[toks], case.win_pool, case.cmp_pool, idx[toks], case.n_win, case.sm_scale)
        assert_attn_close(out[toks], ref, f"tokens {lo} .. {hi - 1}")


def test_prefill_small_full():
    # every token, ragged tail of the last tile, tokens whose window is clipped
    need_gpu()
    case = W.prefill_case(T=333, ratio=4, topk=70, seed=W.SEED_BASE + 34)
    idx = oracle.case_idx(case)
    ref = oracle.case_attn(case, idx=idx)
    assert_attn_close(gpu_attn(case, num_splits=1), ref, "prefill T=333 top-k 70")
    assert_attn_close(gpu_attn(case, num_splits=0), ref, "prefill T=333 auto")


# ------------------------------------------------------------------- edge cases

@pytest.mark.parametrize("H", [20, 16, 128, 1])
def test_head_counts(H):
    need_gpu()
    case = W.decode_case(B=2, pos=4000, ratio=4, H=H, seed=W.SEED_BASE + 40 + H)
    ref = oracle.case_attn(case)
    assert_attn_close(gpu_attn(case), ref, f"H={H} auto")
    assert_attn_close(gpu_attn(case, num_splits=1), ref, f"H={H} one split")


def test_prefill_persistent_chunks_partial_heads():
    """More tokens than workgroups (the prefill launch at head_dim 512 then
    gives a workgroup several tokens), a partial head block (H = 20, where the
    next token's loads wait for every store of the previous one) and more
    columns than one staged index chunk (3128 > 2048)."""
    need_gpu()
    case = W.prefill_case(T=300, start=16000, ratio=4, topk=3000, H=20, seed=W.SEED_BASE + 96)
    assert oracle.case_idx(case).shape[1] > 2048
    ref = oracle.case_attn(case)
    assert_attn_close(gpu_attn(case, num_splits=1), ref, "prefill T=300 H=20 3128 columns")


def _late_jump_case(kv: str, seed: int):
    """One token over 96 columns (three tiles) whose third tile holds a row
    aligned with head 5's query: that head's running max jumps by hundreds of
    log2 units after the first tile, and so do several other heads' (by tens).
    Without the rescale the weights of such a head overflow."""
    g = torch.Generator().manual_seed(seed)
    H, D, N = 64, 512, 96
    q = torch.randn((1, H, D), generator=g)
    if kv == "bf16":
        # rows of the workload's size; head 5's query 8x larger, so that its
        # score against row 70 passes 2^128 in the weights' exponent
        q[0, 5] *= 8.0
        q = q.to(torch.bfloat16)
        sgn = torch.where(q[0, 5].float() >= 0, 1.0, -1.0)
        pool = torch.randn((N, D), generator=g).to(torch.bfloat16)
        pool[70] = (2.0 * sgn).to(torch.bfloat16)
        scale = None
    else:
        q = q.to(torch.bfloat16)
        sgn = torch.where(q[0, 5].float() >= 0, 1.0, -1.0)
        vals = torch.tensor([-1.0, -0.5, 0.5, 1.0])[torch.randint(0, 4, (N, D), generator=g)]
        vals[70] = 16.0 * sgn
        pool = vals.to(torch.float8_e4m3fn).view(torch.uint8)
        scale = torch.exp2(torch.rand(N, generator=g) * 2.0 - 1.0).to(torch.float32)
    idx = torch.arange(N, dtype=torch.int32)[None, :]
    return q, pool, scale, idx


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
def test_late_max_jump_on_any_head(kv):
    """The one-pass kernel rescales when a later tile's max passes the
    running max by more than its slack: every head of the wave must be able
    to raise that flag, not only the first of each 16-head tile."""
    need_gpu()
    q, pool, scale, idx = _late_jump_case(kv, 180 + (kv == "e4m3"))
    sm = 1.0 / math.sqrt(512)
    ref = oracle.sparse_attn(q, pool, None, idx, idx.shape[1], sm, scale, None)
    out = sap.sparse_attn_paged(dev(q), dev(pool), None, dev(idx), idx.shape[1], sm,
                                win_scale=dev(scale), num_splits=1)
    torch.cuda.synchronize()
    assert_attn_close(out, ref, f"late max jump {kv}")


@pytest.mark.parametrize("n_win,topk", [(100, 512), (50, 37), (128, 300), (128, 1), (0, 64), (1, 0)])
def test_window_and_topk_widths(n_win, topk):
    need_gpu()
    case = W.prefill_case(T=260, start=900, ratio=4, n_win=n_win, topk=topk, seed=W.SEED_BASE + 50 + n_win + topk)
    ref = oracle.case_attn(case)
    assert_attn_close(gpu_attn(case, num_splits=1), ref, f"window {n_win} top-k {topk}")
    assert_attn_close(gpu_attn(case, num_splits=0), ref, f"window {n_win} top-k {topk} auto")


@pytest.mark.parametrize("D", [64, 128, 256])
def test_head_dims(D):
    need_gpu()
    case = W.decode_case(B=4, pos=3000, ratio=4, H=64, D=D, topk=200, seed=W.SEED_BASE + 60 + D)
    ref = oracle.case_attn(case)
    assert_attn_close(gpu_attn(case), ref, f"D={D}")
    case8 = W.decode_case(B=2, pos=3000, ratio=4, H=64, D=D, topk=200, kv_dtype="e4m3", seed=W.SEED_BASE + 61 + D)
    assert_attn_close(gpu_attn(case8), oracle.case_attn(case8), f"D={D} e4m3")


def test_zero_counts_and_empty_rows():
    need_gpu()
    case = W.decode_case(B=4, pos=2000, ratio=4, topk=128, seed=W.SEED_BASE + 70)
    idx = oracle.case_idx(case)
    idx[1, :] = -1                       # a token with no valid column -> zeros
    idx[2, case.n_win:] = -1             # window only
    idx[3, :case.n_win] = -1             # compressed only
    idx[3, case.n_win + 5:case.n_win + 40] = -1
    ref = oracle.case_attn(case, idx=idx)
    for splits in (1, 0, 4):
        out = gpu_attn(case, idx=dev(idx), num_splits=splits)
        assert (out[1] == 0).all()
        assert_attn_close(out, ref, f"holes splits={splits}")
    # no columns at all
    e = torch.zeros((case.T, 0), dtype=torch.int32)
    out = sap.sparse_attn_paged(dev(case.q), dev(case.win_pool), None, dev(e), 0, case.sm_scale)
    torch.cuda.synchronize()
    assert (out == 0).all()


def test_ratio0_alias_and_row_offset_views():
    need_gpu()
    case = W.decode_case(B=2, pos=1500, ratio=4, topk=100, seed=W.SEED_BASE + 80)
    idx = oracle.case_idx(case)
    # ratio-0 alias: no compressed columns, the compressed pool pointer aliases the window pool
    widx = idx[:, :case.n_win].contiguous()
    ref0 = oracle.sparse_attn(case.q, case.win_pool, case.win_pool, widx, case.n_win, case.sm_scale)
    wp = dev(case.win_pool)
    out0 = sap.sparse_attn_paged(dev(case.q), wp, wp, dev(widx), case.n_win, case.sm_scale)
    torch.cuda.synchronize()
    assert_attn_close(out0, ref0, "ratio-0 alias")
    # pool views with a row offset (bases stay 16-byte aligned)
    off_w, off_c = 3, 5
    big_w = torch.cat([torch.zeros(off_w, case.D, dtype=torch.bfloat16), case.win_pool])
    big_c = torch.cat([torch.zeros(off_c, case.D, dtype=torch.bfloat16), case.cmp_pool])
    gw, gc = dev(big_w)[off_w:], dev(big_c)[off_c:]
    out1 = sap.sparse_attn_paged(dev(case.q), gw, gc, dev(idx), case.n_win, case.sm_scale)
    torch.cuda.synchronize()
    assert_attn_close(out1, oracle.case_attn(case, idx=idx), "row-offset views")
    # rows padded to a longer stride
    pad = torch.zeros(case.win_pool.shape[0], case.D + 64, dtype=torch.bfloat16)
    pad[:, :case.D] = case.win_pool
    out2 = sap.sparse_attn_paged(dev(case.q), dev(pad)[:, :case.D], dev(case.cmp_pool), dev(idx), case.n_win,
                                 case.sm_scale)
    torch.cuda.synchronize()
    assert_attn_close(out2, oracle.case_attn(case, idx=idx), "strided rows")


def test_bf16_output():
    # A bf16 output adds one rounding on top of the fp32-output bar: half an
    # ulp of an 8-bit significand, at most 2^-8 |x| (just above a power of
    # two), so rel-L2 grows by 2^-8 and max-abs by 2^-8 max|ref|.
    need_gpu()
    for case, splits in ((W.decode_case(B=8, ratio=4, seed=W.SEED_BASE + 90), 0),
                         (W.prefill_case(T=300, ratio=4, seed=W.SEED_BASE + 91), 1)):
        ref = oracle.case_attn(case)
        out = gpu_attn(case, out_dtype=torch.bfloat16, num_splits=splits)
        assert out.dtype == torch.bfloat16
        bound = 1e-2 + 2.0 ** -8 * ref.abs().max().item()
        assert_attn_close(out.float(), ref, f"bf16 out {case.name}", max_abs=bound, rel_l2=2e-3 + 2.0 ** -8)


def test_determinism_sha256():
    need_gpu()
    for case, splits in ((W.prefill_case(T=1024, ratio=4, seed=W.SEED_BASE + 95), 1),
                         (W.decode_case(B=8, ratio=4, seed=W.SEED_BASE + 96), 0),
                         (W.decode_case(B=8, ratio=4, kv_dtype="e4m3", seed=W.SEED_BASE + 97), 0)):
        gidx = gpu_idx(case)
        h = set()
        for _ in range(3):
            out = gpu_attn(case, idx=gidx, num_splits=splits)
            h.add(hashlib.sha256(out.cpu().numpy().tobytes()).hexdigest())
        assert len(h) == 1, case.name


@pytest.mark.parametrize("B", [1, 8])
def test_decode_merge_batches(B):
    """Split counts that take the merge batches of 16 and 24 splits (the
    launch picks the smallest batch that holds the split count), with
    one-wave merge workgroups (B1) and four-wave ones (B8): 1472 columns
    (46 tiles) in 16 splits of 3 tiles and 23 of 2, and the automatic count
    (23 splits at B1, 16 at B8)."""
    need_gpu()
    case = W.decode_case(B=B, topk=1344, seed=W.SEED_BASE + 130 + B)
    idx = oracle.case_idx(case)
    ref = oracle.case_attn(case, idx=idx)
    gidx = gpu_idx(case)
    for splits in (16, 23, 0):
        runs = sap.sparse_attn_num_splits(case.T, 64, 512, idx.shape[1], splits)
        say(f"  B{B} {idx.shape[1]} columns: {splits} splits requested, {runs} run")
        out = gpu_attn(case, idx=gidx, num_splits=splits)
        assert_attn_close(out, ref, f"B{B} splits={splits} (runs {runs})")


@pytest.mark.parametrize("k", [60, -60])
def test_decode_f16_partials_row_magnitudes(k):
    """bf16 rows: a split's partial O is stored in f16 after one power-of-two
    shift per head that brings its largest |O| to [2^14, 2^15), and the
    head's max is lowered by the shift.  Rows scaled by 2^k with q scaled by
    2^-k keep every score and scale every O by 2^k: against the oracle the
    bar scales with the rows, and the output is 2^k times the unscaled one
    up to the rounding of the shifted maxima in fp32 (a few ulps of the
    log2 max, far below the bar)."""
    need_gpu()
    case = W.decode_case(B=2, pos=4000, ratio=4, seed=W.SEED_BASE + 140)
    f = 2.0 ** k
    sc = dataclasses.replace(case, q=(case.q.float() / f).to(torch.bfloat16),
                             win_pool=(case.win_pool.float() * f).to(torch.bfloat16),
                             cmp_pool=(case.cmp_pool.float() * f).to(torch.bfloat16))
    gidx = gpu_idx(case)
    assert sap.sparse_attn_num_splits(case.T, 64, 512, gidx.shape[1], 5) == 5
    base = gpu_attn(case, idx=gidx, num_splits=5)
    out = gpu_attn(sc, idx=gidx, num_splits=5)
    assert torch.isfinite(out).all()
    rel = ((out / f - base).abs().max() / base.abs().max()).item()
    say(f"  rows x 2^{k}: largest deviation from 2^{k} x the unscaled output {rel:.2e} of max|out|")
    assert rel <= 1e-5, rel
    ref = oracle.case_attn(sc)
    assert_attn_close(out / f, ref / f, f"rows x 2^{k}, 5 splits")
