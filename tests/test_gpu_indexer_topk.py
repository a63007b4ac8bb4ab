"""GPU parity of the fp4 indexer logits and the exact top-k selection, and
the small end-to-end chain indexer -> top-k -> index build -> attention.

The indexer reads fp4_e8m0_b32 key rows ('perf(kernel): read dsv41 indexer
key rows as int32 words', Changes; Kernel time: 32 index heads, head_dim
128, decode at contexts of 32768 and 131072, B 1 and 4).

Logit tolerance: each head's dot product sums 128 exact bf16 x bf16
products in fp32 and the head sum adds 32 fp32 terms, so the rounding error
is below (128 + 32) * 2^-24 < 1e-5 of M = sum_h |w_h| sum_d |q_hd k_d|.
Top-k is compared bit for bit when both sides select from the same fp32
logits.
"""
import hashlib

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_paged_amd as sap
import workloads as W
from gpu_helpers import assert_attn_close, dev, need_gpu, say

pytestmark = pytest.mark.gpu


def _magnitude(case, rows_sel=None):
    """M[b, n] = sum_h |w_bh| sum_d |q_bhd k_nd| with keys decoded by the oracle."""
    B, N = case.q.shape[0], case.N
    M = np.zeros((B, N))
    for b in range(B):
        prow = (case.page_table[b].to(torch.int64).repeat_interleave(case.page) * case.page
                + torch.arange(case.page).repeat(case.page_table.shape[1]))[:N]
        k = np.abs(oracle.fp4_rows_decode(case.key_pool[prow]))            # [N, 128]
        q = np.abs(case.q[b].to(torch.float64).numpy())                     # [Hi, 128]
        w = np.abs(case.w[b].to(torch.float64).numpy())
        M[b] = (q @ k.T * w[:, None]).sum(0)
    return M


def _check_logits(got, ref, M, label):
    g = got.cpu().to(torch.float64).numpy()
    r = ref.numpy()
    inf = np.isinf(r)
    assert np.array_equal(np.isinf(g), inf) and (g[inf] < 0).all(), f"{label}: -inf pattern"
    err = np.abs(g[~inf] - r[~inf])
    bound = 1e-5 * M[~inf] + 1e-30
    worst = float((err / bound).max()) if err.size else 0.0
    say(f"  {label}: worst error / bound = {worst:.3f}")
    assert worst <= 1.0, label


def _gpu_logits(case):
    out = sap.indexer_logits_packed(dev(case.q), dev(case.w), dev(case.key_pool), dev(case.page_table), case.page,
                                    case.N, n_keys=dev(case.n_keys))
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("B,N,n_keys", [(1, 8192, None), (4, 2000, [2000, 1999, 1000, 1]), (2, 333, [333, 0]),
                                        (3, 4096, [4096, 2500, 63]), (2, 128, [0, 65])])
def test_indexer_logits_small(B, N, n_keys):
    need_gpu()
    case = W.indexer_case(B=B, N=N, seed=W.SEED_BASE + 500 + B + N, n_keys=n_keys)
    got = _gpu_logits(case)
    ref = oracle.case_indexer(case)
    _check_logits(got, ref, _magnitude(case), f"indexer B{B} N{N}")


def test_indexer_logits_context_131072_b1():
    need_gpu()
    case = W.indexer_case(B=1, N=131072)
    got = _gpu_logits(case)
    ref = oracle.case_indexer(case)
    _check_logits(got, ref, _magnitude(case), "indexer B1 N131072")


def test_indexer_extreme_scales_and_strides():
    # scale bytes across the whole range (the table test covers the decode;
    # here the rows go through the kernel), rows with extra words, no page table
    need_gpu()
    g = W.make_generator(W.SEED_BASE + 520)
    B, N = 2, 256
    rows = W.fp4_key_rows(B * N, g, exp_lo=100, exp_hi=150, row_words=20)
    q = (torch.randn((B, 32, 128), generator=g)).to(torch.bfloat16)
    w = torch.rand((B, 32), generator=g)
    got = sap.indexer_logits_packed(dev(q), dev(w), dev(rows), None, 64, N)
    torch.cuda.synchronize()
    ref = oracle.indexer_logits(q, w, rows, None, 64, None, N)
    k = np.abs(oracle.fp4_rows_decode(rows)).reshape(B, N, 128)
    M = np.stack([(np.abs(q[b].double().numpy()) @ k[b].T * w[b].double().numpy()[:, None]).sum(0)
                  for b in range(B)])
    _check_logits(got, ref, M, "indexer strided rows, no page table")
    # fewer than 32 heads
    got = sap.indexer_logits_packed(dev(q[:, :7].contiguous()), dev(w[:, :7].contiguous()), dev(rows), None, 64, N)
    torch.cuda.synchronize()
    ref = oracle.indexer_logits(q[:, :7], w[:, :7], rows, None, 64, None, N)
    _check_logits(got, ref, M, "indexer 7 heads")


@pytest.mark.parametrize("B,N,k", [(1, 131072, 512), (4, 131072, 512), (1, 8192, 512), (3, 4096, 512),
                                   (2, 1000, 512), (2, 70000, 2048), (1, 100000, 1), (2, 50000, 300),
                                   (2, 12000, 4096), (2, 16384, 512), (2, 16385, 512), (1, 5000, 4096),
                                   (1, 200000, 4096)])
def test_topk_same_logits_bit_exact(B, N, k):
    need_gpu()
    g = torch.Generator().manual_seed(N + k + B)
    x = torch.randn((B, N), generator=g)
    if B > 1:
        x[1] = torch.round(x[1] * 3) / 3             # heavy ties
    x[0, ::11] = float("-inf")
    nv = torch.tensor([N - (b * 977) % max(N, 1) for b in range(B)], dtype=torch.int32).clamp(min=0)
    got = sap.topk_select(dev(x), k, n_valid=dev(nv))
    torch.cuda.synchronize()
    ref = oracle.topk(x, k, nv)
    assert torch.equal(got.cpu(), ref), f"B{B} N{N} k{k}"


def test_topk_signed_zero_ties():
    """-0.0 and +0.0 are equal values: when the k-th largest value is zero,
    zeros of either sign tie and go to the lower index (as in the oracle's
    value order), in the one-launch and the two-launch paths."""
    need_gpu()
    for N, k in ((8192, 512), (4000, 100), (40000, 512)):
        g = torch.Generator().manual_seed(N + 3)
        x = torch.full((2, N), -1.0)
        pos = torch.randperm(N, generator=g)
        x[0, pos[:k // 2]] = 1.0
        zeros = pos[k // 2:k // 2 + 3 * k]
        x[0, zeros] = torch.where(torch.rand(zeros.numel(), generator=g) < 0.5, -0.0, 0.0)
        x[1] = torch.where(torch.rand(N, generator=g) < 0.5, -0.0, 0.0)
        assert (torch.signbit(x[0]) & (x[0] == 0)).any()
        got = sap.topk_select(dev(x), k)
        torch.cuda.synchronize()
        assert torch.equal(got.cpu(), oracle.topk(x, k)), f"N{N} k{k}"


def test_topk_fallback_paths():
    """Long rows whose strided sample misleads the filter threshold: keys at
    the sampled positions dominate (too few keys pass), or one chunk holds
    more passing keys than its slot.  Both must still give the exact set."""
    need_gpu()
    N, k = 131072, 512
    g = torch.Generator().manual_seed(77)
    x = torch.randn((2, N), generator=g)
    pos = (torch.arange(4096, dtype=torch.int64) * N) // 4096          # the sampled positions
    x[0, pos] = 100.0 + torch.rand(4096, generator=g)                  # sample top >> everything else
    x[1, :4096] = 50.0                                                 # chunk 0 passes whole: slot overflow
    got = sap.topk_select(dev(x), k)
    torch.cuda.synchronize()
    assert torch.equal(got.cpu(), oracle.topk(x, k))


def test_topk_on_indexer_logits():
    need_gpu()
    case = W.indexer_case(B=4, N=131072, seed=W.SEED_BASE + 530)
    logits = _gpu_logits(case)
    got = sap.topk_select(logits, 512)
    torch.cuda.synchronize()
    assert torch.equal(got.cpu(), oracle.topk(logits.cpu(), 512))


def test_chain_indexer_topk_attention_small():
    """Small-scale chain: 256 query tokens, 64 compressed entries with packed
    128-d index keys, 32 index heads -> top-32 -> index build -> attention
    with 8 heads, head_dim 64, window 16, r = 4."""
    need_gpu()
    case = W.tiny_case()
    g = W.make_generator(W.SEED_BASE + 540)
    T, n_c = case.T, case.cmp_pool.shape[0]
    keys = W.fp4_key_rows(n_c, g)                                   # index key of each compressed row
    qi = torch.randn((T, 32, 128), generator=g).to(torch.bfloat16)
    wi = torch.rand((T, 32), generator=g)
    n_vis = torch.div(case.pos.to(torch.int64) + 4, 4, rounding_mode="floor").to(torch.int32)
    # every token scores the same key pool (page-table row stride 0), up to its causal count
    pt = case.cmp_pt.expand(T, -1)
    logits = sap.indexer_logits_packed(dev(qi), dev(wi), dev(keys), dev(pt), case.page, n_c, n_keys=dev(n_vis))
    torch.cuda.synchronize()
    ref_logits = oracle.indexer_logits(qi, wi, keys, pt, case.page, n_vis, n_c)
    prow = (case.cmp_pt[0].to(torch.int64).repeat_interleave(case.page) * case.page
            + torch.arange(case.page).repeat(case.cmp_pt.shape[1]))[:n_c]
    k = np.abs(oracle.fp4_rows_decode(keys[prow]))
    M = (np.abs(qi.double().numpy()) @ k.T * np.abs(wi.double().numpy())[:, :, None]).sum(1)
    _check_logits(logits, ref_logits, M, "chain logits")
    sel = sap.topk_select(logits, 32)
    torch.cuda.synchronize()
    assert torch.equal(sel.cpu(), oracle.topk(logits.cpu(), 32))
    # logical entries chosen by the indexer become the compressed columns
    case.cmp_logical = sel.cpu()
    q = case.q.to(torch.bfloat16)
    wp, cp = case.win_pool.to(torch.bfloat16), case.cmp_pool.to(torch.bfloat16)
    idx = sap.build_sparse_idx(dev(case.pos), dev(case.seq), case.n_win, dev(case.win_pt), case.page,
                               dev(case.cmp_logical), dev(case.cmp_pt))
    out = sap.sparse_attn_paged(dev(q), dev(wp), dev(cp), idx, case.n_win, case.sm_scale)
    torch.cuda.synchronize()
    oidx = oracle.case_idx(case)
    assert torch.equal(idx.cpu(), oidx)
    ref = oracle.sparse_attn(q, wp, cp, oidx, case.n_win, case.sm_scale)
    assert_attn_close(out, ref, "chain")


def _tk_idx_inputs(T, N, n_win, nv, seed, page=64):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(T, N, generator=g) * 8).round() / 8          # many ties
    x[torch.rand(T, N, generator=g) < 0.01] = -float("inf")
    x[torch.rand(T, N, generator=g) < 0.002] = float("nan")
    S = max(1, (T + 1) // 2)
    seq = (torch.arange(T) % S).to(torch.int32)
    pos = torch.randint(0, 3 * n_win + 1, (T,), generator=g).to(torch.int32)   # some windows start below 0
    pos[0] = 5000
    wpages = (int(pos.max()) + page) // page
    win_pt = torch.randperm(S * wpages, generator=g).to(torch.int32).view(S, wpages)
    cpages = (N + page - 1) // page
    cmp_pt = torch.randperm(S * cpages, generator=g).to(torch.int32).view(S, cpages)
    n_valid = None if nv is None else torch.tensor(nv, dtype=torch.int32)
    return x, seq, pos, win_pt, cmp_pt, n_valid


@pytest.mark.parametrize("T,N,k,n_win,nv", [
    (1, 8192, 512, 128, None),             # the decode step's selection
    (8, 8192, 512, 128, None),
    (3, 2000, 512, 128, [2000, 300, 0]),   # fewer candidates than k, an empty row
    (2, 40000, 512, 64, None),             # filter + select launches
    (2, 5000, 100, 16, [4999, 17]),
])
def test_topk_sparse_idx_matches_oracle(T, N, k, n_win, nv):
    """The fused selection + index build against the oracle's top-k followed
    by its index build, and against the two GPU calls, bit for bit."""
    need_gpu()
    x, seq, pos, win_pt, cmp_pt, n_valid = _tk_idx_inputs(T, N, n_win, nv, seed=600 + T + N)
    sel_ref = oracle.topk(x, k, n_valid)
    idx_ref = oracle.build_idx(pos, seq, n_win, win_pt, 64, sel_ref, k, cmp_pt)
    got = sap.topk_sparse_idx(dev(x), k, dev(pos), dev(seq), n_win, dev(win_pt), dev(cmp_pt), 64,
                              n_valid=dev(n_valid))
    torch.cuda.synchronize()
    assert torch.equal(got.cpu(), idx_ref), f"T{T} N{N} k{k}: fused index rows differ from the oracle"
    sel = sap.topk_select(dev(x), k, n_valid=dev(n_valid))
    two = sap.build_sparse_idx(dev(pos), dev(seq), n_win, dev(win_pt), 64, sel, dev(cmp_pt))
    torch.cuda.synchronize()
    assert torch.equal(got, two)
    say(f"  topk_sparse_idx T{T} N{N} k{k} n_win{n_win}: identical to oracle and to the two calls")


@pytest.mark.parametrize("T,N,k,page", [
    (2, 8192, 512, 1),       # 8192 page-table entries: more than the LDS stage holds, looked up in memory
    (2, 8192, 512, 3),       # pages of 3 entries: 2731 entries, staged, mapped by division
    (2, 16384, 512, 16),     # 16 keys per thread
    (3, 12000, 2048, 128),   # rows shorter than 16 keys per thread, k = 2048
    (1, 4097, 512, 1),       # 4097 entries: one past the LDS stage
])
def test_topk_sparse_idx_page_sizes(T, N, k, page):
    """The fused selection maps positions to rows through the page table,
    staged in LDS when it fits, read from memory otherwise, for power-of-two
    and other page sizes."""
    need_gpu()
    x, seq, pos, win_pt, cmp_pt, n_valid = _tk_idx_inputs(T, N, 128, None, seed=700 + N + page, page=page)
    sel_ref = oracle.topk(x, k, n_valid)
    idx_ref = oracle.build_idx(pos, seq, 128, win_pt, page, sel_ref, k, cmp_pt)
    got = sap.topk_sparse_idx(dev(x), k, dev(pos), dev(seq), 128, dev(win_pt), dev(cmp_pt), page)
    torch.cuda.synchronize()
    assert torch.equal(got.cpu(), idx_ref), f"T{T} N{N} k{k} page{page}"


@pytest.mark.parametrize("kind", ["negative", "wide", "mixed_sign", "one_value"])
def test_topk_value_distributions(kind):
    """Rows that are all negative, span the whole float range, mix signs
    around zero, or hold one value: the radix passes start at different bits
    and the tie bin is taken whole or in part."""
    need_gpu()
    g = torch.Generator().manual_seed(800 + len(kind))
    N = 8192
    if kind == "negative":
        x = -torch.rand((4, N), generator=g) * 10 - 0.5
    elif kind == "wide":
        x = torch.randn((4, N), generator=g) * torch.pow(2.0, torch.randint(-120, 120, (4, N), generator=g).double()).float()
    elif kind == "mixed_sign":
        x = (torch.randn((4, N), generator=g) * 1e-3).to(torch.bfloat16).float()
    else:
        x = torch.full((4, N), 0.75)
        x[:, ::97] = 2.0
    for k in (1, 512, 4096):
        got = sap.topk_select(dev(x), k)
        torch.cuda.synchronize()
        assert torch.equal(got.cpu(), oracle.topk(x, k)), f"{kind} k{k}"


def test_topk_repeated_launches_identical():
    """The decode step's selection shape (8192 logits, top-512, fused index
    build) launched 50 times in a row on the same inputs gives the same rows
    as the oracle every time."""
    need_gpu()
    x, seq, pos, win_pt, cmp_pt, n_valid = _tk_idx_inputs(8, 8192, 128, None, seed=993)
    idx_ref = oracle.build_idx(pos, seq, 128, win_pt, 64, oracle.topk(x, 512), 512, cmp_pt)
    xd, posd, seqd, wd, cd = dev(x), dev(pos), dev(seq), dev(win_pt), dev(cmp_pt)
    outs = [sap.topk_sparse_idx(xd, 512, posd, seqd, 128, wd, cd, 64) for _ in range(50)]
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert torch.equal(o.cpu(), idx_ref), f"launch {i}"


def test_determinism_sha256_topk():
    """Three runs of the top-k (one-launch and two-launch paths, and the
    selection fused with the index build) give identical bytes."""
    need_gpu()
    g = torch.Generator().manual_seed(991)
    for N in (8192, 131072):
        x = dev((torch.randn(4, N, generator=g) * 4).round() / 4)
        h = set()
        for _ in range(3):
            out = sap.topk_select(x, 512)
            torch.cuda.synchronize()
            h.add(hashlib.sha256(out.cpu().numpy().tobytes()).hexdigest())
        assert len(h) == 1, N
    x, seq, pos, win_pt, cmp_pt, n_valid = _tk_idx_inputs(8, 8192, 128, None, seed=992)
    h = set()
    for _ in range(3):
        got = sap.topk_sparse_idx(dev(x), 512, dev(pos), dev(seq), 128, dev(win_pt), dev(cmp_pt), 64)
        torch.cuda.synchronize()
        h.add(hashlib.sha256(got.cpu().numpy().tobytes()).hexdigest())
    assert len(h) == 1
