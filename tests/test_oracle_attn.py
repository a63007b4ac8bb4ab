"""Pins of the oracle's index build and sparse attention against sources
other than itself: a hand-worked example, torch's fp64 dense softmax
attention (causal, and over both pools), closed-form special cases, column
permutation invariance and a masked brute force on the small fp32 case.

Sparse attention over a paged KV cache is defined on the pages by its call
path and shapes ('perf(kernel): keep 16-byte kv loads in dsv4 sparse
attention and unroll gated pool', Call paths / Changes / Kernel time); the
fp8 dequant identity is in 'Perf/kv fp8 read path' (What this changes).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_index_build_worked_example():
    g = _load("index_build_worked_example.json")
    idx = oracle.build_idx(torch.tensor(g["pos"]), torch.tensor(g["seq"]), g["n_win"],
                           torch.tensor(g["win_pt"]), g["page"], torch.tensor(g["cmp_logical"]),
                           3, torch.tensor(g["cmp_pt"]))
    assert idx.tolist() == g["expected"]


def test_index_build_round_trip_prefill():
    case = W.prefill_case(T=300, start=50, ratio=4, H=1, D=64, n_win=128, topk=64, page=16, seed=11)
    idx = oracle.case_idx(case)
    inv_w = {int(p): l for l, p in enumerate(case.win_pt[0].tolist())}
    inv_c = {int(p): l for l, p in enumerate(case.cmp_pt[0].tolist())}
    for t in range(case.T):
        pos = int(case.pos[t])
        for j in range(case.n_win):
            r = int(idx[t, j])
            p = pos - (case.n_win - 1) + j
            if p < 0:
                assert r == -1
            else:
                assert inv_w[r // case.page] * case.page + r % case.page == p
        for j in range(case.n_cmp):
            r = int(idx[t, case.n_win + j])
            L = int(case.cmp_logical[t, j])
            assert (r == -1) == (L < 0)
            if L >= 0:
                assert inv_c[r // case.page] * case.page + r % case.page == L
                assert L < math.ceil((pos + 1) / 4)


def test_attn_worked_example():
    g = _load("attn_worked_example.json")
    win = torch.zeros((g["win_pool_rows"], g["D"]))
    cmp = torch.zeros((g["cmp_pool_rows"], g["D"]))
    for r, v in g["win_rows"].items():
        win[int(r)] = torch.tensor(v)
    for r, v in g["cmp_rows"].items():
        cmp[int(r)] = torch.tensor(v)
    q = torch.tensor(g["q"], dtype=torch.float32).view(1, 2, g["D"])
    out = oracle.sparse_attn(q, win, cmp, torch.tensor([g["idx"]], dtype=torch.int32), g["n_win"], 1.0)
    np.testing.assert_allclose(out[0].numpy(), np.array(g["expected"]), rtol=0, atol=1e-7)


def _dense_causal_ref(q, keys, sm_scale):
    """torch fp64: causal softmax(q k^T * scale) k for q [T,H,D], keys [T,D]."""
    q = q.to(torch.float64)
    k = keys.to(torch.float64)
    T = q.shape[0]
    s = torch.einsum("thd,sd->hts", q, k) * sm_scale
    mask = torch.ones(T, T, dtype=torch.bool).tril()
    s = s.masked_fill(~mask, float("-inf"))
    p = torch.softmax(s, dim=-1)
    return torch.einsum("hts,sd->thd", p, k)


def test_dense_reduction_window_covers_prefix():
    # ratio 0 and a window of at least T tokens: every token attends to all
    # earlier positions, which is causal dense attention.
    T, H, D = 96, 4, 32
    case = W.prefill_case(T=T, start=0, ratio=0, H=H, D=D, n_win=T, page=16, seed=12, kv_dtype="f32")
    raw = torch.stack([case.win_pool[W.pool_row(case.win_pt, 0, p, 16)] for p in range(T)])
    out = oracle.case_attn(case)
    ref = _dense_causal_ref(case.q, raw, case.sm_scale)
    np.testing.assert_allclose(out.numpy(), ref.numpy(), rtol=1e-10, atol=1e-12)


def test_dense_reduction_all_rows_of_both_pools():
    g = torch.Generator().manual_seed(3)
    T, H, D, Nw, Nc = 5, 3, 16, 24, 10
    q = torch.randn(T, H, D, generator=g).to(torch.bfloat16)
    win = torch.randn(Nw, D, generator=g).to(torch.bfloat16)
    cmp = torch.randn(Nc, D, generator=g).to(torch.bfloat16)
    idx = torch.cat([torch.arange(Nw), torch.arange(Nc)]).to(torch.int32).repeat(T, 1)
    out = oracle.sparse_attn(q, win, cmp, idx, Nw, 0.37)
    kv = torch.cat([win, cmp]).to(torch.float64)
    s = torch.einsum("thd,cd->thc", q.to(torch.float64), kv) * 0.37
    ref = torch.einsum("thc,cd->thd", torch.softmax(s, -1), kv)
    np.testing.assert_allclose(out.numpy(), ref.numpy(), rtol=1e-10, atol=1e-12)


def test_uniform_scores_give_mean_and_special_cases():
    case = W.decode_case(B=2, pos=700, ratio=4, H=4, D=64, topk=40, seed=13)
    idx = oracle.case_idx(case)
    zero_q = torch.zeros_like(case.q)
    out = oracle.case_attn(case, idx=idx, q=zero_q)
    for t in range(case.T):
        rows = []
        for c in range(idx.shape[1]):
            r = int(idx[t, c])
            if r >= 0:
                pool = case.win_pool if c < case.n_win else case.cmp_pool
                rows.append(pool[r].to(torch.float64))
        mean = torch.stack(rows).mean(0)
        for h in range(case.H):
            np.testing.assert_allclose(out[t, h].numpy(), mean.numpy(), rtol=1e-12, atol=1e-12)
    # a single valid column returns that row whatever q is
    one = torch.full_like(idx, -1)
    one[:, case.n_win + 3] = idx[:, case.n_win + 3]
    out1 = oracle.case_attn(case, idx=one)
    for t in range(case.T):
        row = case.cmp_pool[int(one[t, case.n_win + 3])].to(torch.float64)
        for h in range(case.H):
            np.testing.assert_array_equal(out1[t, h].numpy(), row.numpy())
    # identical rows everywhere return that row
    same = case.win_pool.clone()
    same[:] = case.win_pool[0]
    samec = case.cmp_pool.clone()
    samec[:] = case.win_pool[0]
    out2 = oracle.case_attn(case, idx=idx, win_pool=same, cmp_pool=samec)
    np.testing.assert_allclose(out2.numpy(), np.broadcast_to(same[0].double().numpy(), out2.shape),
                               rtol=1e-12, atol=1e-12)
    # no valid column at all gives zeros
    out3 = oracle.case_attn(case, idx=torch.full_like(idx, -1))
    assert (out3 == 0).all()


def test_column_permutation_invariance():
    case = W.decode_case(B=3, pos=500, ratio=4, H=8, D=64, topk=64, seed=14)
    idx = oracle.case_idx(case)
    g = torch.Generator().manual_seed(5)
    pw = torch.randperm(case.n_win, generator=g)
    pc = torch.randperm(case.n_cmp, generator=g) + case.n_win
    idx_p = idx[:, torch.cat([pw, pc])].contiguous()
    a = oracle.case_attn(case, idx=idx)
    b = oracle.case_attn(case, idx=idx_p)
    np.testing.assert_allclose(a.numpy(), b.numpy(), rtol=1e-12, atol=1e-14)
    # moving a column to the other pool's range changes which pool it reads
    bad = idx.clone()
    bad[:, 0], bad[:, case.n_win] = idx[:, case.n_win], idx[:, 0]
    c = oracle.case_attn(case, idx=bad)
    assert not np.allclose(a.numpy(), c.numpy())


def test_tiny_case_matches_masked_brute_force():
    case = W.tiny_case()
    idx = oracle.case_idx(case)
    out = oracle.case_attn(case, idx=idx)
    # brute force: every row of both pools, -inf where the token did not select it
    kv = torch.cat([case.win_pool, case.cmp_pool]).to(torch.float64)
    Nw = case.win_pool.shape[0]
    T = case.T
    sel = torch.zeros(T, kv.shape[0], dtype=torch.bool)
    for t in range(T):
        for c in range(idx.shape[1]):
            r = int(idx[t, c])
            if r >= 0:
                sel[t, r if c < case.n_win else Nw + r] = True
    s = torch.einsum("thd,nd->thn", case.q.to(torch.float64), kv) * case.sm_scale
    s = s.masked_fill(~sel.unsqueeze(1), float("-inf"))
    ref = torch.einsum("thn,nd->thd", torch.softmax(s, -1), kv)
    np.testing.assert_allclose(out.numpy(), ref.numpy(), rtol=1e-10, atol=1e-12)
    # the selected set is the causal window plus the chosen compressed entries
    raw, comp = case.meta["raw"], case.meta["comp"]
    t = 200
    keys = [raw[p] for p in range(t - case.n_win + 1, t + 1)]
    keys += [comp[int(L)] for L in case.cmp_logical[t] if L >= 0]
    kk = torch.stack(keys).to(torch.float64)
    pr = torch.softmax(case.q[t].double() @ kk.T * case.sm_scale, -1) @ kk
    np.testing.assert_allclose(out[t].numpy(), pr.numpy(), rtol=1e-10, atol=1e-12)


def test_e4m3_pools_match_torch_dequant_dense():
    case = W.decode_case(B=2, pos=300, ratio=4, H=4, D=64, topk=32, kv_dtype="e4m3", seed=15)
    idx = oracle.case_idx(case)
    out = oracle.case_attn(case, idx=idx)
    for t in range(case.T):
        keys = []
        for c in range(idx.shape[1]):
            r = int(idx[t, c])
            if r < 0:
                continue
            pool, sc = (case.win_pool, case.win_scale) if c < case.n_win else (case.cmp_pool, case.cmp_scale)
            keys.append(pool[r].view(torch.float8_e4m3fn).to(torch.float64) * float(sc[r]))
        kk = torch.stack(keys)
        ref = torch.softmax(case.q[t].double() @ kk.T * case.sm_scale, -1) @ kk
        np.testing.assert_allclose(out[t].numpy(), ref.numpy(), rtol=1e-10, atol=1e-9)


# ------------------------------------------------------------- gated pool

def test_gated_pool_softmax_reference():
    """Against torch's softmax over R (an independent route), bf16 x and
    fp32 gates, odd R and D."""
    for B, R, D in ((2, 7, 37), (1, 129, 64), (3, 1, 10)):
        case = W.gated_pool_case(B=B, R=R, D=D, seed=W.SEED_BASE + 900 + R)
        out = oracle.gated_pool(case.x, case.gate)
        p = torch.softmax(case.gate.to(torch.float64), dim=1)
        ref = (p * case.x.to(torch.float64)).sum(1)
        np.testing.assert_allclose(out.numpy(), ref.numpy(), rtol=1e-12, atol=1e-13)


def test_gated_pool_closed_forms():
    g = torch.Generator().manual_seed(11)
    x = torch.randn(2, 5, 9, generator=g, dtype=torch.float64)
    # R = 1: the row itself
    assert torch.equal(oracle.gated_pool(x[:, :1], torch.randn(2, 1, 9, generator=g, dtype=torch.float64)), x[:, 0])
    # equal gates: the mean over R
    gate = torch.full((2, 5, 9), 0.37, dtype=torch.float64)
    np.testing.assert_allclose(oracle.gated_pool(x, gate).numpy(), x.mean(1).numpy(), rtol=1e-14, atol=1e-15)
    # one gate far above the rest: exactly that row
    gate = torch.zeros(2, 5, 9, dtype=torch.float64)
    gate[:, 3] = 2000.0
    assert torch.equal(oracle.gated_pool(x, gate), x[:, 3])
    # -inf gates drop their rows; an all -inf column pools to 0
    gate = torch.randn(2, 5, 9, generator=g, dtype=torch.float64)
    gm = gate.clone()
    gm[:, 1] = -math.inf
    keep = [0, 2, 3, 4]
    np.testing.assert_allclose(oracle.gated_pool(x, gm).numpy(), oracle.gated_pool(x[:, keep], gate[:, keep]).numpy(),
                               rtol=1e-14, atol=1e-15)
    gm[:, :, 4] = -math.inf
    assert (oracle.gated_pool(x, gm)[:, 4] == 0).all()


def test_gated_pool_invariances():
    """A per-column shift of the gates and a permutation of the R rows leave
    the pooled row unchanged; the result lies within each column's range."""
    case = W.gated_pool_case(B=2, R=16, D=33, seed=W.SEED_BASE + 910)
    out = oracle.gated_pool(case.x, case.gate)
    shift = torch.randn(2, 1, 33, generator=torch.Generator().manual_seed(3), dtype=torch.float64) * 50
    np.testing.assert_allclose(oracle.gated_pool(case.x, case.gate.to(torch.float64) + shift).numpy(), out.numpy(),
                               rtol=1e-11, atol=1e-12)
    perm = torch.randperm(16, generator=torch.Generator().manual_seed(4))
    np.testing.assert_allclose(oracle.gated_pool(case.x[:, perm], case.gate[:, perm]).numpy(), out.numpy(),
                               rtol=1e-13, atol=1e-14)
    xd = case.x.to(torch.float64)
    assert (out <= xd.max(1).values + 1e-12).all() and (out >= xd.min(1).values - 1e-12).all()
