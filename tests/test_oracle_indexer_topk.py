"""Pins of the oracle's indexer logits and exact top-k selection.

The indexer reads fp4_e8m0_b32 packed key rows ('perf(kernel): read dsv41
indexer key rows as int32 words', Changes) and scores them with
sum_h w_h * max(0, q_h . k); the top-k keeps the k largest scores with ties
to the lower index.  The independent routes here are torch (keys decoded
through torch's float8_e8m0fnu dtype and the page's float32 e2m1
construction) and numpy's lexsort.
"""
import json
import math
import os

import numpy as np
import torch

import oracle
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _torch_decode_rows(rows: torch.Tensor) -> torch.Tensor:
    """[n, 17] int32 -> [n, 128] float64 via torch dtypes (independent of oracle.c)."""
    u = rows.to(torch.int64) & 0xFFFFFFFF
    shifts = torch.arange(8) * 4
    nib = ((u[:, :16].unsqueeze(-1) >> shifts) & 0xF).reshape(-1, 128)
    mag = (((nib & 7) << 22).to(torch.int32).view(torch.float32).to(torch.float64)) * 2.0 ** 126
    val = torch.where((nib & 8) != 0, -mag, mag)
    sbytes = ((u[:, 16:17] >> (torch.arange(4) * 8)) & 0xFF).to(torch.uint8)
    sc = sbytes.view(torch.float8_e8m0fnu).to(torch.float64)        # [n, 4]
    v = val * sc.repeat_interleave(32, dim=1)
    return v.to(torch.bfloat16).to(torch.float64)


def test_indexer_worked_example():
    g = _load("indexer_worked_example.json")
    row = torch.tensor([int(w, 16) - (1 << 32) if int(w, 16) >= 1 << 31 else int(w, 16)
                        for w in g["words"]], dtype=torch.int32)
    pool = torch.stack([row, row])
    q = torch.zeros(1, 3, 128)
    for h, d, v in g["q_nonzero"]:
        q[0, h, d] = v
    w = torch.tensor([g["w"]], dtype=torch.float32)
    out = oracle.indexer_logits(q.to(torch.bfloat16), w, pool, None, 64, torch.tensor([1]), 2)
    assert out[0, 0].item() == g["expected"]
    assert out[0, 1].item() == -math.inf


def test_indexer_matches_torch_reference():
    case = W.indexer_case(B=2, N=300, seed=21, n_keys=[300, 211])
    out = oracle.case_indexer(case)
    for b in range(2):
        rows = torch.stack([case.key_pool[W.pool_row(case.page_table, b, n)] for n in range(case.N)])
        k = _torch_decode_rows(rows)
        s = torch.relu(case.q[b].to(torch.float64) @ k.T)            # [Hi, N]
        ref = (case.w[b].to(torch.float64).unsqueeze(1) * s).sum(0)
        nk = int(case.n_keys[b])
        np.testing.assert_allclose(out[b, :nk].numpy(), ref[:nk].numpy(), rtol=1e-12, atol=1e-12)
        assert torch.isinf(out[b, nk:]).all() and (out[b, nk:] < 0).all()


def test_indexer_special_cases():
    case = W.indexer_case(B=1, N=128, seed=22)
    k = _torch_decode_rows(torch.stack([case.key_pool[W.pool_row(case.page_table, 0, n)]
                                        for n in range(case.N)]))
    for h in (0, 17, 31):
        w = torch.zeros(1, 32)
        w[0, h] = 1.0
        out = oracle.indexer_logits(case.q, w, case.key_pool, case.page_table, 64, None, case.N)
        ref = torch.relu(case.q[0, h].double() @ k.T)
        np.testing.assert_allclose(out[0].numpy(), ref.numpy(), rtol=1e-12, atol=1e-12)
    zero_pool = case.key_pool.clone()
    zero_pool[:, :16] = 0
    out = oracle.indexer_logits(case.q, case.w, zero_pool, case.page_table, 64, None, case.N)
    assert (out == 0).all()


def test_topk_worked_example():
    g = _load("topk_worked_example.json")
    x = torch.tensor([[float(v) for v in r] for r in g["x"]], dtype=torch.float32)
    assert oracle.topk(x, g["k"]).tolist() == g["expected"]


def test_topk_matches_lexsort_with_ties():
    g = torch.Generator().manual_seed(31)
    B, N, k = 4, 5000, 512
    x = torch.round(torch.randn(B, N, generator=g) * 4) / 4          # many ties
    x[1, ::7] = float("-inf")
    x[2, ::5] = float("nan")
    nv = torch.tensor([N, N, 4000, 300], dtype=torch.int32)
    out = oracle.topk(x, k, nv)
    for b in range(B):
        xs = x[b, :int(nv[b])].numpy()
        ok = ~np.isnan(xs) & ~(np.isinf(xs) & (xs < 0))
        ids = np.nonzero(ok)[0]
        order = np.lexsort((ids, -xs[ids]))
        sel = np.sort(ids[order[:k]])
        exp = np.full(k, -1)
        exp[:len(sel)] = sel
        assert out[b].tolist() == exp.tolist()


def test_topk_degenerate_rows():
    x = torch.full((3, 10), float("-inf"))
    x[1, 4] = 1.0
    x[2] = 2.0
    out = oracle.topk(x, 4)
    assert out[0].tolist() == [-1] * 4
    assert out[1].tolist() == [4, -1, -1, -1]
    assert out[2].tolist() == [0, 1, 2, 3]                          # all tied: lowest indices
    assert oracle.topk(x, 0).shape == (3, 0)


def _seq_keys(key_pool, pt_row, n):
    rows = torch.stack([key_pool[int(pt_row[j // W.PAGE]) * W.PAGE + j % W.PAGE] for j in range(n)])
    return _torch_decode_rows(rows)


def test_indexer_candidates_brute_force():
    """Candidate mode against torch, candidate by candidate, with planted -1,
    duplicate and beyond-visible entries and signed head weights."""
    case = W.indexer_cand_case(T=3, n_ctx=700, NC=96, seed=23, extras=True, sort=False)
    out = oracle.indexer_candidates(case.q, case.w, case.key_pool, case.page_table, case.page, case.cand,
                                    case.n_keys)
    assert out.shape == (3, 96)
    assert (case.w < 0).any()
    for t in range(3):
        k_all = _seq_keys(case.key_pool, case.page_table[t], int(case.n_keys[t]))
        s = torch.relu(case.q[t].to(torch.float64) @ k_all.T)            # [Hi, n]
        full = (case.w[t].to(torch.float64).unsqueeze(1) * s).sum(0)
        for c in range(96):
            n = int(case.cand[t, c])
            if n < 0 or n >= int(case.n_keys[t]):
                assert out[t, c].item() == -math.inf
            else:
                assert abs(out[t, c].item() - full[n].item()) <= 1e-12 * max(1.0, abs(full[n].item()))
    assert out[:, 1].eq(-math.inf).all() and out[:, 3].eq(-math.inf).all()
    assert torch.equal(out[:, 0], out[:, 2])


def test_indexer_candidates_gather_full_mode():
    """Listing every key in order reproduces full mode; a permuted list
    permutes the logits; NULL page table means candidates are pool rows."""
    case = W.indexer_case(B=2, N=200, seed=24, n_keys=[200, 150])
    full = oracle.case_indexer(case)
    cand = torch.arange(200, dtype=torch.int32).repeat(2, 1)
    out = oracle.indexer_candidates(case.q, case.w, case.key_pool, case.page_table, case.page, cand, case.n_keys)
    assert torch.equal(out, full)
    perm = torch.randperm(200, generator=torch.Generator().manual_seed(5)).to(torch.int32)
    outp = oracle.indexer_candidates(case.q, case.w, case.key_pool, case.page_table, case.page,
                                     perm.repeat(2, 1), case.n_keys)
    assert torch.equal(outp, full[:, perm.long()])
    rows = torch.tensor([[W.pool_row(case.page_table, b, n) for n in range(200)] for b in range(2)],
                        dtype=torch.int32)
    outr = oracle.indexer_candidates(case.q, case.w, case.key_pool, None, case.page, rows, case.n_keys + 10 ** 6)
    assert torch.equal(outr, torch.where(torch.isinf(full), outr, full))
    assert torch.equal(outr[0], full[0])


def test_indexer_prefill_causal_brute_force():
    """Prefill mode over two sequences against a dense torch product with the
    causal mask n < ceil((p+1)/r) applied afterwards."""
    case = W.indexer_prefill_case(lengths=(70, 33), starts=(0, 230), ratio=2, seed=25)
    out = oracle.indexer_prefill_logits(case.q, case.w, case.key_pool, case.page_table, case.page,
                                        case.tok_start, case.n_keys, case.N)
    assert out.shape == (103, case.N)
    for s in range(2):
        a, b = int(case.tok_start[s]), int(case.tok_start[s + 1])
        k = _seq_keys(case.key_pool, case.page_table[s], case.N)
        sc = torch.relu(torch.einsum("thd,nd->thn", case.q[a:b].to(torch.float64), k))
        ref = (case.w[a:b].to(torch.float64).unsqueeze(2) * sc).sum(1)      # [Ts, N]
        nk = ((case.pos[a:b].to(torch.int64) + 2) // 2)
        mask = torch.arange(case.N).unsqueeze(0) < nk.unsqueeze(1)
        assert torch.equal(nk.to(torch.int32), case.n_keys[a:b])
        np.testing.assert_allclose(out[a:b][mask].numpy(), ref[mask].numpy(), rtol=1e-12, atol=1e-12)
        assert out[a:b][~mask].eq(-math.inf).all()
