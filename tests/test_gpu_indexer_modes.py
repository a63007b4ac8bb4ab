"""GPU parity of the indexer's candidate mode and prefill mode.

Both modes come from "perf(kernel): read dsv41 indexer key rows as int32
words" (Call path: full mode on the Full layers, candidate mode on the
Reindex layers, in prefill and decode; Kernel time: candidate decode B1 / B4
at context 131072 with NC = 16384, candidate prefill of 128 tokens, full
prefill of 2k and 8k prompts from position 0, a 2k chunk at 128k context,
and 128-token bounded decoder variants at contexts 8k and 128k).

Logit tolerance as for full mode: below (128 + 32) * 2^-24 < 1e-5 of
M = sum_h |w_h| sum_d |q_hd k_d| per logit; the -inf pattern (no candidate,
a candidate or key beyond the token's visible count) must match exactly.
"""
import hashlib
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_paged_amd as sap
import workloads as W
from gpu_helpers import dev, need_gpu, say

pytestmark = pytest.mark.gpu


def _pool_rows(pt_row, n, page):
    n = torch.as_tensor(n, dtype=torch.int64)
    return pt_row.to(torch.int64)[n // page] * page + n % page


def _mag(q_t, w_t, keys_abs):
    """sum_h |w_h| sum_d |q_hd k_nd| for decoded |keys| [n, 128]."""
    q = np.abs(q_t.to(torch.float64).numpy())
    w = np.abs(w_t.to(torch.float64).numpy())
    return (q @ keys_abs.T * w[:, None]).sum(0)


def _check(got, ref, M, label):
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    inf = np.isinf(r)
    assert np.array_equal(np.isinf(g), inf) and (g[inf] < 0).all(), f"{label}: -inf pattern"
    err = np.abs(g[~inf] - r[~inf])
    bound = 1e-5 * M[~inf] + 1e-30
    worst = float((err / bound).max()) if err.size else 0.0
    say(f"  {label}: worst error / bound = {worst:.3f} over {err.size} logits")
    assert worst <= 1.0, label


# ---------------------------------------------------------------- candidates

def _cand_gpu(case, use_pt=True, n_keys=True, cand=None):
    out = sap.indexer_logits_candidates(dev(case.q), dev(case.w), dev(case.key_pool),
                                        dev(case.page_table) if use_pt else None, case.page,
                                        dev(case.cand if cand is None else cand),
                                        n_keys=dev(case.n_keys) if n_keys else None)
    torch.cuda.synchronize()
    return out.cpu()


def _cand_check(case, got, ref, label, cand=None, pt=True):
    cand = case.cand if cand is None else cand
    T, NC = cand.shape
    M = np.zeros((T, NC))
    for t in range(T):
        c = cand[t].to(torch.int64).clamp(min=0)
        rows = _pool_rows(case.page_table[t], c, case.page) if pt else c
        k = np.abs(oracle.fp4_rows_decode(case.key_pool[rows]))
        M[t] = _mag(case.q[t], case.w[t], k)
    _check(got.numpy(), ref.numpy(), M, label)


@pytest.mark.parametrize("T,n_ctx,NC,shared,sort", [
    (5, 3000, 700, False, False),       # ragged tail of the candidate list
    (3, 20000, 4160, False, True),      # several chunks of 8 tiles per wave
    (40, 1500, 1000, True, False),      # one sequence, stride-0 page table
    (1, 100, 64, False, True),          # fewer visible keys than candidates
])
def test_candidates_small(T, n_ctx, NC, shared, sort):
    need_gpu()
    case = W.indexer_cand_case(T=T, n_ctx=n_ctx, NC=NC, shared_seq=shared, sort=sort, extras=True,
                               seed=W.SEED_BASE + 600 + T + NC)
    say(f"candidates T{T} ctx{n_ctx} NC{NC} shared={shared}")
    got = _cand_gpu(case)
    ref = oracle.indexer_candidates(case.q, case.w, case.key_pool, case.page_table, case.page, case.cand,
                                    case.n_keys)
    _cand_check(case, got, ref, case.name)


def test_candidates_raw_rows_no_bound_and_hi20():
    """NULL page table (candidates are pool rows), no visible-count bound,
    20 index heads."""
    need_gpu()
    case = W.indexer_cand_case(T=4, n_ctx=2000, NC=300, Hi=20, sort=False, seed=W.SEED_BASE + 610)
    rows = torch.where(case.cand >= 0,
                       torch.stack([_pool_rows(case.page_table[t], case.cand[t].clamp(min=0).to(torch.int64),
                                               case.page) for t in range(4)]).to(torch.int32),
                       case.cand)
    got = _cand_gpu(case, use_pt=False, n_keys=False, cand=rows)
    ref = oracle.indexer_candidates(case.q, case.w, case.key_pool, None, case.page, rows, None)
    _cand_check(case, got, ref, "candidates raw rows Hi20", cand=rows, pt=False)


@pytest.mark.parametrize("T,shared", [(1, False), (4, False), (128, True)])
def test_candidates_nc16384_ctx131072(T, shared):
    """The page's candidate shapes: decode B1 / B4 at context 131072 and the
    128-token candidate prefill (positions 130944 ..), NC = 16384; every
    logit is checked."""
    need_gpu()
    case = W.indexer_cand_case(T=T, n_ctx=131072, NC=16384, shared_seq=shared, seed=W.SEED_BASE + 620 + T)
    say(f"candidates T{T} NC16384 shared={shared}")
    got = _cand_gpu(case)
    ref = oracle.indexer_candidates(case.q, case.w, case.key_pool, case.page_table, case.page, case.cand,
                                    case.n_keys)
    _cand_check(case, got, ref, case.name)


# ------------------------------------------------------------------- prefill

def _pf_gpu(case, n_keys=True, max_tokens=None):
    out = sap.indexer_logits_prefill(dev(case.q), dev(case.w), dev(case.key_pool), dev(case.page_table),
                                     case.page, dev(case.tok_start),
                                     case.max_tokens if max_tokens is None else max_tokens, case.N,
                                     n_keys=dev(case.n_keys) if n_keys else None)
    torch.cuda.synchronize()
    return out


def _pf_check(case, got, tokens, label, n_keys=None):
    """Compare the listed tokens' rows with the oracle and check the causal
    -inf pattern of every row."""
    nk = case.n_keys if n_keys is None else n_keys
    g = got.cpu()
    col = torch.arange(case.N).unsqueeze(0)
    vis = col < nk.to(torch.int64).unsqueeze(1)
    assert torch.isneginf(g[~vis]).all(), f"{label}: keys beyond the visible count must be -inf"
    assert torch.isfinite(g[vis]).all(), f"{label}: visible keys must be finite"
    ts = case.tok_start.to(torch.int64)
    seq = torch.repeat_interleave(torch.arange(ts.numel() - 1), ts[1:] - ts[:-1])
    tokens = torch.as_tensor(tokens, dtype=torch.int64)
    sel_q, sel_w, sel_nk = case.q[tokens], case.w[tokens], nk[tokens]
    pt_tok = case.page_table[seq[tokens]]
    ref = oracle.indexer_logits(sel_q, sel_w, case.key_pool, pt_tok, case.page, sel_nk, case.N)
    M = np.zeros((tokens.numel(), case.N))
    cache = {}
    for i, t in enumerate(tokens.tolist()):
        s = int(seq[t])
        if s not in cache:
            rows = _pool_rows(case.page_table[s], torch.arange(case.N), case.page)
            cache[s] = np.abs(oracle.fp4_rows_decode(case.key_pool[rows]))
        M[i] = _mag(case.q[t], case.w[t], cache[s])
    _check(g[tokens].numpy(), ref.numpy(), M, label)


@pytest.mark.parametrize("lengths,starts,ratio,page", [
    ((37, 100, 8), (0, 500, 129), 2, 64),     # three sequences, ragged token tiles
    ((300,), (700,), 1, 64),                  # one key per token, chunk boundary inside the keys
    ((64, 19), (0, 1000), 4, 16),             # pages of 16 rows (per-key page lookups)
])
def test_prefill_small(lengths, starts, ratio, page):
    need_gpu()
    case = W.indexer_prefill_case(lengths=lengths, starts=starts, ratio=ratio, page=page,
                                  seed=W.SEED_BASE + 630 + sum(lengths))
    say(f"prefill {case.name} N{case.N} page {page}")
    got = _pf_gpu(case)
    _pf_check(case, got, range(case.T), case.name)


def test_prefill_no_bound_hi24_extra_tokens():
    """NULL n_keys (every key visible), 24 heads, max_tokens above the longest
    sequence."""
    need_gpu()
    case = W.indexer_prefill_case(lengths=(50, 13), starts=(200, 300), ratio=2, Hi=24, seed=W.SEED_BASE + 640)
    got = _pf_gpu(case, n_keys=False, max_tokens=case.max_tokens + 20)
    _pf_check(case, got, range(case.T), "prefill no bound Hi24", n_keys=torch.full((case.T,), case.N))


@pytest.mark.parametrize("length,start,ratio,sample", [
    (8192, 0, 2, [0, 1, 2, 7, 8, 1000, 4095, 4096, 6001, 8190, 8191]),   # full prefill, 8k prompt
    (2048, 0, 2, [0, 5, 1023, 2047]),                                     # full prefill, 2k prompt
    (2048, 129024, 2, [0, 777, 2047]),                                    # 2k chunk at 128k context
    (128, 8064, 1, [0, 63, 127]),                                         # bounded decoder, ctx 8k
    (128, 130944, 1, [0, 127]),                                           # bounded decoder, ctx 128k
])
def test_prefill_page_shapes(length, start, ratio, sample):
    """The page's full-prefill shapes at full size: sampled rows against the
    oracle, the causal -inf pattern on every row."""
    need_gpu()
    case = W.indexer_prefill_case(lengths=(length,), starts=(start,), ratio=ratio,
                                  seed=W.SEED_BASE + 650 + length + ratio)
    say(f"prefill {case.name} N{case.N}")
    got = _pf_gpu(case)
    _pf_check(case, got, sample, case.name)


def test_determinism_sha256_indexer_modes():
    """Three runs of each indexer mode give identical bytes (sha256 of the
    full logits), as the pages check output hashes across builds."""
    need_gpu()
    runs = []
    case = W.indexer_case(B=4, N=131072, seed=W.SEED_BASE + 560)
    q, w, pool, pt = (dev(x) for x in (case.q, case.w, case.key_pool, case.page_table))
    runs.append(("full B4 N131072", lambda: sap.indexer_logits_packed(q, w, pool, pt, case.page, case.N)))
    cc = W.indexer_cand_case(T=4, n_ctx=131072, NC=16384, seed=W.SEED_BASE + 561)
    cq, cw, cpool, cpt, cand, cnk = (dev(x) for x in (cc.q, cc.w, cc.key_pool, cc.page_table, cc.cand, cc.n_keys))
    runs.append(("candidates T4", lambda: sap.indexer_logits_candidates(cq, cw, cpool, cpt, cc.page, cand, n_keys=cnk)))
    pc = W.indexer_prefill_case(lengths=(300, 200), starts=(1000, 0), ratio=2, seed=W.SEED_BASE + 562)
    pq, pw, ppool, ppt, pts, pnk = (dev(x) for x in (pc.q, pc.w, pc.key_pool, pc.page_table, pc.tok_start, pc.n_keys))
    runs.append(("prefill", lambda: sap.indexer_logits_prefill(pq, pw, ppool, ppt, pc.page, pts, pc.max_tokens, pc.N,
                                                               n_keys=pnk)))
    for name, fn in runs:
        h = set()
        for _ in range(3):
            out = fn()
            torch.cuda.synchronize()
            h.add(hashlib.sha256(out.cpu().numpy().tobytes()).hexdigest())
        assert len(h) == 1, name
        say(f"  {name}: identical sha256 over 3 runs")
