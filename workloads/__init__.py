"""Seeded synthetic inputs for top-k sparse attention over a paged KV cache.

This module is shared by both sides of every parity check: the CPU oracle
(``oracle/``) and the HIP library (``sparse_attention_paged_amd``).  It only
draws random numbers and lays them out -- pools of KV rows split into pages,
randomly permuted page tables, token positions, lists of compressed-pool
indices, packed indexer key rows -- and performs none of the method's own
arithmetic (no dot products, softmax, decoding or selection).

Every generator takes an integer seed and uses its own ``torch.Generator`` on
the CPU, so the oracle and the GPU path read byte-identical inputs.

Shapes follow the pages' workloads (FreeToken PR #633, "Kernel time": 64 query
heads sharing one KV head, head_dim 512, a 128-token window, top-k 512 over a
compressed pool with one entry per r tokens; FreeToken PR #634, "Kernel time":
32 index heads, head_dim 128, fp4_e8m0_b32 packed key rows).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

PAGE = 64          # rows per page in every paged pool
SEED_BASE = 20260000

__all__ = [
    "PAGE", "SEED_BASE", "AttnCase", "IndexerCase", "make_generator", "page_table",
    "random_unique_indices", "e4m3_finite_codes", "decode_case", "prefill_case",
    "tiny_case", "indexer_case", "fp4_key_rows", "pool_row",
]


def make_generator(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def page_table(n_seq: int, pages_per_seq: int, g: torch.Generator) -> torch.Tensor:
    """[n_seq, pages_per_seq] int32: disjoint physical pages per sequence, in a
    random permutation of the pool's pages."""
    perm = torch.randperm(n_seq * pages_per_seq, generator=g).to(torch.int32)
    return perm.view(n_seq, pages_per_seq).contiguous()


def pool_row(pt: torch.Tensor, seq: int, logical: int, page: int = PAGE) -> int:
    """Physical row of logical entry ``logical`` of sequence ``seq`` (layout
    helper used by generators and tests to place data; plain addressing)."""
    return int(pt[seq, logical // page]) * page + logical % page


def random_unique_indices(n_visible: torch.Tensor, k: int, g: torch.Generator,
                          chunk: int = 1024) -> torch.Tensor:
    """[T, k] int32.  Row t holds min(k, n_visible[t]) distinct integers drawn
    uniformly from [0, n_visible[t]) in random order, padded with -1."""
    T = int(n_visible.numel())
    out = torch.full((T, k), -1, dtype=torch.int32)
    if T == 0 or k == 0:
        return out
    for s in range(0, T, chunk):
        nv = n_visible[s:s + chunk].to(torch.int64)
        M = int(nv.max().item()) if nv.numel() else 0
        if M == 0:
            continue
        r = torch.rand((nv.numel(), M), generator=g)
        col = torch.arange(M).unsqueeze(0)
        r = torch.where(col < nv.unsqueeze(1), r, torch.full_like(r, 2.0))
        kk = min(k, M)
        vals, ind = torch.topk(r, kk, dim=1, largest=False, sorted=True)
        ind = torch.where(vals < 2.0, ind, torch.full_like(ind, -1))
        out[s:s + chunk, :kk] = ind.to(torch.int32)
    return out


def e4m3_finite_codes(shape, g: torch.Generator) -> torch.Tensor:
    """uint8 codes uniform over the 254 finite OCP E4M3 encodings (0x7F and
    0xFF, the two NaN encodings, are never drawn)."""
    r = torch.randint(0, 254, shape, generator=g, dtype=torch.int32)
    r = torch.where(r >= 0x7F, r + 1, r)       # skip 0x7F; 0xFF is never reached
    return r.to(torch.uint8)


def _normal_bf16(shape, g, scale=1.0):
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16)


@dataclass
class AttnCase:
    """Inputs of one sparse-attention workload (all CPU tensors).

    q          [T, H, D]  bf16 (or fp32 for the tiny oracle-only case)
    win_pool   [Nw, D]    bf16 / fp32 / uint8 (e4m3 codes) rows, paged
    cmp_pool   [Nc, D]    same dtype, or None when the compress ratio is 0
    win_scale, cmp_scale  [Nw], [Nc] fp32 per-row dequant scales (e4m3 only)
    pos, seq   [T] int32  position and sequence of each query token
    win_pt     [B, pages] int32 window page table (PAGE rows per page)
    cmp_pt     [B, pages] int32 compressed page table, or None
    cmp_logical[T, n_cmp] int32 selected logical compressed entries, -1 = pad
    """
    name: str
    q: torch.Tensor
    win_pool: torch.Tensor
    cmp_pool: Optional[torch.Tensor]
    pos: torch.Tensor
    seq: torch.Tensor
    win_pt: torch.Tensor
    cmp_pt: Optional[torch.Tensor]
    cmp_logical: torch.Tensor
    n_win: int
    n_cmp: int
    sm_scale: float
    ratio: int
    page: int = PAGE
    kv_dtype: str = "bf16"            # "bf16" | "f32" | "e4m3"
    win_scale: Optional[torch.Tensor] = None
    cmp_scale: Optional[torch.Tensor] = None
    meta: dict = field(default_factory=dict)

    @property
    def T(self):
        return int(self.q.shape[0])

    @property
    def H(self):
        return int(self.q.shape[1])

    @property
    def D(self):
        return int(self.q.shape[2])


def _n_visible_cmp(pos: torch.Tensor, ratio: int) -> torch.Tensor:
    # compressed entries visible to a token at position p: ceil((p+1)/r)
    return torch.div(pos.to(torch.int64) + ratio, ratio, rounding_mode="floor")


def _rows(n, D, g, kv_dtype, q_like_scale=1.0):
    if kv_dtype == "bf16":
        return _normal_bf16((n, D), g)
    if kv_dtype == "f32":
        return torch.randn((n, D), generator=g)
    if kv_dtype == "e4m3":
        return e4m3_finite_codes((n, D), g)
    raise ValueError(kv_dtype)


def _scales(n, g):
    # log-uniform in [2^-8, 2^2]
    return torch.exp2(torch.rand(n, generator=g) * 10.0 - 8.0).to(torch.float32)


def decode_case(B: int = 1, pos: int = 32767, ratio: int = 4, H: int = 64, D: int = 512,
                n_win: int = 128, topk: int = 512, kv_dtype: str = "bf16",
                seed: int = SEED_BASE + 2, q_scale: Optional[float] = None,
                page: int = PAGE) -> AttnCase:
    """B sequences, one query token each, all at position ``pos``.

    Window pool: every sequence owns ceil((pos+1)/page) pages of raw rows.
    Compressed pool (ratio > 0): ceil((pos+1)/ratio) entries per sequence,
    paged the same way; each token selects min(topk, that count) distinct
    random entries.  ratio == 0 means window only.
    """
    g = make_generator(seed)
    if q_scale is None:
        q_scale = 2.0 ** -7 if kv_dtype == "e4m3" else 1.0
    q = _normal_bf16((B, H, D), g, q_scale)
    n_pos = pos + 1
    wpages = math.ceil(n_pos / page)
    win_pt = page_table(B, wpages, g)
    win_pool = _rows(B * wpages * page, D, g, kv_dtype)
    win_scale = _scales(B * wpages * page, g) if kv_dtype == "e4m3" else None
    posv = torch.full((B,), pos, dtype=torch.int32)
    seqv = torch.arange(B, dtype=torch.int32)
    if ratio > 0:
        n_c = math.ceil(n_pos / ratio)
        cpages = math.ceil(n_c / page)
        cmp_pt = page_table(B, cpages, g)
        cmp_pool = _rows(B * cpages * page, D, g, kv_dtype)
        cmp_scale = _scales(B * cpages * page, g) if kv_dtype == "e4m3" else None
        n_cmp = min(topk, n_c)
        cmp_logical = random_unique_indices(_n_visible_cmp(posv, ratio), n_cmp, g)
    else:
        cmp_pt, cmp_pool, cmp_scale, n_cmp = None, None, None, 0
        cmp_logical = torch.zeros((B, 0), dtype=torch.int32)
    return AttnCase(
        name=f"decode_b{B}_pos{pos}_r{ratio}_{kv_dtype}", q=q, win_pool=win_pool,
        cmp_pool=cmp_pool, pos=posv, seq=seqv, win_pt=win_pt, cmp_pt=cmp_pt,
        cmp_logical=cmp_logical, n_win=n_win, n_cmp=n_cmp, sm_scale=1.0 / math.sqrt(D),
        ratio=ratio, page=page, kv_dtype=kv_dtype, win_scale=win_scale, cmp_scale=cmp_scale)


def prefill_case(T: int = 8192, start: int = 0, ratio: int = 4, H: int = 64, D: int = 512,
                 n_win: int = 128, topk: int = 512, kv_dtype: str = "bf16",
                 seed: int = SEED_BASE + 3, page: int = PAGE, q_scale: float = 1.0) -> AttnCase:
    """One sequence; T query tokens at positions start .. start+T-1.  Token at
    position p sees the causal window p-n_win+1 .. p and min(topk,
    ceil((p+1)/ratio)) distinct random compressed entries below
    ceil((p+1)/ratio)."""
    g = make_generator(seed)
    q = _normal_bf16((T, H, D), g, q_scale) if kv_dtype != "f32" else torch.randn((T, H, D), generator=g) * q_scale
    n_pos = start + T
    wpages = max(1, math.ceil(n_pos / page))
    win_pt = page_table(1, wpages, g)
    win_pool = _rows(wpages * page, D, g, kv_dtype)
    win_scale = _scales(wpages * page, g) if kv_dtype == "e4m3" else None
    posv = torch.arange(start, start + T, dtype=torch.int32)
    seqv = torch.zeros(T, dtype=torch.int32)
    if ratio > 0:
        n_c = max(1, math.ceil(n_pos / ratio))
        cpages = math.ceil(n_c / page)
        cmp_pt = page_table(1, cpages, g)
        cmp_pool = _rows(cpages * page, D, g, kv_dtype)
        cmp_scale = _scales(cpages * page, g) if kv_dtype == "e4m3" else None
        n_cmp = topk
        cmp_logical = random_unique_indices(_n_visible_cmp(posv, ratio), n_cmp, g)
    else:
        cmp_pt, cmp_pool, cmp_scale, n_cmp = None, None, None, 0
        cmp_logical = torch.zeros((T, 0), dtype=torch.int32)
    return AttnCase(
        name=f"prefill_s{T}_at{start}_r{ratio}_{kv_dtype}", q=q, win_pool=win_pool,
        cmp_pool=cmp_pool, pos=posv, seq=seqv, win_pt=win_pt, cmp_pt=cmp_pt,
        cmp_logical=cmp_logical, n_win=n_win, n_cmp=n_cmp, sm_scale=1.0 / math.sqrt(D),
        ratio=ratio, page=page, kv_dtype=kv_dtype, win_scale=win_scale, cmp_scale=cmp_scale)


def tiny_case(seed: int = SEED_BASE + 1, T: int = 256, H: int = 8, D: int = 64, n_win: int = 16,
              ratio: int = 4, topk: int = 32, page: int = 16) -> AttnCase:
    """The small fp32 case: one sequence of T tokens, raw rows ~N(0,1), q ~N(0,1)/8.

    The compressed pool holds T/ratio entries, entry j being the mean of raw
    rows ratio*j .. ratio*j+ratio-1 (the pooled input the compressed pool
    stands for; this is input preparation, not part of the attention).  Both
    pools are paged with ``page`` rows per page.  sm_scale is 1.0 because q
    already carries the 1/sqrt(D) factor through its /8.
    """
    g = make_generator(seed)
    q = torch.randn((T, H, D), generator=g) / 8.0
    raw = torch.randn((T, D), generator=g)                     # logical order
    n_c = T // ratio
    comp = raw.view(n_c, ratio, D).mean(dim=1)                 # logical order
    wpages = math.ceil(T / page)
    cpages = math.ceil(n_c / page)
    win_pt = page_table(1, wpages, g)
    cmp_pt = page_table(1, cpages, g)
    win_pool = torch.zeros((wpages * page, D))
    cmp_pool = torch.zeros((cpages * page, D))
    for p in range(T):
        win_pool[pool_row(win_pt, 0, p, page)] = raw[p]
    for j in range(n_c):
        cmp_pool[pool_row(cmp_pt, 0, j, page)] = comp[j]
    posv = torch.arange(T, dtype=torch.int32)
    seqv = torch.zeros(T, dtype=torch.int32)
    cmp_logical = random_unique_indices(_n_visible_cmp(posv, ratio), topk, g)
    return AttnCase(
        name="tiny_s256_h8_d64", q=q, win_pool=win_pool, cmp_pool=cmp_pool, pos=posv, seq=seqv,
        win_pt=win_pt, cmp_pt=cmp_pt, cmp_logical=cmp_logical, n_win=n_win, n_cmp=topk,
        sm_scale=1.0, ratio=ratio, page=page, kv_dtype="f32",
        meta={"raw": raw, "comp": comp})


def fp4_key_rows(n_rows: int, g: torch.Generator, exp_lo: int = 120, exp_hi: int = 134,
                 row_words: int = 17) -> torch.Tensor:
    """[n_rows, row_words] int32 packed fp4_e8m0_b32 rows: words 0..15 hold 128
    uniform random 4-bit codes, word 16 holds four scale bytes drawn uniformly
    from the integers exp_lo..exp_hi; extra words (row_words > 17) are zero."""
    rows = torch.zeros((n_rows, row_words), dtype=torch.int64)
    rows[:, :16] = torch.randint(0, 2 ** 32, (n_rows, 16), generator=g, dtype=torch.int64)
    sb = torch.randint(exp_lo, exp_hi + 1, (n_rows, 4), generator=g, dtype=torch.int64)
    rows[:, 16] = sb[:, 0] | (sb[:, 1] << 8) | (sb[:, 2] << 16) | (sb[:, 3] << 24)
    rows = torch.where(rows >= 2 ** 31, rows - 2 ** 32, rows)
    return rows.to(torch.int32).contiguous()


@dataclass
class IndexerCase:
    """q [B, Hi, Dk] bf16, w [B, Hi] fp32, key_pool [B*pages*PAGE, 17] int32,
    page_table [B, pages] int32, n_keys [B] int32, N keys per sequence."""
    name: str
    q: torch.Tensor
    w: torch.Tensor
    key_pool: torch.Tensor
    page_table: torch.Tensor
    n_keys: torch.Tensor
    N: int
    page: int = PAGE


def indexer_case(B: int = 1, N: int = 131072, Hi: int = 32, Dk: int = 128,
                 seed: int = SEED_BASE + 5, n_keys: Optional[list] = None,
                 page: int = PAGE, exp_lo: int = 120, exp_hi: int = 134) -> IndexerCase:
    g = make_generator(seed)
    q = _normal_bf16((B, Hi, Dk), g)
    w = torch.rand((B, Hi), generator=g).to(torch.float32)
    pages = math.ceil(N / page)
    pt = page_table(B, pages, g)
    pool = fp4_key_rows(B * pages * page, g, exp_lo, exp_hi)
    nk = torch.tensor(n_keys if n_keys is not None else [N] * B, dtype=torch.int32)
    return IndexerCase(name=f"indexer_b{B}_n{N}", q=q, w=w, key_pool=pool, page_table=pt,
                       n_keys=nk, N=N, page=page)


@dataclass
class IndexerPrefillCase:
    """S sequences of query tokens: the tokens of sequence s are rows
    tok_start[s] .. tok_start[s+1]-1 of q [T, Hi, Dk] bf16 and w [T, Hi] fp32
    and sit at positions pos[t]; n_keys[t] = keys visible to token t (causal);
    key_pool / page_table [S, pages] as in IndexerCase; N = logits width."""
    name: str
    q: torch.Tensor
    w: torch.Tensor
    key_pool: torch.Tensor
    page_table: torch.Tensor
    tok_start: torch.Tensor
    pos: torch.Tensor
    n_keys: torch.Tensor
    N: int
    ratio: int
    page: int = PAGE

    @property
    def T(self):
        return int(self.q.shape[0])

    @property
    def max_tokens(self):
        return int((self.tok_start[1:] - self.tok_start[:-1]).max()) if self.tok_start.numel() > 1 else 0


def indexer_prefill_case(lengths=(8192,), starts=(0,), ratio: int = 2, Hi: int = 32, Dk: int = 128,
                         seed: int = SEED_BASE + 40, w_signed: bool = True, N: Optional[int] = None,
                         exp_lo: int = 120, exp_hi: int = 134, page: int = PAGE) -> IndexerPrefillCase:
    """Sequence s holds lengths[s] query tokens at positions starts[s] ..;
    its keys are the compressed entries at ratio r (r = 1: one key per token)
    and token p sees ceil((p+1)/r) of them.  N defaults to the largest
    visible count.  w ~ U(-1, 1) when w_signed (the score allows any sign)."""
    g = make_generator(seed)
    S = len(lengths)
    pos = torch.cat([torch.arange(st, st + ln, dtype=torch.int32) for ln, st in zip(lengths, starts)]) \
        if S else torch.zeros(0, dtype=torch.int32)
    nk = _n_visible_cmp(pos, ratio).to(torch.int32)
    if N is None:
        N = int(nk.max()) if nk.numel() else 0
    T = int(pos.numel())
    q = _normal_bf16((T, Hi, Dk), g)
    w = torch.rand((T, Hi), generator=g).to(torch.float32)
    if w_signed:
        w = w * 2.0 - 1.0
    pages = max(1, math.ceil(N / page))
    pt = page_table(S, pages, g)
    pool = fp4_key_rows(S * pages * page, g, exp_lo, exp_hi)
    ts = torch.zeros(S + 1, dtype=torch.int32)
    if S:
        ts[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int32), 0)
    name = "indexer_prefill_" + "_".join(f"n{ln}s{st}" for ln, st in zip(lengths, starts)) + f"_r{ratio}"
    return IndexerPrefillCase(name=name, q=q, w=w, key_pool=pool, page_table=pt, tok_start=ts, pos=pos,
                              n_keys=nk, N=N, ratio=ratio, page=page)


@dataclass
class IndexerCandCase:
    """T query tokens, each scoring the NC candidates cand[t] (logical key
    positions, -1 = none) of its sequence: q [T, Hi, Dk] bf16, w [T, Hi] fp32,
    page_table [T, pages] (one row per token; an expanded view with stride 0
    when all tokens share one sequence), n_keys [T]."""
    name: str
    q: torch.Tensor
    w: torch.Tensor
    key_pool: torch.Tensor
    page_table: torch.Tensor
    cand: torch.Tensor
    n_keys: torch.Tensor
    page: int = PAGE

    @property
    def T(self):
        return int(self.q.shape[0])

    @property
    def NC(self):
        return int(self.cand.shape[1])


def indexer_cand_case(T: int = 1, n_ctx: int = 131072, NC: int = 16384, shared_seq: bool = False,
                      start: Optional[int] = None, Hi: int = 32, Dk: int = 128, seed: int = SEED_BASE + 45,
                      sort: bool = True, w_signed: bool = True, extras: bool = False) -> IndexerCandCase:
    """Decode (shared_seq False): T sequences with n_ctx keys each, one query
    token each.  Prefill (shared_seq True): T tokens of one sequence at
    positions start .. start+T-1 (r = 1: token p sees p+1 keys).  Each token's
    candidates are min(NC, visible) distinct visible keys (ascending when
    sort, as a top-k hands them over), padded with -1.  extras plants, per
    token, a -1 inside the list, a duplicate and a key beyond the visible
    count (those score -inf)."""
    g = make_generator(seed)
    if shared_seq:
        st = n_ctx - T if start is None else start
        nk = torch.arange(st, st + T, dtype=torch.int32) + 1
        n_keys_pool, S = int(nk.max()) if T else 0, 1
    else:
        nk = torch.full((T,), n_ctx, dtype=torch.int32)
        n_keys_pool, S = n_ctx, T
    q = _normal_bf16((T, Hi, Dk), g)
    w = torch.rand((T, Hi), generator=g).to(torch.float32)
    if w_signed:
        w = w * 2.0 - 1.0
    pages = max(1, math.ceil((n_keys_pool + 1) / PAGE))
    pt = page_table(S, pages, g)
    pool = fp4_key_rows(S * pages * PAGE, g)
    cand = random_unique_indices(nk, NC, g)
    if sort:
        big = torch.iinfo(torch.int32).max
        cand = torch.where(cand < 0, torch.full_like(cand, big), cand).sort(dim=1).values
        cand = torch.where(cand == big, torch.full_like(cand, -1), cand)
    if extras and NC >= 4:
        for t in range(T):
            cand[t, 1] = -1
            cand[t, 2] = cand[t, 0]
            cand[t, 3] = int(nk[t])          # one past the visible keys
    pt_tok = pt.expand(T, pages) if shared_seq else pt
    name = f"indexer_cand_t{T}_ctx{n_ctx}_nc{NC}" + ("_shared" if shared_seq else "")
    return IndexerCandCase(name=name, q=q, w=w, key_pool=pool, page_table=pt_tok, cand=cand, n_keys=nk)


@dataclass
class GatedPoolCase:
    """x [B, R, D] (raw rows to pool) and gate [B, R, D] (per-channel gate
    scores); either may be a strided view of a larger buffer."""
    name: str
    x: torch.Tensor
    gate: torch.Tensor

    @property
    def B(self):
        return int(self.x.shape[0])

    @property
    def R(self):
        return int(self.x.shape[1])

    @property
    def D(self):
        return int(self.x.shape[2])


def gated_pool_case(B: int = 1, R: int = 128, D: int = 512, x_dtype=torch.bfloat16, gate_dtype=torch.float32,
                    seed: int = SEED_BASE + 70, gate_scale: float = 2.0, strided: bool = False) -> GatedPoolCase:
    """x ~ N(0, 1), gate ~ N(0, gate_scale^2), rounded to their dtypes.
    strided: x and gate are views with padded row and batch strides."""
    g = make_generator(seed)
    if strided:
        xb = torch.randn((B, R + 1, D + 24), generator=g).to(x_dtype)
        gb = (torch.randn((B, R + 2, D + 40), generator=g) * gate_scale).to(gate_dtype)
        x, gate = xb[:, 1:, 8:8 + D], gb[:, :R, 16:16 + D]
    else:
        x = torch.randn((B, R, D), generator=g).to(x_dtype)
        gate = (torch.randn((B, R, D), generator=g) * gate_scale).to(gate_dtype)
    name = f"gated_pool_b{B}_r{R}_d{D}" + ("_strided" if strided else "")
    return GatedPoolCase(name=name, x=x, gate=gate)
