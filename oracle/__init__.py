"""Python access to the CPU parity oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  It never touches the HIP library and
the HIP library never touches it.  All arithmetic is in the C file, in double
precision; this module only marshals CPU tensors through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

BF16, F32, E4M3 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (plain -O2, OpenMP over independent outputs)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(_LIB)
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.orc_bf16_to_double.argtypes = [ctypes.c_uint16]; L.orc_bf16_to_double.restype = D
        L.orc_e4m3_to_double.argtypes = [ctypes.c_uint8]; L.orc_e4m3_to_double.restype = D
        L.orc_e2m1_to_double.argtypes = [ctypes.c_uint]; L.orc_e2m1_to_double.restype = D
        L.orc_ue8m0_to_double.argtypes = [ctypes.c_uint]; L.orc_ue8m0_to_double.restype = D
        L.orc_double_to_bf16.argtypes = [D]; L.orc_double_to_bf16.restype = ctypes.c_uint16
        L.orc_fp4_row_element.argtypes = [P, I]; L.orc_fp4_row_element.restype = D
        L.orc_fp4_table.argtypes = [P]; L.orc_fp4_table.restype = None
        L.orc_fp4_decode_rows.argtypes = [P, I64, I64, P]; L.orc_fp4_decode_rows.restype = None
        L.orc_e4m3_table.argtypes = [P]; L.orc_e4m3_table.restype = None
        L.orc_build_idx.argtypes = [I, P, P, I, P, I64, I, P, I64, I, P, I64, P, I64]
        L.orc_build_idx.restype = I
        L.orc_sparse_attn.argtypes = [I, I, I, P, I, I64, I64, P, I64, P, I64, I, P, P,
                                      P, I64, I, I, D, P]
        L.orc_sparse_attn.restype = I
        L.orc_indexer_logits.argtypes = [I, I, I, P, I64, P, I64, P, I64, P, I64, I, P, I,
                                         P, I64]
        L.orc_indexer_logits.restype = I
        L.orc_indexer_candidates.argtypes = [I, I, I, P, I64, P, I64, P, I64, P, I64, I, P, I64, P, I,
                                             P, I64]
        L.orc_indexer_candidates.restype = I
        L.orc_gated_pool.argtypes = [I, I, I, P, P, P]
        L.orc_gated_pool.restype = I
        L.orc_topk.argtypes = [I, I, P, I64, P, I, P, I64]
        L.orc_topk.restype = I
        L.orc_num_threads.argtypes = []; L.orc_num_threads.restype = I
        _lib = L
    return _lib


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _cpu(t, dtype=None):
    if t is None:
        return None
    t = t.detach().cpu()
    if dtype is not None:
        t = t.to(dtype)
    return t.contiguous()


def num_threads() -> int:
    return int(lib().orc_num_threads())


# --- formats ----------------------------------------------------------------

def e4m3_table() -> np.ndarray:
    out = np.zeros(256, dtype=np.float64)
    lib().orc_e4m3_table(out.ctypes.data_as(ctypes.c_void_p))
    return out


def fp4_table() -> np.ndarray:
    """uint16 [256, 256, 2]: bf16 bits of the low/high nibble of each code byte
    times each ue8m0 scale byte."""
    out = np.zeros(256 * 256 * 2, dtype=np.uint16)
    lib().orc_fp4_table(out.ctypes.data_as(ctypes.c_void_p))
    return out.reshape(256, 256, 2)


def e2m1(nibble: int) -> float:
    return float(lib().orc_e2m1_to_double(nibble))


def ue8m0(e: int) -> float:
    return float(lib().orc_ue8m0_to_double(e))


def to_bf16_bits(x: float) -> int:
    return int(lib().orc_double_to_bf16(float(x)))


def fp4_rows_decode(rows: torch.Tensor) -> np.ndarray:
    """[n, >=17] int32 packed rows -> [n, 128] float64 dequantised values."""
    rows = _cpu(rows, torch.int32)
    n = rows.shape[0]
    out = np.zeros((n, 128), dtype=np.float64)
    lib().orc_fp4_decode_rows(_p(rows), n, rows.stride(0), out.ctypes.data_as(ctypes.c_void_p))
    return out


# --- index build ------------------------------------------------------------

def build_idx(pos, seq, n_win, win_pt, page, cmp_logical, n_cmp, cmp_pt) -> torch.Tensor:
    pos, seq, win_pt = _cpu(pos, torch.int32), _cpu(seq, torch.int32), _cpu(win_pt, torch.int32)
    cmp_logical = _cpu(cmp_logical, torch.int32)
    cmp_pt = _cpu(cmp_pt, torch.int32) if cmp_pt is not None else torch.zeros((1, 1), dtype=torch.int32)
    T = pos.numel()
    idx = torch.empty((T, n_win + n_cmp), dtype=torch.int32)
    rc = lib().orc_build_idx(T, _p(pos), _p(seq), n_win, _p(win_pt), win_pt.stride(0), page,
                             _p(cmp_logical), cmp_logical.stride(0) if cmp_logical.dim() == 2 else 0,
                             n_cmp, _p(cmp_pt), cmp_pt.stride(0), _p(idx), idx.stride(0))
    if rc != 0:
        raise ValueError(f"orc_build_idx rejected its arguments ({rc})")
    return idx


def case_idx(case) -> torch.Tensor:
    return build_idx(case.pos, case.seq, case.n_win, case.win_pt, case.page,
                     case.cmp_logical, case.n_cmp, case.cmp_pt)


# --- sparse attention -------------------------------------------------------

_DT = {torch.bfloat16: BF16, torch.float32: F32, torch.uint8: E4M3}


def sparse_attn(q, win_pool, cmp_pool, idx, n_win, sm_scale, win_scale=None, cmp_scale=None,
                kv_fp8=None) -> torch.Tensor:
    """Returns float64 [T, H, D].  q: [T,H,D] bf16/fp32; pools [N, D] bf16/fp32
    or uint8 e4m3 codes (then per-row fp32 scales are required)."""
    q = _cpu(q)
    win_pool = _cpu(win_pool)
    cmp_pool = _cpu(cmp_pool) if cmp_pool is not None else None
    idx = _cpu(idx, torch.int32)
    T, H, D = q.shape
    n_cmp = idx.shape[1] - n_win
    kvd = _DT[win_pool.dtype]
    cmpp = cmp_pool if cmp_pool is not None else win_pool
    if cmp_pool is not None and _DT[cmp_pool.dtype] != kvd:
        raise ValueError("both pools must share one dtype")
    ws = _cpu(win_scale, torch.float32)
    cs = _cpu(cmp_scale, torch.float32)
    out = torch.empty((T, H, D), dtype=torch.float64)
    rc = lib().orc_sparse_attn(T, H, D, _p(q), _DT[q.dtype], q.stride(0), q.stride(1),
                               _p(win_pool), win_pool.stride(0) * win_pool.element_size(),
                               _p(cmpp), cmpp.stride(0) * cmpp.element_size(), kvd,
                               _p(ws), _p(cs), _p(idx), idx.stride(0), n_win, n_cmp,
                               float(sm_scale), _p(out))
    if rc != 0:
        raise ValueError(f"orc_sparse_attn rejected its arguments ({rc})")
    return out


def case_attn(case, idx=None, q=None, win_pool=None, cmp_pool=None) -> torch.Tensor:
    idx = case_idx(case) if idx is None else idx
    return sparse_attn(case.q if q is None else q,
                       case.win_pool if win_pool is None else win_pool,
                       case.cmp_pool if cmp_pool is None else cmp_pool,
                       idx, case.n_win, case.sm_scale, case.win_scale, case.cmp_scale)


# --- indexer and top-k ------------------------------------------------------

def indexer_logits(q, w, key_pool, page_table, page, n_keys, N) -> torch.Tensor:
    """float64 [B, N]."""
    q = _cpu(q, torch.bfloat16)
    w = _cpu(w, torch.float32)
    key_pool = _cpu(key_pool, torch.int32)
    pt = _cpu(page_table, torch.int32) if page_table is not None else None
    nk = _cpu(n_keys, torch.int32) if n_keys is not None else None
    B, Hi, Dk = q.shape
    out = torch.empty((B, N), dtype=torch.float64)
    rc = lib().orc_indexer_logits(B, Hi, Dk, _p(q), q.stride(0), _p(w), w.stride(0),
                                  _p(key_pool), key_pool.stride(0), _p(pt),
                                  pt.stride(0) if pt is not None else 0, page, _p(nk), N,
                                  _p(out), out.stride(0))
    if rc != 0:
        raise ValueError(f"orc_indexer_logits rejected its arguments ({rc})")
    return out


def case_indexer(case) -> torch.Tensor:
    return indexer_logits(case.q, case.w, case.key_pool, case.page_table, case.page,
                          case.n_keys, case.N)


def indexer_prefill_logits(q, w, key_pool, page_table, page, tok_start, n_keys, N) -> torch.Tensor:
    """float64 [T, N].  Prefill mode: token t of sequence s (rows tok_start[s]
    .. tok_start[s+1]-1) is scored like a full-mode query over sequence s's
    keys, with its own visible count n_keys[t] (the causal mask)."""
    ts = _cpu(tok_start, torch.int64)
    pt = _cpu(page_table, torch.int32)
    T = int(ts[-1])
    seq = torch.repeat_interleave(torch.arange(ts.numel() - 1), ts[1:] - ts[:-1])
    assert seq.numel() == T
    return indexer_logits(q, w, key_pool, pt[seq].contiguous(), page, n_keys, N)


def indexer_candidates(q, w, key_pool, page_table, page, cand, n_keys) -> torch.Tensor:
    """float64 [T, NC]: candidate-mode logits (page_table [T, pages], one row
    per token, or None: candidates are pool rows)."""
    q = _cpu(q, torch.bfloat16)
    w = _cpu(w, torch.float32)
    key_pool = _cpu(key_pool, torch.int32)
    pt = _cpu(page_table, torch.int32) if page_table is not None else None
    cand = _cpu(cand, torch.int32)
    nk = _cpu(n_keys, torch.int32) if n_keys is not None else None
    T, Hi, Dk = q.shape
    NC = cand.shape[1]
    out = torch.empty((T, NC), dtype=torch.float64)
    rc = lib().orc_indexer_candidates(T, Hi, Dk, _p(q), q.stride(0), _p(w), w.stride(0),
                                      _p(key_pool), key_pool.stride(0), _p(pt),
                                      pt.stride(0) if pt is not None else 0, page, _p(cand), cand.stride(0),
                                      _p(nk), NC, _p(out), out.stride(0))
    if rc != 0:
        raise ValueError(f"orc_indexer_candidates rejected its arguments ({rc})")
    return out


def gated_pool(x, gate) -> torch.Tensor:
    """float64 [B, D]: softmax over R of the gates weighting the R rows
    (x, gate [B, R, D] of any float dtype; values are taken exactly)."""
    xd = _cpu(x, torch.float64)
    gd = _cpu(gate, torch.float64)
    B, R, D = xd.shape
    out = torch.empty((B, D), dtype=torch.float64)
    rc = lib().orc_gated_pool(B, R, D, _p(xd), _p(gd), _p(out))
    if rc != 0:
        raise ValueError(f"orc_gated_pool rejected its arguments ({rc})")
    return out


def topk(x, k, n_valid=None) -> torch.Tensor:
    """x: [B, N] float32 (the selection is made on float32 values); int32 [B, k]."""
    x = _cpu(x, torch.float32)
    B, N = x.shape
    nv = _cpu(n_valid, torch.int32) if n_valid is not None else None
    out = torch.empty((B, k), dtype=torch.int32)
    rc = lib().orc_topk(B, N, _p(x), x.stride(0), _p(nv), k, _p(out), out.stride(0))
    if rc != 0:
        raise ValueError(f"orc_topk rejected its arguments ({rc})")
    return out
