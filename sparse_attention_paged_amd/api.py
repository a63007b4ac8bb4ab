"""Torch-facing wrappers with the names of the C ABI (include/sap.h).

Argument marshalling only: each function checks that tensors live on the
GPU, reads pointers, strides and dtypes, allocates outputs/workspace through
torch when the caller did not pass them, and calls the library on the
current HIP stream.  Every step of the computation runs in libsap.so.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from ._lib import SAP_BF16, SAP_F32, SAP_FP8_E4M3, check, lib

_FP8_DTYPES = {torch.uint8}
if hasattr(torch, "float8_e4m3fn"):
    _FP8_DTYPES.add(torch.float8_e4m3fn)


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("sparse_attention_paged_amd takes GPU tensors only")


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ws(workspace: Optional[torch.Tensor]):
    """(pointer, size in bytes) of a caller's workspace; the ABI wants it
    256-byte aligned."""
    if workspace is None:
        return None, 0
    if workspace.data_ptr() % 256:
        raise ValueError("workspace must be 256-byte aligned")
    return _p(workspace), workspace.numel() * workspace.element_size()


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _kv_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SAP_BF16
    if t.dtype in _FP8_DTYPES:
        return SAP_FP8_E4M3
    raise ValueError(f"unsupported KV pool dtype {t.dtype}")


def _out_dtype(dt) -> int:
    if dt == torch.float32:
        return SAP_F32
    if dt == torch.bfloat16:
        return SAP_BF16
    raise ValueError(f"unsupported output dtype {dt}")


def build_sparse_idx(pos, seq, n_win: int, win_pt, page: int, cmp_logical=None, cmp_pt=None,
                     out=None) -> torch.Tensor:
    """int32 [T, n_win + n_cmp] physical rows (window columns, then compressed)."""
    _dev(pos, seq, win_pt, cmp_logical, cmp_pt, out)
    T = pos.numel()
    n_cmp = 0 if cmp_logical is None else int(cmp_logical.shape[1])
    if out is None:
        out = torch.empty((T, n_win + n_cmp), dtype=torch.int32, device=pos.device)
    rc = lib().sap_build_sparse_idx(
        _p(pos), _p(seq), T, n_win, _p(win_pt), win_pt.stride(0) if win_pt is not None else 0, page,
        _p(cmp_logical), cmp_logical.stride(0) if cmp_logical is not None else 0, n_cmp,
        _p(cmp_pt), cmp_pt.stride(0) if cmp_pt is not None else 0, _p(out), out.stride(0), _stream(pos))
    check(rc, "sap_build_sparse_idx")
    return out


def sparse_attn_num_splits(T: int, H: int, D: int, n_cols: int, num_splits: int = 0) -> int:
    return int(lib().sap_sparse_attn_num_splits(T, H, D, n_cols, num_splits))


def sparse_attn_workspace_bytes(T: int, H: int, D: int, n_cols: int, num_splits: int = 0) -> int:
    return int(lib().sap_sparse_attn_workspace_bytes(T, H, D, n_cols, num_splits))


def sparse_attn_paged(q, win_pool, cmp_pool, idx, n_win: int, sm_scale: float, *, out=None,
                      out_dtype=torch.float32, win_scale=None, cmp_scale=None, num_splits: int = 0,
                      workspace=None) -> torch.Tensor:
    """q [T, H, D] bf16; pools [N, D] bf16 or e4m3 codes (uint8 / float8_e4m3fn) with
    per-row fp32 scales; idx [T, n_win + n_cmp] int32 physical rows, -1 = unused."""
    _dev(q, win_pool, cmp_pool, idx, win_scale, cmp_scale, out, workspace)
    T, H, D = q.shape
    C = int(idx.shape[1])
    n_cmp = C - n_win
    if out is None:
        out = torch.empty((T, H, D), dtype=out_dtype, device=q.device)
    if q.stride(2) != 1 or out.stride(2) != 1 or idx.stride(1) != 1:
        raise ValueError("the innermost dimension must be contiguous")
    kv = _kv_dtype(win_pool)
    cmp = cmp_pool if cmp_pool is not None else win_pool
    if cmp_pool is not None and _kv_dtype(cmp_pool) != kv:
        raise ValueError("both pools must share one dtype")
    need = sparse_attn_workspace_bytes(T, H, D, C, num_splits)
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    rc = lib().sap_sparse_attn_paged(
        _p(q), SAP_BF16 if q.dtype == torch.bfloat16 else -1, q.stride(0), q.stride(1),
        _p(win_pool), win_pool.stride(0) * win_pool.element_size(),
        _p(cmp), cmp.stride(0) * cmp.element_size(), kv,
        _p(idx), idx.stride(0), n_win, n_cmp,
        _p(win_scale), _p(cmp_scale),
        _p(out), _out_dtype(out.dtype), out.stride(0), out.stride(1),
        T, H, D, float(sm_scale), int(num_splits),
        *_ws(workspace), _stream(q))
    check(rc, "sap_sparse_attn_paged")
    return out


def sparse_attn_noalloc_max_bytes() -> int:
    return int(lib().sap_sparse_attn_noalloc_max_bytes())


def sparse_attn_paged_noalloc(q, win_pool, cmp_pool, idx, n_win: int, sm_scale: float, *, out,
                              win_scale=None, cmp_scale=None, num_splits: int = 0) -> torch.Tensor:
    """sparse_attn_paged without a workspace: the split partials live in the
    library's fixed device array, and the call allocates nothing (`out` is
    required for the same reason)."""
    _dev(q, win_pool, cmp_pool, idx, win_scale, cmp_scale, out)
    T, H, D = q.shape
    C = int(idx.shape[1])
    if q.stride(2) != 1 or out.stride(2) != 1 or idx.stride(1) != 1:
        raise ValueError("the innermost dimension must be contiguous")
    kv = _kv_dtype(win_pool)
    cmp = cmp_pool if cmp_pool is not None else win_pool
    if cmp_pool is not None and _kv_dtype(cmp_pool) != kv:
        raise ValueError("both pools must share one dtype")
    rc = lib().sap_sparse_attn_paged_noalloc(
        _p(q), SAP_BF16 if q.dtype == torch.bfloat16 else -1, q.stride(0), q.stride(1),
        _p(win_pool), win_pool.stride(0) * win_pool.element_size(),
        _p(cmp), cmp.stride(0) * cmp.element_size(), kv,
        _p(idx), idx.stride(0), n_win, C - n_win,
        _p(win_scale), _p(cmp_scale),
        _p(out), _out_dtype(out.dtype), out.stride(0), out.stride(1),
        T, H, D, float(sm_scale), int(num_splits), _stream(q))
    check(rc, "sap_sparse_attn_paged_noalloc")
    return out


def indexer_logits_packed(q, w, key_pool, page_table, page: int, N: int, n_keys=None,
                          out=None) -> torch.Tensor:
    """q [B, Hi, 128] bf16, w [B, Hi] fp32, key_pool [rows, >=17] int32 -> logits [B, N] fp32."""
    _dev(q, w, key_pool, page_table, n_keys, out)
    B, Hi, D = q.shape
    if out is None:
        out = torch.empty((B, N), dtype=torch.float32, device=q.device)
    rc = lib().sap_indexer_logits_packed(
        _p(q), q.stride(0), _p(w), w.stride(0), _p(key_pool), key_pool.stride(0),
        _p(page_table), page_table.stride(0) if page_table is not None else 0, page,
        _p(n_keys), _p(out), out.stride(0), B, Hi, D, N, _stream(q))
    check(rc, "sap_indexer_logits_packed")
    return out


def indexer_logits_candidates(q, w, key_pool, page_table, page: int, cand, n_keys=None,
                              out=None) -> torch.Tensor:
    """q [T, Hi, 128] bf16, w [T, Hi] fp32, cand [T, NC] int32 logical key
    positions (-1 = none), page_table [T, pages] (stride 0 rows allowed) or
    None -> logits [T, NC] fp32."""
    _dev(q, w, key_pool, page_table, cand, n_keys, out)
    T, Hi, D = q.shape
    NC = cand.shape[1]
    if out is None:
        out = torch.empty((T, NC), dtype=torch.float32, device=q.device)
    rc = lib().sap_indexer_logits_candidates(
        _p(q), q.stride(0), _p(w), w.stride(0), _p(key_pool), key_pool.stride(0),
        _p(page_table), page_table.stride(0) if page_table is not None else 0, page,
        _p(cand), cand.stride(0), _p(n_keys), _p(out), out.stride(0), T, Hi, D, NC, _stream(q))
    check(rc, "sap_indexer_logits_candidates")
    return out


def indexer_logits_prefill(q, w, key_pool, page_table, page: int, tok_start, max_tokens: int, N: int,
                           n_keys=None, out=None) -> torch.Tensor:
    """q [T, Hi, 128] bf16, w [T, Hi] fp32, page_table [S, pages] or None,
    tok_start [S + 1] int32, n_keys [T] int32 -> logits [T, N] fp32."""
    _dev(q, w, key_pool, page_table, tok_start, n_keys, out)
    T, Hi, D = q.shape
    S = tok_start.numel() - 1
    if out is None:
        out = torch.empty((T, N), dtype=torch.float32, device=q.device)
    rc = lib().sap_indexer_logits_prefill(
        _p(q), q.stride(0), _p(w), w.stride(0), _p(key_pool), key_pool.stride(0),
        _p(page_table), page_table.stride(0) if page_table is not None else 0, page,
        _p(tok_start), S, max_tokens, _p(n_keys), _p(out), out.stride(0), Hi, D, N, _stream(q))
    check(rc, "sap_indexer_logits_prefill")
    return out


def _float_dtype(dt) -> int:
    if dt == torch.bfloat16:
        return SAP_BF16
    if dt == torch.float32:
        return SAP_F32
    raise ValueError(f"unsupported dtype {dt} (bf16 or fp32)")


def gated_pool(x, gate, out_dtype=torch.float32, out=None) -> torch.Tensor:
    """x, gate [B, R, D] (bf16 or fp32, unit stride along D) -> [B, D]:
    softmax over R of the gates weighting the rows."""
    _dev(x, gate, out)
    B, R, D = x.shape
    if gate.shape != x.shape:
        raise ValueError("x and gate must have the same shape")
    if D > 1 and (x.stride(2) != 1 or gate.stride(2) != 1):
        raise ValueError("x and gate need unit stride along D")
    if out is None:
        out = torch.empty((B, D), dtype=out_dtype, device=x.device)
    rc = lib().sap_gated_pool(_p(x), _float_dtype(x.dtype), x.stride(0), x.stride(1),
                              _p(gate), _float_dtype(gate.dtype), gate.stride(0), gate.stride(1),
                              _p(out), _float_dtype(out.dtype), out.stride(0), B, R, D, _stream(x))
    check(rc, "sap_gated_pool")
    return out


def topk_workspace_bytes(B: int, N: int, k: int) -> int:
    return int(lib().sap_topk_workspace_bytes(B, N, k))


def topk_select(logits, k: int, n_valid=None, out=None, workspace=None) -> torch.Tensor:
    """logits [B, N] fp32 -> int32 [B, k] indices in ascending order, -1 padded."""
    _dev(logits, n_valid, out, workspace)
    B, N = logits.shape
    if out is None:
        out = torch.empty((B, k), dtype=torch.int32, device=logits.device)
    need = topk_workspace_bytes(B, N, k)
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=logits.device)
    rc = lib().sap_topk_select(
        _p(logits), logits.stride(0), _p(n_valid), B, N, k, _p(out), out.stride(0), *_ws(workspace),
        _stream(logits))
    check(rc, "sap_topk_select")
    return out


def topk_sparse_idx(logits, k: int, pos, seq, n_win: int, win_pt, cmp_pt, page: int, n_valid=None, out=None,
                    workspace=None) -> torch.Tensor:
    """Top-k of logits [T, N] fused with the index build -> int32 [T, n_win + k]
    attention column rows (window rows, then the selected entries' rows)."""
    _dev(logits, pos, seq, win_pt, cmp_pt, n_valid, out, workspace)
    T, N = logits.shape
    if out is None:
        out = torch.empty((T, n_win + k), dtype=torch.int32, device=logits.device)
    need = topk_workspace_bytes(T, N, k)
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=logits.device)
    rc = lib().sap_topk_sparse_idx(
        _p(logits), logits.stride(0), _p(n_valid), T, N, k, _p(pos), _p(seq), n_win,
        _p(win_pt), win_pt.stride(0) if win_pt is not None else 0, _p(cmp_pt), cmp_pt.stride(0), page,
        _p(out), out.stride(0), *_ws(workspace), _stream(logits))
    check(rc, "sap_topk_sparse_idx")
    return out


def debug_e4m3_table(device="cuda"):
    """(uint16 [256] bf16 bits from the attention row loader, fold factor)."""
    out = torch.empty(256, dtype=torch.int16, device=device)
    fold = torch.empty(1, dtype=torch.float32, device=device)
    check(lib().sap_debug_e4m3_table(_p(out), _p(fold), _stream(out)), "sap_debug_e4m3_table")
    return out, fold


def debug_e4m3_f16_table(device="cuda"):
    """uint16 [256]: f16 bits of each e4m3 code from the one-pass kernel's V^T widening."""
    out = torch.empty(256, dtype=torch.int16, device=device)
    check(lib().sap_debug_e4m3_f16_table(_p(out), _stream(out)), "sap_debug_e4m3_f16_table")
    return out


def debug_fp4_table(device="cuda"):
    """int16 [256, 256, 2]: bf16 bits of (code byte, scale byte, nibble) from the indexer's decoder."""
    out = torch.empty((256, 256, 2), dtype=torch.int16, device=device)
    check(lib().sap_debug_fp4_table(_p(out), _stream(out)), "sap_debug_fp4_table")
    return out
