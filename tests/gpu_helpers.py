"""Shared helpers of the GPU parity tests: run a seeded workload through the
HIP library (via the thin binding) and compare with the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import sparse_attention_paged_amd as sap

# Attention parity bar (bf16 inputs, fp32 accumulation, fp32 output).
ATTN_MAX_ABS = 1e-2
ATTN_REL_L2 = 2e-3


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X GPU")
    sap.lib()          # loud failure if the HIP library is missing


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(t):
    return None if t is None else t.cuda()


def gpu_idx(case):
    return sap.build_sparse_idx(dev(case.pos), dev(case.seq), case.n_win, dev(case.win_pt), case.page,
                                dev(case.cmp_logical) if case.n_cmp > 0 else None,
                                dev(case.cmp_pt) if case.n_cmp > 0 else None)


def gpu_attn(case, idx=None, q=None, out_dtype=torch.float32, num_splits=0, win_pool=None, cmp_pool=None):
    idx = gpu_idx(case) if idx is None else idx
    q = dev(case.q if q is None else q).to(torch.bfloat16)
    wp = dev(case.win_pool if win_pool is None else win_pool)
    cp = dev(case.cmp_pool if cmp_pool is None else cmp_pool)
    out = sap.sparse_attn_paged(q, wp, cp, idx, case.n_win, case.sm_scale, out_dtype=out_dtype,
                                win_scale=dev(case.win_scale), cmp_scale=dev(case.cmp_scale),
                                num_splits=num_splits)
    torch.cuda.synchronize()
    return out


def attn_errors(gpu: torch.Tensor, ref: torch.Tensor):
    g = gpu.detach().cpu().to(torch.float64)
    r = ref.to(torch.float64)
    d = g - r
    max_abs = float(d.abs().max()) if d.numel() else 0.0
    den = float(r.norm())
    rel = float(d.norm()) / den if den > 0 else float(d.norm())
    return max_abs, rel


def assert_attn_close(gpu, ref, label, max_abs=ATTN_MAX_ABS, rel_l2=ATTN_REL_L2):
    """The parity bar on fp32 outputs; callers widen it only by a derived term."""
    assert torch.isfinite(gpu).all(), f"{label}: non-finite output"
    ma, rl = attn_errors(gpu, ref)
    say(f"  {label}: max-abs {ma:.3e} rel-L2 {rl:.3e}")
    assert ma <= max_abs and rl <= rel_l2, f"{label}: max-abs {ma:.3e} rel-L2 {rl:.3e}"


def bf16_copy(t):
    return t.to(torch.bfloat16)
