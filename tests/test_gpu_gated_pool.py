"""GPU parity of the gated pool ("perf(kernel): keep 16-byte kv loads in
dsv4 sparse attention and unroll gated pool": Kernel time shapes B 1 / 8,
R 8 / 128, D 128 / 512; Correctness and tests: R = 1/3/5/7/9/16/127/129,
D = 300/100/64, bf16 and fp32 output, strided views).

Tolerance: fp32 exponentials and sums over R <= 129 terms stay below
1e-5 of M = sum_r p_r |x_r| (p = the softmax weights); a bf16 output adds
its rounding, at most 2^-8 of the value.
"""
import hashlib
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_paged_amd as sap
import workloads as W
from gpu_helpers import need_gpu, say

pytestmark = pytest.mark.gpu


def _check(case, out_dtype, label, gate=None):
    gate = case.gate if gate is None else gate
    got = sap.gated_pool(case.x.cuda(), gate.cuda(), out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref = oracle.gated_pool(case.x, gate)
    g64 = gate.to(torch.float64)
    p = torch.softmax(g64, dim=1).nan_to_num(0.0)
    M = (p * case.x.to(torch.float64).abs()).sum(1)
    err = (got.cpu().to(torch.float64) - ref).abs()
    bound = 1e-5 * M + (2.0 ** -8 * ref.abs() if out_dtype == torch.bfloat16 else 0.0) + 1e-30
    worst = float((err / bound).max())
    say(f"  {label}: worst error / bound = {worst:.3f}")
    assert torch.isfinite(got).all(), label
    assert worst <= 1.0, label


@pytest.mark.parametrize("B", [1, 8])
@pytest.mark.parametrize("R", [8, 128])
@pytest.mark.parametrize("D", [128, 512])
def test_gated_pool_page_shapes(B, R, D):
    need_gpu()
    case = W.gated_pool_case(B=B, R=R, D=D, seed=W.SEED_BASE + 700 + B + R + D)
    _check(case, torch.float32, case.name)
    _check(case, torch.bfloat16, case.name + " bf16 out")


@pytest.mark.parametrize("R", [1, 3, 5, 7, 9, 16, 127, 129])
@pytest.mark.parametrize("D", [300, 100, 64])
def test_gated_pool_edge_shapes(R, D):
    need_gpu()
    case = W.gated_pool_case(B=3, R=R, D=D, x_dtype=torch.float32, gate_dtype=torch.bfloat16,
                             seed=W.SEED_BASE + 720 + R + D, strided=(R % 2 == 1))
    _check(case, torch.float32, case.name)
    _check(case, torch.bfloat16, case.name + " bf16 out")


def test_gated_pool_masked_and_dominant_gates():
    """-inf gates (some rows; every row of some columns) and a gate far
    above the rest (the pooled value is that row's)."""
    need_gpu()
    case = W.gated_pool_case(B=2, R=20, D=96, seed=W.SEED_BASE + 740)
    gate = case.gate.clone()
    gate[:, 3] = -math.inf
    gate[:, :, 5] = -math.inf
    gate[1, 7, 10:20] = 300.0
    _check(case, torch.float32, "masked and dominant", gate=gate)
    got = sap.gated_pool(case.x.cuda(), gate.cuda()).cpu()
    assert (got[:, 5] == 0).all()
    assert torch.equal(got[1, 10:20], case.x[1, 7, 10:20].to(torch.float32))


def test_determinism_sha256_gated_pool():
    need_gpu()
    case = W.gated_pool_case(B=8, R=128, D=512, seed=W.SEED_BASE + 790)
    x, g = case.x.cuda(), case.gate.cuda()
    h = set()
    for _ in range(3):
        out = sap.gated_pool(x, g)
        torch.cuda.synchronize()
        h.add(hashlib.sha256(out.cpu().numpy().tobytes()).hexdigest())
    assert len(h) == 1
