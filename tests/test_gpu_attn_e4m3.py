"""GPU parity of the one-pass kernel at head_dim 512 with e4m3 rows (fp8 KV
in prefill, 'Perf/kv fp8 read path', What this changes) against the CPU
oracle: the raw codes are gathered into LDS, widened in registers, the row
scale multiplies the scores and the weights enter PV as two f16 terms after
the scale's power of two has been moved into the log2 score.

The cases mirror the bf16 prefill edge cases (every persistent workgroup
slot over two rounds, ragged last tiles, one to three tiles per token, a
partial head block with more than one staged index chunk, empty rows, bf16
output) and add scale values the pages' workload never draws: zero,
negative, tiny and huge scales, which the exponent fold must handle with the
same relative accuracy.
"""
import dataclasses
import hashlib

import pytest
import torch

import oracle
import sparse_attention_paged_amd as sap
import workloads as W
from gpu_helpers import assert_attn_close, dev, gpu_attn, gpu_idx, need_gpu, say

pytestmark = pytest.mark.gpu

E4 = dict(kv_dtype="e4m3", q_scale=2.0 ** -7)


def test_e4m3_prefill_every_workgroup_slot_two_rounds():
    """S8192 r4 e4m3: tokens 0 .. 511 (every (workgroup, round) slot of the
    first two rounds of the 256 persistent workgroups) and the last 512."""
    need_gpu()
    case = W.prefill_case(T=8192, ratio=4, seed=W.SEED_BASE + 150, **E4)
    gidx = gpu_idx(case)
    out = gpu_attn(case, idx=gidx, num_splits=1)
    idx = oracle.case_idx(case)
    assert torch.equal(gidx.cpu(), idx)
    for lo, hi in ((0, 512), (8192 - 512, 8192)):
        toks = list(range(lo, hi))
        ref = oracle.sparse_attn(case.q[toks], case.win_pool, case.cmp_pool, idx[toks], case.n_win, case.sm_scale,
                                 case.win_scale, case.cmp_scale)
        assert_attn_close(out[toks], ref, f"e4m3 tokens {lo} .. {hi - 1}")


def test_e4m3_prefill_small_full():
    # every token; ragged last tiles and clipped windows
    need_gpu()
    case = W.prefill_case(T=333, ratio=4, topk=70, seed=W.SEED_BASE + 151, **E4)
    assert_attn_close(gpu_attn(case, num_splits=1), oracle.case_attn(case), "e4m3 prefill T=333 top-k 70")


def test_e4m3_prefill_chunks_partial_heads():
    """More tokens than workgroups, H = 20 (a partial head block) and 3128
    columns (two staged index chunks)."""
    need_gpu()
    case = W.prefill_case(T=300, start=16000, ratio=4, topk=3000, H=20, seed=W.SEED_BASE + 152, **E4)
    assert oracle.case_idx(case).shape[1] > 2048
    assert_attn_close(gpu_attn(case, num_splits=1), oracle.case_attn(case), "e4m3 T=300 H=20 3128 columns")


@pytest.mark.parametrize("n_win,topk", [(0, 64), (1, 0), (128, 1), (50, 37), (100, 512)])
def test_e4m3_tile_counts(n_win, topk):
    # tokens with one, two, three and more tiles (the tile loop's peeled paths)
    need_gpu()
    case = W.prefill_case(T=260, start=900, ratio=4, n_win=n_win, topk=topk,
                          seed=W.SEED_BASE + 153 + n_win + topk, **E4)
    assert_attn_close(gpu_attn(case, num_splits=1), oracle.case_attn(case), f"e4m3 window {n_win} top-k {topk}")


@pytest.mark.parametrize("H", [1, 16, 128])
def test_e4m3_head_counts(H):
    need_gpu()
    case = W.decode_case(B=3, pos=4000, ratio=4, H=H, kv_dtype="e4m3", seed=W.SEED_BASE + 160 + H)
    assert_attn_close(gpu_attn(case, num_splits=1), oracle.case_attn(case), f"e4m3 H={H} one pass")


def test_e4m3_empty_rows():
    need_gpu()
    case = W.decode_case(B=4, pos=2000, ratio=4, topk=128, kv_dtype="e4m3", seed=W.SEED_BASE + 165)
    idx = oracle.case_idx(case)
    idx[1, :] = -1                       # no valid column -> zeros
    idx[2, case.n_win:] = -1             # window only
    idx[3, :case.n_win] = -1             # compressed only, with a hole
    idx[3, case.n_win + 5:case.n_win + 40] = -1
    out = gpu_attn(case, idx=dev(idx), num_splits=1)
    assert (out[1] == 0).all()
    assert_attn_close(out, oracle.case_attn(case, idx=idx), "e4m3 holes one pass")


def _with_scales(case, fw, fc):
    return dataclasses.replace(case, win_scale=fw(case.win_scale.clone()), cmp_scale=fc(case.cmp_scale.clone()))


def test_e4m3_zero_and_negative_scales():
    """A zero scale makes a row's key and value zero: its score is 0 and it
    still counts in the softmax sum.  A negative scale flips the row."""
    need_gpu()
    base = W.prefill_case(T=400, ratio=4, topk=200, seed=W.SEED_BASE + 170, **E4)
    g = torch.Generator().manual_seed(171)

    def mix(s):
        r = torch.rand(s.shape, generator=g)
        s[r < 0.2] = 0.0
        s[(r >= 0.2) & (r < 0.5)] *= -1.0
        return s

    case = _with_scales(base, mix, mix)
    assert (case.win_scale == 0).any() and (case.cmp_scale < 0).any()
    assert_attn_close(gpu_attn(case, num_splits=1), oracle.case_attn(case), "e4m3 zero/negative scales")


@pytest.mark.parametrize("lo,hi", [(-40.0, -20.0), (6.0, 14.0), (-30.0, 10.0)])
def test_e4m3_scale_ranges(lo, hi):
    """Row scales log-uniform in [2^lo, 2^hi]: the power of two of each scale
    goes into the log2 score, so the weights' f16 terms neither overflow nor
    lose precision whatever the range.  Every error term of the kernel is
    relative to the magnitude of the rows' values (|out| reaches 448 max|s|),
    so the bar is the pages' one at their largest row values (448 * 4)
    scaled by max|ref| / 1792 where that is larger; q is scaled down with the
    keys so the scores keep a spread of a few units."""
    need_gpu()
    g = torch.Generator().manual_seed(172)

    def draw(s):
        return torch.exp2(torch.rand(s.shape, generator=g) * (hi - lo) + lo).to(torch.float32)

    base = W.prefill_case(T=300, ratio=4, topk=150, seed=W.SEED_BASE + 173, **E4)
    case = _with_scales(base, draw, draw)
    qs = 2.0 ** -(max(hi, 2.0) - 2.0)
    case = dataclasses.replace(case, q=(case.q.float() * qs).to(torch.bfloat16))
    ref = oracle.case_attn(case)
    scale = max(1.0, ref.abs().max().item() / 1792.0)
    say(f"  scales 2^[{lo}, {hi}]: max|ref| {ref.abs().max().item():.3e}")
    assert_attn_close(gpu_attn(case, num_splits=1), ref, f"e4m3 scales 2^[{lo}, {hi}]", max_abs=1e-2 * scale)


def test_e4m3_bf16_output_and_determinism():
    # bf16 output: one more rounding, half an ulp of an 8-bit significand
    # (<= 2^-8 |x|); three runs give identical bytes
    need_gpu()
    case = W.prefill_case(T=500, ratio=4, seed=W.SEED_BASE + 175, **E4)
    ref = oracle.case_attn(case)
    gidx = gpu_idx(case)
    out = gpu_attn(case, idx=gidx, out_dtype=torch.bfloat16, num_splits=1)
    bound = 1e-2 + 2.0 ** -8 * ref.abs().max().item()
    assert_attn_close(out.float(), ref, "e4m3 bf16 out", max_abs=bound, rel_l2=2e-3 + 2.0 ** -8)
    h = set()
    for _ in range(3):
        o = gpu_attn(case, idx=gidx, num_splits=1)
        h.add(hashlib.sha256(o.cpu().numpy().tobytes()).hexdigest())
    assert len(h) == 1
    assert sap.sparse_attn_num_splits(case.T, 64, 512, gidx.shape[1], 1) == 1


# ------------------------------------------------- split-K decode, e4m3 rows

@pytest.mark.parametrize("B", [1, 8])
@pytest.mark.parametrize("ratio", [4, 128, 0])
def test_e4m3_decode_splits(B, ratio):
    """The decode kernel with e4m3 rows (raw codes gathered two rows per
    DMA, K widened to bf16 in registers, V^T by ds_read_b64_tr_b8 widened to
    f16, the weights as two f16 terms) over the automatic split count and
    forced ones; the merge combines the splits' (max, sum) in the same
    shifted log2 units."""
    need_gpu()
    case = W.decode_case(B=B, ratio=ratio, kv_dtype="e4m3", seed=W.SEED_BASE + 180 + 10 * B + ratio)
    idx = oracle.case_idx(case)
    ref = oracle.case_attn(case, idx=idx)
    gidx = gpu_idx(case)
    for splits in (0, 2, 5):
        runs = sap.sparse_attn_num_splits(case.T, 64, 512, idx.shape[1], splits)
        assert_attn_close(gpu_attn(case, idx=gidx, num_splits=splits), ref, f"e4m3 B{B} r{ratio} splits={splits} ({runs})")


@pytest.mark.parametrize("H", [20, 1])
def test_e4m3_decode_head_counts(H):
    # partial head groups through the split-K decode kernel (rows past H
    # read a stand-in q row and write nothing)
    need_gpu()
    case = W.decode_case(B=2, pos=4000, ratio=4, H=H, kv_dtype="e4m3", seed=W.SEED_BASE + 195 + H)
    assert_attn_close(gpu_attn(case), oracle.case_attn(case), f"e4m3 H={H} auto splits")


def test_e4m3_decode_holes_and_scales():
    # unused columns (a token without any, window only, compressed only with
    # a hole) and zero / negative scales, through the split-K decode path
    need_gpu()
    base = W.decode_case(B=4, pos=2000, ratio=4, topk=300, kv_dtype="e4m3", seed=W.SEED_BASE + 190)
    g = torch.Generator().manual_seed(191)

    def mix(s):
        r = torch.rand(s.shape, generator=g)
        s[r < 0.2] = 0.0
        s[(r >= 0.2) & (r < 0.5)] *= -1.0
        return s

    case = _with_scales(base, mix, mix)
    idx = oracle.case_idx(case)
    idx[1, :] = -1
    idx[2, case.n_win:] = -1
    idx[3, :case.n_win] = -1
    idx[3, case.n_win + 5:case.n_win + 40] = -1
    ref = oracle.case_attn(case, idx=idx)
    for splits in (0, 3):
        out = gpu_attn(case, idx=dev(idx), num_splits=splits)
        assert (out[1] == 0).all()
        assert_attn_close(out, ref, f"e4m3 decode holes splits={splits}")
