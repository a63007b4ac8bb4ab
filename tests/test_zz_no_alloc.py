"""The allocation-free sparse attention entry point (split partials in the
library's fixed device array, no workspace argument) against the entry point
with a caller's workspace: identical bits on the same inputs, and the parity
bar against the oracle, on two calls in a row, the second with a smaller
input (the array keeps the first call's partials)."""
import pytest
import torch

import oracle
import sparse_attention_paged_amd as sap
import workloads as W
from gpu_helpers import assert_attn_close, dev, gpu_idx, need_gpu, say

pytestmark = pytest.mark.gpu


def _both(case, num_splits=0):
    idx = gpu_idx(case)
    q, wp, cp = dev(case.q), dev(case.win_pool), dev(case.cmp_pool)
    ws_, cs_ = dev(case.win_scale), dev(case.cmp_scale)
    ref_out = sap.sparse_attn_paged(q, wp, cp, idx, case.n_win, case.sm_scale, win_scale=ws_, cmp_scale=cs_,
                                    num_splits=num_splits)
    out = torch.full_like(ref_out, float("nan"))
    sap.sparse_attn_paged_noalloc(q, wp, cp, idx, case.n_win, case.sm_scale, out=out, win_scale=ws_,
                                  cmp_scale=cs_, num_splits=num_splits)
    torch.cuda.synchronize()
    return idx, ref_out, out


def test_noalloc_matches_workspace_entry_point():
    need_gpu()
    big = W.decode_case(B=8, ratio=4, seed=W.SEED_BASE + 160)
    small = W.decode_case(B=2, pos=3000, ratio=4, topk=200, seed=W.SEED_BASE + 161)
    for case in (big, small):
        splits = sap.sparse_attn_num_splits(case.T, 64, 512, case.n_win + case.n_cmp, 0)
        say(f"  {case.name}: {splits} splits through the fixed scratch array")
        idx, ref_out, out = _both(case)
        assert splits > 1
        assert torch.equal(out, ref_out), f"{case.name}: differs from the workspace entry point"
        assert_attn_close(out, oracle.case_attn(case, idx=idx.cpu()), f"{case.name} no-alloc vs oracle")


def test_noalloc_fp8_and_explicit_splits():
    need_gpu()
    case = W.decode_case(B=2, pos=2000, ratio=4, topk=300, kv_dtype="e4m3", seed=W.SEED_BASE + 162)
    for splits in (5, 1):
        idx, ref_out, out = _both(case, num_splits=splits)
        assert torch.equal(out, ref_out), f"e4m3 splits={splits}"
        assert_attn_close(out, oracle.case_attn(case, idx=idx.cpu()), f"e4m3 splits={splits} no-alloc")
