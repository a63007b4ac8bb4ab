"""Run one named workload a few times on cuda:0, for rocprofv3 trace and
counter runs (the counter runs need a program that launches only the kernel
being measured).

Usage: python -m sparse_attention_paged_amd.profile_run WORKLOAD [REPS]

  prefill      sparse attention, 8192 query tokens from position 0, r = 4,
               one pass per token (64 heads, head_dim 512, bf16 pools, fp32 out)
  decode_attn  split-K sparse attention + merge, one sequence at position
               32767, r = 4 (the decode step's attention call)
  copy         a plain 1 GiB device-to-device copy: the calibration for the
               FETCH_SIZE / WRITE_SIZE counters
"""
from __future__ import annotations

import math
import sys

import torch

import workloads as W

from . import api as sap


def prefill(reps: int) -> None:
    case = W.prefill_case(T=8192, ratio=4)
    d = torch.device("cuda")
    q, win, cmp = case.q.to(d), case.win_pool.to(d), case.cmp_pool.to(d)
    idx = sap.build_sparse_idx(case.pos.to(d), case.seq.to(d), case.n_win, case.win_pt.to(d), case.page,
                               case.cmp_logical.to(d), case.cmp_pt.to(d))
    out = torch.empty((case.T, 64, 512), dtype=torch.float32, device=d)
    torch.cuda.synchronize()
    for _ in range(reps):
        sap.sparse_attn_paged(q, win, cmp, idx, case.n_win, case.sm_scale, out=out, num_splits=1)
    torch.cuda.synchronize()


def decode_attn(reps: int) -> None:
    c = W.decode_case(B=1, pos=32767, ratio=4, seed=W.SEED_BASE + 2)
    d = torch.device("cuda")
    idx = sap.build_sparse_idx(c.pos.to(d), c.seq.to(d), c.n_win, c.win_pt.to(d), c.page,
                               c.cmp_logical.to(d), c.cmp_pt.to(d))
    q, win, cmp = c.q.to(d), c.win_pool.to(d), c.cmp_pool.to(d)
    out = torch.empty((1, 64, 512), dtype=torch.float32, device=d)
    n_cols = c.n_win + c.n_cmp
    ws = torch.empty(max(sap.sparse_attn_workspace_bytes(1, 64, 512, n_cols, 0), 1), dtype=torch.uint8, device=d)
    torch.cuda.synchronize()
    for _ in range(reps):
        sap.sparse_attn_paged(q, win, cmp, idx, c.n_win, c.sm_scale, out=out, workspace=ws)
    torch.cuda.synchronize()


def copy(reps: int) -> None:
    a = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()


def main(argv) -> None:
    if len(argv) < 1 or argv[0] not in ("prefill", "decode_attn", "copy"):
        print(__doc__, file=sys.stderr)
        sys.exit(2)
    reps = int(argv[1]) if len(argv) > 1 else 3
    torch.cuda.set_device(0)
    {"prefill": prefill, "decode_attn": decode_attn, "copy": copy}[argv[0]](reps)
    print(f"{argv[0]}: {reps} runs done", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:])
