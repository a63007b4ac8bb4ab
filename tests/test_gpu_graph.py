"""A decode step captured in a HIP graph gives, on every replay, the bits of
the same step launched eagerly (the graph holds only the library's kernels:
no memset nodes).  Replays are interleaved with eager work and host syncs."""
import pytest
import torch

import sparse_attention_paged_amd as sap
import workloads as W
from gpu_helpers import dev, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fused,kv", [(False, "bf16"), (True, "bf16"), (True, "e4m3")])
def test_decode_step_graph_replays_match_eager(fused, kv):
    """fused: the selection runs as one top-k + index build launch; kv: the
    attention pools' row format (e4m3 with per-row scales)."""
    need_gpu()
    c = W.decode_case(B=2, pos=4095, ratio=4, kv_dtype=kv, seed=W.SEED_BASE + 900)
    g = W.make_generator(W.SEED_BASE + 901)
    n_c = (4095 + 1 + 3) // 4
    keys = dev(W.fp4_key_rows(c.cmp_pool.shape[0], g))
    qi = dev(torch.randn((2, 32, 128), generator=g).to(torch.bfloat16))
    wi = dev(torch.rand((2, 32), generator=g))
    nv = torch.full((2,), n_c, dtype=torch.int32, device="cuda")
    logits = torch.empty((2, n_c), dtype=torch.float32, device="cuda")
    sel = torch.empty((2, c.n_cmp), dtype=torch.int32, device="cuda")
    idx = torch.empty((2, c.n_win + c.n_cmp), dtype=torch.int32, device="cuda")
    out = torch.empty((2, 64, 512), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(sap.sparse_attn_workspace_bytes(2, 64, 512, c.n_win + c.n_cmp, 0), 1),
                     dtype=torch.uint8, device="cuda")
    q, win, cmp = dev(c.q), dev(c.win_pool), dev(c.cmp_pool)
    wsc, csc = dev(c.win_scale), dev(c.cmp_scale)
    pos, seq, win_pt, cmp_pt = dev(c.pos), dev(c.seq), dev(c.win_pt), dev(c.cmp_pt)

    def step():
        sap.indexer_logits_packed(qi, wi, keys, cmp_pt, c.page, n_c, n_keys=nv, out=logits)
        if fused:
            sap.topk_sparse_idx(logits, c.n_cmp, pos, seq, c.n_win, win_pt, cmp_pt, c.page, out=idx)
        else:
            sap.topk_select(logits, c.n_cmp, out=sel)
            sap.build_sparse_idx(pos, seq, c.n_win, win_pt, c.page, sel, cmp_pt, out=idx)
        sap.sparse_attn_paged(q, win, cmp, idx, c.n_win, c.sm_scale, out=out, win_scale=wsc, cmp_scale=csc,
                              workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (logits, sel, idx, out)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        for t in (logits, sel, idx, out):
            t.fill_(0) if t.dtype != torch.int32 else t.fill_(-7)     # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("logits", "top-k", "idx", "out"), (logits, sel, idx, out), ref):
            if fused and name == "top-k":
                continue   # the fused selection writes the index rows only
            assert torch.equal(a, b), f"replay {r}: {name} differs from the eager step"
        say(f"  replay {r}: identical to eager")
