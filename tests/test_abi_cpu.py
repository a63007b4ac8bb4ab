"""Host-side checks of the C-ABI library with no GPU: it loads, exports every
entry point include/sap.h declares, and rejects bad arguments before any HIP
call (the wrapper asserts of 'perf(kernel): keep 16-byte kv loads in dsv4
sparse attention and unroll gated pool', Changes: 16-byte aligned pools, and
'perf(kernel): read dsv41 indexer key rows as int32 words', Changes: a 4-byte
aligned key pool, become error codes).  Only invalid calls are made, so no
kernel is ever launched here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sap.h")

sap_lib = pytest.importorskip("sparse_attention_paged_amd._lib")

OK, ENULL, EALIGN, ESHAPE, EDTYPE, EWS, ESCRATCH = 0, -1, -2, -3, -4, -5, -7
BF16, F32, FP8 = 0, 1, 2
A = 0x10000          # a fake, 16-byte aligned "device" address; never dereferenced


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(sap_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(sap_lib.LIB_PATH):
        pytest.fail("libsap.so is not built; run python -m sparse_attention_paged_amd.build")
    return sap_lib.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(sap_lib.SIGNATURES), "binding and header disagree"
    assert L.sap_version() == 100
    assert sap_lib.status_string(-2).startswith("a base address")


def _attn(L, **kw):
    a = dict(q=A, q_dtype=BF16, q_st=64 * 512, q_sh=512, win=A, win_rs=1024, cmp=A, cmp_rs=1024,
             kv=BF16, idx=A, idx_st=640, n_win=128, n_cmp=512, ws_=None, cs_=None, out=A, od=F32,
             out_st=64 * 512, out_sh=512, T=1, H=64, D=512, sm=0.04, splits=1, ws=None, wsb=0)
    a.update(kw)
    return L.sap_sparse_attn_paged(a["q"], a["q_dtype"], a["q_st"], a["q_sh"], a["win"], a["win_rs"],
                                   a["cmp"], a["cmp_rs"], a["kv"], a["idx"], a["idx_st"], a["n_win"],
                                   a["n_cmp"], a["ws_"], a["cs_"], a["out"], a["od"], a["out_st"],
                                   a["out_sh"], a["T"], a["H"], a["D"], a["sm"], a["splits"], a["ws"],
                                   a["wsb"], None)


def test_attention_argument_checks(L):
    assert _attn(L, T=0) == OK                               # nothing to do, nothing launched
    assert _attn(L, win=A + 8) == EALIGN                      # misaligned pool base
    assert _attn(L, cmp=A + 4) == EALIGN
    assert _attn(L, win_rs=1032) == EALIGN                    # row stride not a multiple of 16
    assert _attn(L, q=A + 2) == EALIGN
    assert _attn(L, out=A + 4) == EALIGN
    assert _attn(L, q_sh=500) == EALIGN
    assert _attn(L, win=None) == ENULL
    assert _attn(L, cmp=None) == ENULL
    assert _attn(L, idx=None) == ENULL
    assert _attn(L, kv=FP8) == ENULL                          # e4m3 needs scales
    assert _attn(L, kv=F32) == EDTYPE
    assert _attn(L, q_dtype=F32) == EDTYPE
    assert _attn(L, od=FP8) == EDTYPE
    assert _attn(L, D=100) == ESHAPE
    assert _attn(L, H=0) == ESHAPE
    assert _attn(L, idx_st=600) == ESHAPE                     # fewer than n_win + n_cmp columns
    assert _attn(L, n_win=60000, n_cmp=6000, idx_st=70000) == ESHAPE
    assert _attn(L, win_rs=512) == ESHAPE                     # rows shorter than D elements
    assert _attn(L, splits=4) == EWS                          # split-K needs a workspace
    need = L.sap_sparse_attn_workspace_bytes(1, 64, 512, 640, 4)
    # 4 splits requested over 5 rounds of 128 columns: 3 splits of 2 rounds,
    # partial O of 64 heads + (max, sum) per head, each 256-aligned
    assert need == 3 * 64 * 512 * 4 + 3 * 64 * 2 * 4
    assert _attn(L, splits=4, ws=A, wsb=need - 1) == EWS
    assert _attn(L, splits=4, ws=A + 16, wsb=need) == EWS     # workspace must be 256-byte aligned


def test_noalloc_argument_checks(L):
    """The allocation-free entry point validates like sap_sparse_attn_paged
    and refuses a plan larger than its fixed scratch before any HIP call."""
    def call(**kw):
        a = dict(q=A, q_dtype=BF16, q_st=64 * 512, q_sh=512, win=A, win_rs=1024, cmp=A, cmp_rs=1024,
                 kv=BF16, idx=A, idx_st=640, n_win=128, n_cmp=512, ws_=None, cs_=None, out=A, od=F32,
                 out_st=64 * 512, out_sh=512, T=1, H=64, D=512, sm=0.04, splits=1)
        a.update(kw)
        return L.sap_sparse_attn_paged_noalloc(a["q"], a["q_dtype"], a["q_st"], a["q_sh"], a["win"], a["win_rs"],
                                               a["cmp"], a["cmp_rs"], a["kv"], a["idx"], a["idx_st"], a["n_win"],
                                               a["n_cmp"], a["ws_"], a["cs_"], a["out"], a["od"], a["out_st"],
                                               a["out_sh"], a["T"], a["H"], a["D"], a["sm"], a["splits"], None)
    mx = L.sap_sparse_attn_noalloc_max_bytes()
    assert mx == 32 << 20
    assert call(T=0) == OK
    assert call(win=A + 8) == EALIGN
    assert call(idx=None) == ENULL
    assert call(kv=F32) == EDTYPE
    assert call(D=100) == ESHAPE
    # an explicit split count whose partials exceed the fixed array
    assert L.sap_sparse_attn_workspace_bytes(128, 64, 512, 640, 20) > mx
    assert call(T=128, splits=20) == ESCRATCH
    assert "allocation-free" in sap_lib.status_string(ESCRATCH)
    # the automatic plan fits at every batch size and column count for D <= 512
    for H in (1, 20, 64, 128):
        for C in (1, 128, 384, 640, 1472, 4096):
            for T in list(range(1, 140)) + [256, 8192]:
                assert L.sap_sparse_attn_workspace_bytes(T, H, 512, C, 0) <= mx, (H, C, T)


def test_split_planning(L):
    ns = L.sap_sparse_attn_num_splits
    # head_dim 512: the decode kernel splits a token's columns in rounds of 128
    assert ns(8192, 64, 512, 640, 0) == 1            # prefill: one pass per token
    assert ns(128, 64, 512, 640, 0) == 1             # a batch that fills the GPU: one pass per token
    assert ns(1, 64, 512, 640, 0) == 5               # decode B1: one round per split
    assert ns(8, 64, 512, 640, 0) == 5               # B8: 160 workgroups
    assert ns(1, 64, 512, 384, 0) == 3
    assert ns(1, 64, 512, 128, 0) == 1               # window only: one split, no merge
    assert ns(1, 64, 512, 40, 0) == 1
    assert ns(16, 64, 512, 640, 0) == 3              # 192 workgroups of 2 rounds: every one resident
    assert ns(32, 64, 512, 640, 0) == 2              # 256 workgroups: 2 splits of 3 rounds
    assert ns(64, 64, 512, 640, 0) == 1              # 256 workgroups of 5 rounds, no merge
    assert ns(1, 64, 512, 32 * 40, 0) == 10
    assert ns(1, 64, 512, 640, 7) == 5               # never more splits than rounds
    assert ns(1, 64, 512, 640, 4) == 3               # 4 requested: 2 rounds each
    assert ns(1, 64, 512, 0, 0) == 1
    assert L.sap_sparse_attn_workspace_bytes(8192, 64, 512, 640, 0) == 0
    assert L.sap_sparse_attn_workspace_bytes(1, 64, 512, 128, 0) == 0
    # other head_dims: 32-column tiles per split, the launch within about 128 workgroups
    assert ns(1, 64, 128, 640, 0) == 20
    assert ns(8, 64, 128, 640, 0) == 10
    assert ns(1, 64, 128, 640, 100) == 20            # never more splits than tiles
    assert ns(8192, 64, 256, 640, 0) == 1


def test_indexer_argument_checks(L):
    def call(**kw):
        a = dict(q=A, qsb=32 * 128, w=A, wsb=32, pool=A, rw=17, pt=A, ptsb=2048, page=64, nk=None,
                 out=A, osb=131072, B=1, Hi=32, D=128, N=131072)
        a.update(kw)
        return L.sap_indexer_logits_packed(a["q"], a["qsb"], a["w"], a["wsb"], a["pool"], a["rw"],
                                           a["pt"], a["ptsb"], a["page"], a["nk"], a["out"], a["osb"],
                                           a["B"], a["Hi"], a["D"], a["N"], None)
    assert call(B=0) == OK
    assert call(pool=A + 2) == EALIGN                 # key pool must be 4-byte aligned
    assert call(q=A + 8) == EALIGN
    assert call(Hi=33) == ESHAPE
    assert call(D=64) == ESHAPE
    assert call(rw=16) == ESHAPE
    assert call(page=0) == ESHAPE
    assert call(osb=100) == ESHAPE
    assert call(w=None) == ENULL


def test_topk_argument_checks(L):
    ws = L.sap_topk_workspace_bytes
    assert ws(1, 4096, 512) == 0                      # rows of <= 16384 entries: one launch, no workspace
    assert ws(2, 16384, 512) == 0
    assert ws(4, 131072, 512) > ws(1, 131072, 512) > 0  # longer rows: per-chunk candidate slots

    def call(**kw):
        a = dict(x=A, sb=131072, nv=None, B=1, N=131072, k=512, out=A, osb=512, ws=None, wsb=0)
        a.update(kw)
        return L.sap_topk_select(a["x"], a["sb"], a["nv"], a["B"], a["N"], a["k"], a["out"], a["osb"],
                                 a["ws"], a["wsb"], None)
    assert call(B=0) == OK
    assert call(k=0) == ESHAPE
    assert call(k=5000) == ESHAPE
    assert call(osb=100) == ESHAPE
    assert call(out=None) == ENULL
    assert call(x=None) == ENULL
    assert call(sb=100) == ESHAPE
    assert call() == EWS                       # 131072 entries need the slots
    assert call(ws=A, wsb=ws(1, 131072, 512) - 1) == EWS


def test_index_build_argument_checks(L):
    f = L.sap_build_sparse_idx
    assert f(A, A, 4, 128, A, 512, 0, A, 512, 512, A, 128, A, 640, None) == ESHAPE     # page 0
    assert f(A, A, 4, 128, A, 512, 64, None, 512, 512, A, 128, A, 640, None) == ENULL
    assert f(A, A, 4, 128, A, 512, 64, A, 512, 512, A, 128, A, 600, None) == ESHAPE    # idx too narrow
    assert f(A, A, 0, 128, A, 512, 64, A, 512, 512, A, 128, A, 640, None) == OK
