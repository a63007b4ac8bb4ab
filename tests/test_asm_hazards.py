"""The bf16 prefill kernel issues its MFMAs from inline assembly (to pin O and
Q to AGPRs), so the compiler's hazard tracking does not see them: a vector
write that the compiler places just before such an MFMA, into a register the
MFMA reads, would get none of the wait states the hardware needs between the
two, and the MFMA could read the register's old value.  This test compiles
the kernel to gfx950 assembly (on the CPU) and checks that no register
written by a VALU or AGPR-write instruction is read by an MFMA within a few
instructions after the write.  It also checks the order of vector memory
instructions that the kernel's hand-counted vmcnt waits rely on, and that m0
(which the row-gather assembly sets) is used by nothing else.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_paged_amd", "csrc")

# Wait states (issued instructions, s_nop N counting N + 1) that must lie
# between a write and an MFMA reading the written register.  The hardware
# needs a few; the kernel keeps far more between every write it makes and
# the MFMAs, so any compiler-placed write shows up here.
AGPR_MIN = 8
VGPR_MIN = 4


def _regs(op: str, kind: str) -> set:
    op = op.strip()
    m = re.match(kind + r"\[(\d+):(\d+)\]$", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(kind + r"(\d+)$", op)
    return {int(m.group(1))} if m else set()


def _hazards(lines):
    """(write line, mfma line, distance) for each write read too soon by an MFMA."""
    code = [l.split(";")[0].strip() for l in lines]
    found = []
    for i, t in enumerate(code):
        if not t.startswith("v_") or t.startswith(("v_mfma", "v_cmp", "v_readlane", "v_readfirstlane")):
            continue
        parts = t.split(None, 1)
        if len(parts) < 2:
            continue
        dst = parts[1].split(",")[0]
        agpr = _regs(dst, "a")
        vgpr = _regs(dst, "v")
        if not agpr and not vgpr:
            continue
        n = 0
        for j in range(i + 1, min(len(code), i + 40)):
            u = code[j]
            if not u or u.startswith("."):
                continue
            if u.startswith("s_nop"):
                n += int(u.split()[1]) + 1
                continue
            n += 1
            if n >= max(AGPR_MIN, VGPR_MIN):
                break
            if u.startswith("v_mfma"):
                ops = [o.strip() for o in u.split(None, 1)[1].split(",")]
                srcs = set()
                if agpr:
                    srcs = set().union(*(_regs(o, "a") for o in ops[1:])) & agpr
                    if srcs and n < AGPR_MIN:
                        found.append((t, u, n))
                if vgpr:
                    srcs = set().union(*(_regs(o, "v") for o in ops[1:])) & vgpr
                    if srcs and n < VGPR_MIN:
                        found.append((t, u, n))
    return found


def test_hazard_scan_catches_a_planted_case():
    """The scan itself: an AGPR write right before an MFMA that accumulates
    into it, and a VGPR write right before an MFMA that reads it, are found;
    the same pairs with enough wait states between them are not."""
    bad = ["v_accvgpr_write_b32 a5, v7",
           "v_mfma_f32_16x16x32_bf16 a[4:7], v[0:3], v[8:11], a[4:7]",
           "v_add_f32_e32 v9, v1, v2",
           "v_mfma_f32_16x16x32_bf16 a[12:15], v[0:3], v[8:11], a[12:15]"]
    assert len(_hazards(bad)) == 2
    good = ["v_accvgpr_write_b32 a5, v7", "s_nop 7",
            "v_mfma_f32_16x16x32_bf16 a[4:7], v[0:3], v[8:11], a[4:7]",
            "v_add_f32_e32 v9, v1, v2", "s_nop 3",
            "v_mfma_f32_16x16x32_bf16 a[12:15], v[0:3], v[8:11], a[12:15]"]
    assert _hazards(good) == []


def test_prefill_kernel_has_no_write_next_to_an_asm_mfma(tmp_path):
    lines = _compile(tmp_path, "attn_d512")
    n_mfma = sum(1 for l in lines if l.strip().startswith("v_mfma"))
    assert n_mfma > 100, "the kernel's MFMAs were not found in the assembly"
    found = _hazards(lines)
    assert not found, f"{len(found)} writes too close to an MFMA, e.g. {found[:3]}"


def _early_reads(lines):
    """Loads issued from inline assembly with no compiler tracking
    ("global_load_dword vN, vaddr, off"): their destination must not be read or
    written before an s_waitcnt vmcnt(0) (the kernel ties the values to such a
    wait); a compiler copy of the register before that would copy the old
    value."""
    code = [l.split(";")[0].strip() for l in lines]
    found = []
    for i, t in enumerate(code):
        if not (t.startswith("global_load_dword ") and t.endswith(", off")):
            continue
        dst = _regs(t.split(None, 1)[1].split(",")[0], "v")
        for j in range(i + 1, len(code)):
            u = code[j]
            if not u or u.startswith("."):
                continue
            if u.startswith("s_waitcnt") and "vmcnt(0)" in u:
                break
            parts = u.split(None, 1)
            if len(parts) == 2 and set().union(*(_regs(o, "v") for o in parts[1].split(","))) & dst:
                found.append((t, u))
                break
    return found


def test_untracked_loads_untouched_until_waited(tmp_path):
    assert len(_early_reads(["global_load_dword v4, v[2:3], off", "v_mov_b32_e32 v9, v4",
                             "s_waitcnt vmcnt(0)"])) == 1
    assert _early_reads(["global_load_dword v4, v[2:3], off", "s_waitcnt vmcnt(0)",
                         "v_mov_b32_e32 v9, v4"]) == []
    lines = _compile(tmp_path, "attn_d512")
    assert sum(1 for l in lines if l.strip().startswith("global_load_dword ") and l.strip().endswith(", off")) >= 4
    found = _early_reads(lines)
    assert not found, f"{len(found)} untracked load results used before their wait, e.g. {found[:3]}"


_VM = ("global_", "buffer_", "flat_", "scratch_")


_ASM = {}


def _compile(tmp_path, name):
    """gfx950 assembly of csrc/<name>.hip (compiled once per test session)."""
    if name in _ASM:
        return _ASM[name]
    hipcc = next((c for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc"))
                  if c and os.path.exists(c)), None)
    if hipcc is None:
        pytest.skip("hipcc not available")
    out = tmp_path / f"{name}.s"
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           os.path.join(CSRC, f"{name}.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    _ASM[name] = out.read_text().splitlines()
    return _ASM[name]


def _kernels(lines, stem):
    """{symbol: [instructions]} of every kernel whose name contains stem."""
    out, cur = {}, None
    for l in lines:
        m = re.match(r"^(_Z\S+):", l)
        if m:
            cur = m.group(1) if stem in m.group(1) else None
            if cur:
                out[cur] = []
            continue
        if cur and l.startswith(".Lfunc_end"):
            cur = None
            continue
        if cur:
            t = l.split(";")[0].strip()
            if t and not t.startswith(".") and not t.endswith(":"):
                out[cur].append(t)
    return out


def test_prefill_token_switch_wait_counts(tmp_path):
    """The prefill kernel waits for the next token's first tiles with
    hand-counted vmcnt values that assume exactly this order of vector memory
    instructions at a token switch: the gathers of tiles 0 and 1 (bf16 rows:
    8 row DMAs per wave and tile; e4m3 rows: 4 DMAs of two rows each, then
    the rows' scales), then the previous token's 32 output stores (8 m-steps
    x 4 head blocks), then the next token's index loads.  Fewer or merged
    stores would let a wait pass before its tile has landed, so the order and
    the count are checked here."""
    kern = _kernels(_compile(tmp_path, "attn_d512"), "attn_d512_kernel")
    assert len(kern) == 4, list(kern)
    for name, code in kern.items():
        e4 = "Lb1E" in name   # attn_d512_kernel<OUT, E4 = true>
        vm = [t for t in code if t.startswith(_VM)]
        first_store = next(i for i, t in enumerate(vm) if t.startswith("global_store"))
        if e4:
            before = vm[first_store - 10:first_store]
            tile = ["global_load_lds_dwordx4"] * 4 + ["global_load_lds_dword"]
            assert [t.split()[0] for t in before] == tile * 2, (name, before)
        else:
            before = vm[first_store - 16:first_store]
            assert all(t.startswith("global_load_lds_dwordx4") for t in before), (name, before)
        run = 0
        for t in vm[first_store:]:
            if not t.startswith("global_store"):
                break
            run += 1
        assert run == 32, f"{name}: {run} consecutive output stores after the token-switch DMAs, expected 32"
        assert sum(1 for t in vm if t.startswith("global_store")) == 32, name


def test_m0_written_only_by_the_row_gathers(tmp_path):
    """The row (and row-scale) gathers set m0 (the LDS address of global_load_lds) from inline
    assembly, which the compiler does not preserve around: no compiler-placed
    instruction may read or write m0 in these kernels (indirect register
    indexing, s_sendmsg and the like would)."""
    for name in ("attn_d512", "attn_dec", "attn"):
        lines = _compile(tmp_path, name)
        code = [l.split(";")[0].strip() for l in lines]
        bad = []
        for i, t in enumerate(code):
            if not re.search(r"\bm0\b", t):
                continue
            if t.startswith("s_mov_b32 m0, s"):
                nxt = [u for u in code[i + 1:i + 4] if u and not u.startswith("s_nop")]
                if nxt and nxt[0].startswith(("global_load_lds_dwordx4", "global_load_lds_dword ")):
                    continue
            bad.append(t)
        assert not bad, f"{name}: m0 used outside the row-gather assembly: {bad[:3]}"
        assert not any(t.startswith(("s_set_gpr_idx", "v_movrel", "s_movrel")) for t in code), name
