"""Pins of the oracle's number formats against sources other than itself.

- e4m3: torch's own float8_e4m3fn conversion, OCP spec points, and the
  "scaled16" facts of 'Perf/kv fp8 read path' (What this changes).
- e2m1 / ue8m0: the bit construction described in 'perf(kernel): read dsv41
  indexer key rows as int32 words' (Changes; Correctness and tests), evaluated
  here with numpy float32 arithmetic, torch's float8_e8m0fnu dtype, and the
  OCP MX points.
- bf16 rounding: torch's float32 -> bfloat16 conversion (ties to even).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _same(a, b):
    if isinstance(b, str) and b == "nan":
        return math.isnan(a)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


def test_e4m3_matches_torch_float8_for_all_codes():
    tab = oracle.e4m3_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        if math.isnan(ref[c]):
            assert math.isnan(tab[c]), hex(c)
        else:
            assert tab[c] == ref[c] and math.copysign(1, tab[c]) == math.copysign(1, ref[c]), hex(c)


def test_e4m3_ocp_points():
    g = _load("e4m3_ocp_points.json")
    tab = oracle.e4m3_table()
    for code, val in g["points"]:
        assert _same(tab[int(code, 16)], val), code


def test_e4m3_scaled16_facts():
    # After dividing by 2^8 every finite e4m3 value has |x| <= 1.75 and carries
    # at most 4 significant bits (implicit bit + 3 mantissa bits).
    tab = oracle.e4m3_table()
    finite = [v for v in tab if not math.isnan(v)]
    assert len(finite) == 254
    assert len(set(abs(v) for v in finite)) == 127
    for v in finite:
        x = v / 256.0
        assert abs(x) <= 1.75
        if x != 0:
            m, _ = math.frexp(abs(x))
            assert (m * 16).is_integer()          # <= 4 significant bits
    assert max(finite) == 448.0 and min(abs(v) for v in finite if v) == 2.0 ** -9


def test_e2m1_points_and_page_construction():
    g = _load("e2m1_points.json")
    for code, val in g["points"]:
        assert _same(oracle.e2m1(code), val), code
    # The page's decode: place (c & 7) << 22 in an fp32 bit pattern and
    # multiply by 2^126 (code 1 goes through an fp32 subnormal).
    for c in range(16):
        bits = np.array([(c & 7) << 22], dtype=np.uint32)
        mag = bits.view(np.float32)[0] * np.float32(2.0 ** 126)
        val = -float(mag) if c & 8 else float(mag)
        assert _same(oracle.e2m1(c), val), c


def test_ue8m0_matches_torch_e8m0():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for e in range(256):
        if math.isnan(ref[e]):
            assert math.isnan(oracle.ue8m0(e))
        else:
            assert oracle.ue8m0(e) == ref[e], e
    for e, val in _load("e2m1_points.json")["ue8m0"]:
        assert _same(oracle.ue8m0(e), val), e


def test_bf16_rounding_matches_torch():
    g = torch.Generator().manual_seed(7)
    xs = torch.cat([
        torch.randn(20000, generator=g) * torch.exp2(torch.randint(-140, 128, (20000,), generator=g).float()),
        # exact ties: halfway between adjacent bf16 values
        (torch.randint(0, 2 ** 16, (4000,), generator=g).to(torch.int32) << 16 | 0x8000).view(torch.float32),
        torch.tensor([0.0, -0.0, float("inf"), -float("inf"), 3.3895e38, 3.4e38, 1e-45, -1e-40]),
    ]).to(torch.float32)
    xs = xs[torch.isfinite(xs) | torch.isinf(xs)]
    ref = xs.to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    for x, r in zip(xs.tolist(), ref.tolist()):
        assert oracle.to_bf16_bits(x) == r, (x, hex(r))


def test_fp4_table_matches_torch_composition():
    tab = oracle.fp4_table()                                         # [256, 256, 2]
    # independent route: e2m1 magnitudes from the page's float32 construction,
    # scales from torch's float8_e8m0fnu, product rounded by torch to bf16
    nib = np.arange(16, dtype=np.uint32)
    mag = ((nib & 7) << 22).view(np.float32).astype(np.float64) * 2.0 ** 126
    e2m1 = np.where(nib & 8, -mag, mag)
    sc = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64)
    codes = torch.arange(256)
    for j, sel in enumerate([codes & 0xF, codes >> 4]):
        v = torch.from_numpy(e2m1)[sel].unsqueeze(1) * sc.unsqueeze(0)    # [256 code, 256 scale]
        bits = v.to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
        got = tab[:, :, j]
        nan_ref = torch.isnan(v).numpy()
        assert (got[nan_ref] & 0x7FFF > 0x7F80).all()               # NaN stays NaN
        assert np.array_equal(got[~nan_ref], bits[~nan_ref])
    # code 0x8 (negative zero) keeps its sign for every finite scale
    assert (tab[0x08, :255, 0] == 0x8000).all() and (tab[0x80, :255, 1] == 0x8000).all()


def test_fp4_row_element_layout():
    # element 2i is the low nibble of byte i; block b of 32 uses scale byte b
    row = torch.zeros(17, dtype=torch.int32)
    row[0] = 0x00000072           # d0 = code 2 (1.0), d1 = code 7 (6.0)
    row[3] = 0x50000000           # d31 = code 5 (3.0)
    row[4] = 0x0000000F           # d32 = code 15 (-6.0)
    row[16] = 0x7F81807E          # scales: b0 = 126, b1 = 128, b2 = 129, b3 = 127
    v = oracle.fp4_rows_decode(row.view(1, 17))[0]
    assert v[0] == 0.5 and v[1] == 3.0 and v[31] == 1.5 and v[32] == -12.0
    assert v[2] == 0.0 and not math.copysign(1, v[2]) < 0
