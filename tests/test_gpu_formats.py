"""Bit-exact checks of the device row decoders over every code
('Perf/kv fp8 read path', Tests: all 256 e4m3 codes; 'perf(kernel): read
dsv41 indexer key rows as int32 words', Correctness and tests: every code
byte against every scale byte)."""
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_paged_amd as sap
from gpu_helpers import need_gpu, say

pytestmark = pytest.mark.gpu


def test_e4m3_loader_table_bit_exact():
    need_gpu()
    bits, fold = sap.debug_e4m3_table()
    torch.cuda.synchronize()
    bits = bits.cpu().numpy().astype(np.uint16)
    f = float(fold.cpu()[0])
    ref = oracle.e4m3_table()
    vals = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64) * f
    for c in range(256):
        got = float(vals[c])
        if math.isnan(ref[c]):
            assert math.isnan(got), hex(c)          # the two NaN codes stay NaN
        else:
            assert got == ref[c] and math.copysign(1, got) == math.copysign(1, ref[c]), (hex(c), got, ref[c])
    say(f"  e4m3: 254 finite codes exact, fold factor {f}")


def test_e4m3_f16_loader_table_bit_exact():
    """The one-pass kernel at head_dim 512 widens V^T to f16: every finite
    e4m3 value (4 significant bits, |x| in [2^-9, 448]) is exactly an f16."""
    need_gpu()
    bits = sap.debug_e4m3_f16_table()
    torch.cuda.synchronize()
    vals = bits.cpu().numpy().astype(np.uint16).view(np.float16).astype(np.float64)
    ref = oracle.e4m3_table()
    for c in range(256):
        got = float(vals[c])
        if math.isnan(ref[c]):
            assert math.isnan(got), hex(c)
        else:
            assert got == ref[c] and math.copysign(1, got) == math.copysign(1, ref[c]), (hex(c), got, ref[c])
    say("  e4m3 -> f16: 254 finite codes exact")


def test_fp4_loader_table_bit_exact():
    need_gpu()
    got = sap.debug_fp4_table().cpu().numpy().astype(np.uint16)      # [code, scale, nibble]
    ref = oracle.fp4_table()
    nan_ref = (ref & 0x7FFF) > 0x7F80
    nan_got = (got & 0x7FFF) > 0x7F80
    assert np.array_equal(nan_ref, nan_got)
    mism = np.argwhere((got != ref) & ~nan_ref)
    assert mism.size == 0, f"{len(mism)} mismatches, first {mism[:5].tolist()}"
    say("  fp4: 256 x 256 x 2 entries exact")
