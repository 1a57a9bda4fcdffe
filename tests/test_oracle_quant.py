"""Pins of the oracle's binary16 conversion and its q8_1 / Q8_0 quantizers (CPU only).

The q8_1 block (36 bytes: fp16 d, fp16 s, int8 q[32]) is the activation format named on
"#2058 Verify window: the routed experts' gate/up with the group's q8_1 rows in shared memory",
section "Why". Pins used here, none of which re-types the oracle's code:
  * numpy's float16 conversion (a library round-to-nearest-even routine) over every fp16 bit
    pattern, crafted ties, subnormals and the overflow edge;
  * hand-derived golden blocks (tests/golden/q8_1_blocks.json);
  * properties that hold for any input: the amax element maps to +-127, |x - d q| <= d/2,
    the s field equals fp16(f(d16) * sum q) computed from the stored bytes, d16 = fp16(amax/127);
  * Q8_0 round-trip idempotence (exact, see test_q8_0_roundtrip).
"""
import json
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _f16_bits(x):
    with np.errstate(over="ignore"):
        return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def test_h2f_all_patterns(orc):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float32)
    got = np.array([orc.h2f(int(p)) for p in pats], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f2h_matches_numpy(orc):
    g = np.random.default_rng(7)
    vals = [g.standard_normal(4000) * s for s in (1e-7, 1e-5, 1e-3, 1.0, 1e2, 1e4, 6e4)]
    vals = np.concatenate(vals).astype(np.float32)
    # exact midpoints between neighbouring fp16 values (ties), normal and subnormal
    h = np.arange(1, 0x7BFF, 37, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    ties = ((lo + hi) / 2).astype(np.float32)
    edges = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 1e9, 2.0 ** -24,
                      2.0 ** -25, 2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 6.1e-5, np.inf, -np.inf],
                     np.float32)
    allv = np.concatenate([vals, ties, -ties, edges])
    got = np.array([orc.f2h(float(v)) for v in allv], np.uint16)
    ref = _f16_bits(allv)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, [(float(allv[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]
    assert orc.f2h(float("nan")) & 0x7C00 == 0x7C00 and orc.f2h(float("nan")) & 0x3FF


def test_q8_1_golden(orc):
    doc = json.load(open(os.path.join(GOLD, "q8_1_blocks.json")))
    for blk in doc["blocks"]:
        out = orc.quantize_q8_1(np.array(blk["x"], np.float32))
        assert out.shape == (36,)
        d16 = int(out[0]) | int(out[1]) << 8
        s16 = int(out[2]) | int(out[3]) << 8
        q = out[4:].view(np.int8).astype(int).tolist()
        assert d16 == int(blk["d16"], 16), blk["name"]
        assert s16 == int(blk["s16"], 16), blk["name"]
        assert q == blk["q"], blk["name"]
        assert sum(q) == blk["isum"]


def _fields(out):
    b = out.reshape(-1, 36)
    d16 = b[:, 0:2].copy().view(np.uint16)[:, 0]
    s16 = b[:, 2:4].copy().view(np.uint16)[:, 0]
    q = b[:, 4:].view(np.int8).astype(np.int64)
    return d16, s16, q


@pytest.mark.parametrize("scale", [1.0, 1e-3, 40.0, 3e-6])
def test_q8_1_properties(orc, scale):
    g = np.random.default_rng(int(scale * 1e6) + 3)
    x = (g.standard_normal((64, 32 * 16)) * scale).astype(np.float32)
    out = orc.quantize_q8_1(x)
    d16, s16, q = _fields(out)
    xb = x.reshape(-1, 32)
    amax = np.abs(xb).max(axis=1)
    d = (amax / np.float32(127)).astype(np.float32)           # IEEE float32 division
    assert np.array_equal(d16, _f16_bits(d))
    # the largest-magnitude element maps to +-127, with its sign
    imax = np.abs(xb).argmax(axis=1)
    rows = np.arange(xb.shape[0])
    assert np.array_equal(q[rows, imax], np.where(xb[rows, imax] > 0, 127, -127))
    # nearest rounding: |x/d - q| <= 1/2 (checked in float64 on the float32 quotient)
    quot = (xb / d[:, None]).astype(np.float32).astype(np.float64)
    assert np.all(np.abs(quot - q) <= 0.5)
    # ties go away from zero: where the quotient is exactly k + 1/2, |q| = |k| + 1
    frac = np.abs(quot) - np.floor(np.abs(quot))
    tie = frac == 0.5
    assert np.all(np.abs(q[tie]) == np.floor(np.abs(quot[tie])) + 1)
    # s field = fp16(f(d16) * sum q), from the stored bytes and numpy's conversion
    s_ref = _f16_bits(d16.view(np.float16).astype(np.float32) * q.sum(axis=1).astype(np.float32))
    assert np.array_equal(s16, s_ref)
    # |s - d * sum q| within half an fp16 ulp of s plus the d16 rounding
    assert np.all(np.isfinite(d16.view(np.float16)))


def test_q8_1_crafted_ties(orc):
    # amax 127 -> d = 1 exactly, so x/d = x and every k + 1/2 is an exact tie
    ks = np.arange(-63, 63, dtype=np.float32)
    x = np.zeros((len(ks), 32), np.float32)
    x[:, 0] = 127.0
    x[:, 1] = ks + 0.5
    _, _, q = _fields(orc.quantize_q8_1(x))
    expect = np.where(ks + 0.5 > 0, ks + 1, ks).astype(np.int64)   # away from zero
    assert np.array_equal(q[:, 1], expect)


def test_q8_1_zero_and_clamp(orc):
    x = np.zeros(64, np.float32)
    x[32:] = np.linspace(-5, 5, 32, dtype=np.float32)
    out = orc.quantize_q8_1(x)
    d16, s16, q = _fields(out)
    assert d16[0] == 0 and s16[0] == 0 and not q[0].any()
    assert q[1].max() == 127 and q[1].min() == -127


def test_q8_0_roundtrip(orc):
    """Re-quantizing a dequantized Q8_0 block gives the same bytes: f(d16)*127 and f(d16)*q are
    exact in float32, so amax' = 127 f(d16), d' = f(d16), q' = q, d16' = d16."""
    g = np.random.default_rng(11)
    x = (g.standard_normal((50, 256)) * 0.7).astype(np.float32)
    b = orc.quantize_q8_0(x).reshape(-1, 34)
    d = b[:, 0:2].copy().view(np.float16)[:, 0].astype(np.float32)
    q = b[:, 2:].view(np.int8).astype(np.float32)
    y = (d[:, None] * q).reshape(x.shape)
    b2 = orc.quantize_q8_0(y).reshape(-1, 34)
    assert np.array_equal(b, b2)
    # error bound: |x - f(d16) q| <= d/2 + 127 |d - f(d16)| (+ float32 rounding)
    xb = x.reshape(-1, 32)
    dd = np.abs(xb).max(axis=1).astype(np.float32) / np.float32(127)
    err = np.abs(xb.astype(np.float64) - (d[:, None] * q))
    bound = (dd / 2 + 127 * np.abs(dd - d))[:, None] + 1e-6 * np.abs(xb)
    assert np.all(err <= bound)


def test_planted_mistake_detected(orc):
    """A corrupted quant byte must be seen by the golden comparison (the checker is not blind)."""
    doc = json.load(open(os.path.join(GOLD, "q8_1_blocks.json")))
    blk = doc["blocks"][0]
    out = orc.quantize_q8_1(np.array(blk["x"], np.float32))
    out[4 + 5] ^= 1
    assert out[4:].view(np.int8).astype(int).tolist() != blk["q"]
