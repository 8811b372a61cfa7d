"""Pins of the oracle's number formats and the gate against library routines
and closed forms (CPU)."""
import math

import numpy as np
import pytest
import torch

from oracle import oracle


def test_bf16_decode_all_codes():
    """Every bf16 bit pattern decodes as torch.bfloat16 -> float64 does."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_e4m3_decode_all_codes():
    """Every OCP e4m3fn byte decodes as torch.float8_e4m3fn -> float32 does
    (0x7F and 0xFF are NaN; there are no infinities)."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = np.array([oracle.e4m3_to_double(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan].astype(np.float64), got[~nan])
    # closed forms: largest finite 448, smallest subnormal 2^-9
    assert oracle.e4m3_to_double(0x7E) == 448.0
    assert oracle.e4m3_to_double(0x01) == 2.0 ** -9
    assert oracle.e4m3_to_double(0x80) == 0.0 and math.copysign(1, oracle.e4m3_to_double(0x80)) < 0


def test_f32_to_bf16_rounding_matches_torch():
    rng = np.random.default_rng(3)
    xs = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(5000) * 1e-38).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.0078125, 1.01171875, 3.0e38, np.inf, -np.inf],
                 dtype=np.float32),
        # exact halfway cases: ties to even
        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], dtype=np.float32),
    ])
    ref = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f32_to_bf16_bits(float(x)) for x in xs], dtype=np.uint16)
    assert np.array_equal(ref, got)


def test_gate_closed_forms():
    """sigmoid(0) = 1/2 exactly; for g >= 17, 1 + exp(-g) rounds to 1 in fp32,
    so the gate is exactly 1; for very negative g it is 0 or a tiny value."""
    assert oracle.gate_value(0x0000) == 0.5
    assert oracle.gate_value(0x8000) == 0.5  # -0.0
    for g in (17.0, 20.0, 100.0, 3.0e38):
        b = int(torch.tensor(g).to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF
        assert oracle.gate_value(b) == 1.0
    b = int(torch.tensor(-200.0).to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF
    assert oracle.gate_value(b) == 0.0
    # the result is always a bf16 value
    for g in np.linspace(-10, 10, 101):
        b = int(torch.tensor(float(g)).to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF
        v = oracle.gate_value(b)
        vb = torch.tensor(v, dtype=torch.float32).to(torch.bfloat16).to(torch.float32).item()
        assert v == vb


def test_gate_against_torch_sigmoid_all_codes():
    """Against torch.sigmoid in fp32 rounded to bf16 (the unfused gate), for
    every finite bf16 logit: equal, or one bf16 ulp apart on a near-tie."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    finite = torch.isfinite(x).numpy()
    ref = torch.sigmoid(x.to(torch.float32)).to(torch.bfloat16).to(torch.float32).numpy()
    got = np.array([oracle.gate_value(int(b)) for b in bits], dtype=np.float32)
    ref, got = ref[finite], got[finite]
    diff = got != ref
    assert diff.mean() < 1e-3
    if diff.any():
        ulp = np.abs(got[diff].astype(np.float64) - ref[diff]) / np.maximum(
            np.abs(ref[diff]), 1e-30) * 256
        assert (ulp <= 1.0 + 1e-9).all()


def _pages_splits_table():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "splits_b300.txt")
    rows = []
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            a, b = line.split()
            rows.append((int(a), int(b)))
    return rows


@pytest.mark.parametrize("rows,splits", _pages_splits_table())
def test_pages_split_heuristic(rows, splits):
    """The pages' B300 split rule, evaluated by hand into tests/golden."""
    assert oracle.splits_pages(rows) == splits
