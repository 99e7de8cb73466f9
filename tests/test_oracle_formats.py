"""Pins of the oracle's number formats against values fixed outside its code."""
import numpy as np
import torch

import oracle

# E2M1 magnitudes as listed in the OCP Microscaling Formats v1.0 specification
# (FP4 E2M1 element table): 0, 0.5, 1, 1.5, 2, 3, 4, 6; codes 8..15 are negatives.
SPEC_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table_matches_spec_listing():
    for c in range(8):
        assert oracle.e2m1_value(c) == SPEC_E2M1[c]
        neg = oracle.e2m1_value(c + 8)
        assert neg == -SPEC_E2M1[c] and np.signbit(neg)
    assert list(oracle.E2M1_MAGNITUDES) == SPEC_E2M1
    assert oracle.E2M1_EMAX == 2           # 6 = 1.5 * 2^2 is the largest normal


def test_e8m0_values():
    assert oracle.e8m0_value(127) == 1.0
    assert oracle.e8m0_value(0) == 2.0 ** -127
    assert oracle.e8m0_value(254) == 2.0 ** 127
    assert oracle.e8m0_value(128) == 2.0
    assert np.isnan(oracle.e8m0_value(255))


def test_bf16_decode_matches_torch_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_bits_to_f64(bits)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    assert (np.signbit(got) == np.signbit(ref))[~np.isnan(ref)].all()


def test_f32_decode_matches_numpy_view():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, size=100000, dtype=np.uint64).astype(np.uint32)
    with np.errstate(invalid="ignore"):           # signalling-NaN patterns
        ref = bits.view(np.float32).astype(np.float64)
    got = oracle.f32_bits_to_f64(bits)
    assert ((got == ref) | (np.isnan(got) & np.isnan(ref))).all()
