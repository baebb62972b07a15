"""Comparison helpers shared by the tests (no arithmetic of the method here)."""

import numpy as np


def bf16_ordinal(bits):
    """Map bf16 bit patterns onto integers that count representable values
    (sign-magnitude to two's-complement order; +0 and -0 both map to 0)."""
    b = np.asarray(bits, np.uint16).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def bf16_value(bits):
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def assert_bf16_close(got_bits, ref_bits, atol, ulps=1, err_msg=""):
    """Every element within `ulps` bf16 steps of the reference, or within
    `atol` of it in value (for results near zero, where a bf16 step is far
    finer than the fp32 accumulation error)."""
    got_bits = np.asarray(got_bits, np.uint16)
    ref_bits = np.asarray(ref_bits, np.uint16)
    d_ulp = np.abs(bf16_ordinal(got_bits) - bf16_ordinal(ref_bits))
    d_val = np.abs(bf16_value(got_bits) - bf16_value(ref_bits))
    bad = (d_ulp > ulps) & ~(d_val <= atol)
    if bad.any():
        i = np.flatnonzero(bad.ravel())[:8]
        raise AssertionError(
            f"{err_msg}: {bad.sum()} of {bad.size} bf16 values off by more than {ulps} ulp "
            f"and {atol} abs; first at flat {i.tolist()}: got {bf16_value(got_bits.ravel()[i]).tolist()} "
            f"ref {bf16_value(ref_bits.ravel()[i]).tolist()}")
    # report the largest step difference away from zero and how many differ
    away = np.abs(bf16_value(ref_bits)) > 1e-3
    return (int(d_ulp[away].max()) if away.any() else 0), int((d_ulp > 0).sum())
