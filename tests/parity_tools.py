"""Comparison helpers for the GPU-vs-oracle parity tests (no method arithmetic)."""
import numpy as np


def bf16_ordinal(bits: np.ndarray) -> np.ndarray:
    """Maps bf16 bit patterns to integers ordered like their values (adjacent
    representable values differ by 1; +0 and -0 map to the same integer)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    return np.abs(bf16_ordinal(a_bits) - bf16_ordinal(b_bits))


def rel_frobenius(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    return float(num / den) if den > 0 else float(num)


def assert_bf16_close(got_bits, ref_bits, max_ulp=1, max_mismatch_frac=1e-3, what=""):
    dist = ulp_distance(got_bits, ref_bits)
    worst = int(dist.max()) if dist.size else 0
    frac = float(np.count_nonzero(dist)) / max(dist.size, 1)
    assert worst <= max_ulp, f"{what}: {worst} ulp apart (limit {max_ulp})"
    assert frac <= max_mismatch_frac, f"{what}: {frac:.2e} of elements differ (limit {max_mismatch_frac:.0e})"
    return worst, frac


def assert_sum_close(got_bits, ref_bits, abs_terms, rel_sum=2.0**-20, max_mismatch_frac=1e-3, what=""):
    """bf16 results of long fp32 sums: each element within one bf16 ulp of the
    reference plus rel_sum * sum_i |a_i b_i| (the fp32 summation error, which
    dominates where the terms cancel to a value near zero)."""
    got = np.asarray(__import__("oracle").bf16_to_f64(got_bits))
    ref = np.asarray(__import__("oracle").bf16_to_f64(ref_bits))
    ulp = np.maximum(np.abs(ref), np.abs(got)) * 2.0**-7
    excess = np.abs(got - ref) - ulp - rel_sum * np.asarray(abs_terms)
    worst = float(excess.max()) if excess.size else 0.0
    frac = float(np.count_nonzero(got_bits != ref_bits)) / max(got.size, 1)
    assert worst <= 0, f"{what}: error exceeds ulp + {rel_sum:.1e}*sum|ab| by {worst:.3e}"
    assert frac <= max_mismatch_frac, f"{what}: {frac:.2e} of elements differ (limit {max_mismatch_frac:.0e})"
    return frac


def assert_update_close(got_bits, ref_bits, s, abs_terms, rel_h=2.0**-15, max_mismatch_frac=1e-4, what="",
                        prev_got_bits=None, prev_ref_bits=None):
    """Weights after the update: each element within one bf16 ulp of the
    reference, plus s * rel_h * sum_a |c_ia p_ja| where w and s*h cancel (the
    fp32 / two-term-bf16 error of h, scaled by s, can then exceed an ulp of
    the small result); at most max_mismatch_frac of the elements differ.

    In a chain of updates the two sides start from their own previous weights;
    where those differ (prev_got_bits vs prev_ref_bits), the same random bits
    carry the difference through the rounding, so it is allowed on top."""
    orc = __import__("oracle")
    got = np.asarray(orc.bf16_to_f64(got_bits))
    ref = np.asarray(orc.bf16_to_f64(ref_bits))
    ulp = np.maximum(np.abs(ref), np.abs(got)) * 2.0**-7
    excess = np.abs(got - ref) - ulp - abs(float(s)) * rel_h * np.asarray(abs_terms)
    if prev_got_bits is not None:
        excess -= np.abs(orc.bf16_to_f64(prev_got_bits) - orc.bf16_to_f64(prev_ref_bits))
    worst = float(excess.max()) if excess.size else 0.0
    frac = float(np.count_nonzero(got_bits != ref_bits)) / max(got.size, 1)
    assert worst <= 0, f"{what}: error exceeds ulp + s*{rel_h:.1e}*sum|cp| by {worst:.3e}"
    assert frac <= max_mismatch_frac, f"{what}: {frac:.2e} of elements differ (limit {max_mismatch_frac:.0e})"
    return frac


def qr_margin_mismatches(got_bits, seed, k, r, rel=1e-12):
    """Number of QR projection elements that differ from the oracle's; each
    difference must sit where the oracle's fp64 pre-rounding value is within
    1e-12 (relative) of a rounding boundary, so that either neighbour is a
    correct rounding of the exact frame."""
    orc = __import__("oracle")
    ref_pre = orc.qr_projection_preround(seed, k, r)
    ref = orc.f64_to_bf16_via_f32(ref_pre)
    bad = np.argwhere(got_bits != ref)
    for i, j in bad:
        v = ref_pre[i, j]
        lo = orc.f64_to_bf16_via_f32(np.array([v * (1 - rel)]))[0]
        hi = orc.f64_to_bf16_via_f32(np.array([v * (1 + rel)]))[0]
        assert got_bits[i, j] in (lo, hi), (i, j, v, hex(got_bits[i, j]), hex(ref[i, j]))
    return len(bad)

