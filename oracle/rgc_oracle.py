"""CPU oracle for the randomized low-rank gradient-sketch path.

TEST INFRASTRUCTURE ONLY. Nothing in the product library imports, links or calls
this module; only the tests, the smoke check and the benchmark's CPU-baseline leg
may use it. It shares no code, constant table or helper with the HIP kernels.

Plain numpy, float64 wherever the pages leave the precision open, slow on purpose
so that each function can be read against the pages by eye.

Sources, by page title (sections as they appear on each page):
  [RGC]     "Randomized Gradient Compression" (blog post): "How it works",
            footnote 1 (the projection), "Memory you can predict".
  [LoGRA-S] "LoGRA: Scaling LLM Reinforcement Learning with Low-Rank Gradient
            Sketches" (paper summary): "Key Contributions" item 1 and 2,
            "Methodology in Plain English".
  [LoGRA-M] "LoGRA: Low-Rank Gradient Sketches" (tutorial module): "The Core Move",
            "Why the Sketch Can Be Accumulated Without a Full Gradient",
            "Why the Update Is Low-Rank but Not an Exact Recovery",
            "Why Refreshing the Projection Enables New Update Directions",
            "Minimal Causal Code".
  Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
            as 1, 2, 3", SC'11 (the published counter-based generator).

Notation (shared with the C header): W is d x k (out x in, like a linear
layer's weight), X is T x k (tokens x in), D = dL/dY is T x d, the gradient is
G = D^T X (d x k), P is k x r, XP = X P is T x r, the sketch C = D^T (X P) is
d x r in fp32, and the rebuilt update is H = C P^T (d x k).

Readings of the pages where they are silent are listed with each function.
Parity status: every function here is pinned by a test in tests/ against a
library routine, a closed form, an invariant or a value the pages print, except
the exact bits of the Gaussian draw (gaussian_matrix), which is pinned only in
distribution (parity unpinned for its bits; its effect on P is checked with a
rounding-margin rule).
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Philox4x32-10 (SC'11 paper): a 4-word counter is encrypted by ten rounds of
# two 32x32->64 multiplies and xors with a 2-word key that is bumped by the
# Weyl constants between rounds.
# ---------------------------------------------------------------------------
_MASK32 = np.uint64(0xFFFFFFFF)
_PHILOX_MUL0 = np.uint64(0xD2511F53)
_PHILOX_MUL1 = np.uint64(0xCD9E8D57)
_PHILOX_WEYL0 = np.uint64(0x9E3779B9)
_PHILOX_WEYL1 = np.uint64(0xBB67AE85)

# Stream tags, placed in counter word 2 so that the projection and rounding
# draws made from one caller seed never overlap.
TAG_RADEMACHER = 1
TAG_GAUSSIAN = 2
TAG_ROUNDING = 3


def seed_to_key(seed: int) -> tuple[int, int]:
    """Split a 64-bit seed into the two 32-bit Philox key words (low, high)."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & 0xFFFFFFFF, seed >> 32


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Ten Philox rounds on counters (c0..c3) under key (k0, k1).

    All arguments broadcast against each other (uint32 arrays or ints);
    returns four uint32 arrays, the output words 0..3.
    """
    c = [np.asarray(x, dtype=np.uint64) & _MASK32 for x in (c0, c1, c2, c3)]
    k0 = np.asarray(k0, dtype=np.uint64) & _MASK32
    k1 = np.asarray(k1, dtype=np.uint64) & _MASK32
    for _ in range(10):
        p0 = _PHILOX_MUL0 * c[0]  # full 64-bit products of 32-bit words
        p1 = _PHILOX_MUL1 * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
        k0 = (k0 + _PHILOX_WEYL0) & _MASK32
        k1 = (k1 + _PHILOX_WEYL1) & _MASK32
    return tuple(x.astype(np.uint32) for x in c)


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------
def f32_bits(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)


def bits_f32(b) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(b, dtype=np.uint32)).view(np.float32)


def bf16_to_f64(b) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return bits_f32(b).astype(np.float64)


def f32_to_bf16_rne(x) -> np.ndarray:
    """IEEE round-to-nearest-even of fp32 values to bf16; returns uint16 bits.

    The dropped low half is compared with one half-unit of the kept bf16 and
    ties go to the even pattern; NaN stays a quiet NaN with its sign.
    """
    b = f32_bits(x).astype(np.uint64)
    keep = b >> np.uint64(16)
    low = b & np.uint64(0xFFFF)
    up = (low > 0x8000) | ((low == 0x8000) & ((keep & np.uint64(1)) == 1))
    out = keep + up.astype(np.uint64)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    out = np.where(nan, keep | np.uint64(0x40), out)
    return out.astype(np.uint16)


def f64_to_bf16_via_f32(x) -> np.ndarray:
    """Round float64 to fp32 (RNE), then to bf16 (RNE): the storage rounding of P."""
    return f32_to_bf16_rne(np.asarray(x, dtype=np.float64).astype(np.float32))


# ---------------------------------------------------------------------------
# Projection P (k x r), regenerated from a 64-bit seed.
# ---------------------------------------------------------------------------
def rademacher_projection(seed, k: int, r: int) -> np.ndarray:
    """Random-sign projection, entries +-bf16(1/sqrt(r)); returns uint16 k x r.

    [LoGRA-M, "Why the Sketch Can Be Accumulated Without a Full Gradient"]: the
    default projection has random sign entries scaled by 1/sqrt(r), drawn
    independently of the batch. Stream: for row i and column block j>>7 one
    Philox call (counter (i, j>>7, TAG_RADEMACHER, 0), key = seed) gives 128
    sign bits; column j takes bit (j & 31) of word ((j >> 5) & 3); a set bit
    means a negative entry.

    `seed` may be an int or an array of seeds (batched draws along axis 0).
    """
    seeds = np.atleast_1d(np.asarray(seed, dtype=np.uint64))
    k0 = (seeds & _MASK32)[:, None, None]
    k1 = (seeds >> np.uint64(32))[:, None, None]
    i = np.arange(k, dtype=np.uint64)[None, :, None]
    j = np.arange(r, dtype=np.uint64)[None, None, :]
    words = philox4x32_10(i, j >> np.uint64(7), TAG_RADEMACHER, 0, k0, k1)
    shape = (len(seeds), k, r)
    w = np.stack([np.broadcast_to(x, shape) for x in words], axis=0).astype(np.uint64)
    sel = np.broadcast_to(((j >> np.uint64(5)) & np.uint64(3)).astype(np.int64), shape)
    word = np.take_along_axis(w, sel[None], axis=0)[0]
    bit = (word >> (j & np.uint64(31))) & np.uint64(1)
    mag = int(f64_to_bf16_via_f32(np.array([1.0 / np.sqrt(float(r))]))[0])
    out = np.where(bit == 1, np.uint16(mag | 0x8000), np.uint16(mag)).astype(np.uint16)
    return out if np.ndim(seed) else out[0]


def gaussian_matrix(seed, k: int, r: int) -> np.ndarray:
    """Standard normal k x r matrix in float64 by the Box-Muller transform.

    The pages draw the frame from a Gaussian matrix [RGC, footnote 1] but fix
    no generator; this reading: counter (i, j>>2, TAG_GAUSSIAN, 0) gives four
    words; columns 4q, 4q+1 use words (0, 1) and columns 4q+2, 4q+3 use words
    (2, 3). With u1 = (w_a + 1/2)/2^32 and u2 = (w_b + 1/2)/2^32, both exact,
    rho = sqrt(-2 ln u1) and theta = 2 pi u2; the even column takes
    rho*cos(theta), the odd one rho*sin(theta).

    `seed` may be an int or an array of seeds (batched draws along axis 0).
    """
    seeds = np.atleast_1d(np.asarray(seed, dtype=np.uint64))
    k0 = (seeds & _MASK32)[:, None, None]
    k1 = (seeds >> np.uint64(32))[:, None, None]
    i = np.arange(k, dtype=np.uint64)[None, :, None]
    j = np.arange(r, dtype=np.uint64)[None, None, :]
    w = philox4x32_10(i, j >> np.uint64(2), TAG_GAUSSIAN, 0, k0, k1)
    w = np.stack([np.broadcast_to(x, (len(seeds), k, r)) for x in w], axis=0)
    pair = ((j >> np.uint64(1)) & np.uint64(1)).astype(np.int64)
    idx_a = np.broadcast_to(2 * pair, w.shape[1:])[None]
    wa = np.take_along_axis(w, idx_a, axis=0)[0].astype(np.float64)
    wb = np.take_along_axis(w, idx_a + 1, axis=0)[0].astype(np.float64)
    u1 = (wa + 0.5) * 2.0**-32
    u2 = (wb + 0.5) * 2.0**-32
    rho = np.sqrt(-2.0 * np.log(u1))
    theta = (2.0 * np.pi) * u2
    odd = np.broadcast_to((j & np.uint64(1)) == 1, w.shape[1:])
    z = np.where(odd, rho * np.sin(theta), rho * np.cos(theta))
    return z if np.ndim(seed) else z[0]


def orthonormal_frame(a: np.ndarray) -> np.ndarray:
    """Q of the thin QR factorization a = Q R with diag(R) > 0.

    [RGC, footnote 1]: QR of a Gaussian matrix with the standard sign
    correction, which makes R's diagonal positive and Q unique. Works on a
    single k x r matrix or a stack (..., k, r).
    """
    q, rr = np.linalg.qr(a, mode="reduced")
    sgn = np.sign(np.diagonal(rr, axis1=-2, axis2=-1))
    sgn = np.where(sgn == 0, 1.0, sgn)
    return q * sgn[..., None, :]


def qr_projection_preround(seed, k: int, r: int) -> np.ndarray:
    """sqrt(k/r) * Q in float64, before storage rounding [RGC, footnote 1]."""
    return np.sqrt(float(k) / float(r)) * orthonormal_frame(gaussian_matrix(seed, k, r))


def qr_projection(seed: int, k: int, r: int) -> np.ndarray:
    """QR-of-Gaussian projection stored as bf16 bits (fp64 -> fp32 -> bf16, RNE)."""
    return f64_to_bf16_via_f32(qr_projection_preround(seed, k, r))


def sample_projection(kind: str, seed: int, k: int, r: int) -> np.ndarray:
    if kind == "rademacher":
        return rademacher_projection(seed, k, r)
    if kind == "qr":
        return qr_projection(seed, k, r)
    raise ValueError(kind)


# ---------------------------------------------------------------------------
# The sketch: projection of the saved activations and accumulation.
# ---------------------------------------------------------------------------
def project(x_bits: np.ndarray, p_bits: np.ndarray) -> np.ndarray:
    """XP = X P, the activation the layer keeps instead of X [RGC, "How it works"].

    Exact float64 products of the bf16 inputs, one rounding to fp32 and one to
    bf16 (the activation dtype; the pages leave XP's storage type open).
    """
    xp = bf16_to_f64(x_bits) @ bf16_to_f64(p_bits)
    return f32_to_bf16_rne(xp.astype(np.float32))


def accumulate(c: np.ndarray, d_bits: np.ndarray, xp_bits: np.ndarray) -> np.ndarray:
    """C <- C + D^T (X P) for one microbatch, stored in fp32.

    [RGC, "How it works"] accumulates the narrow d x r matrix per microbatch;
    [LoGRA-S, Key Contributions 1] keeps it in fp32 and never forms the d x k
    gradient. The microbatch product is exact-ish float64; C is rounded to fp32
    once per microbatch, as a caller-held fp32 buffer would be.
    """
    prod = bf16_to_f64(d_bits).T @ bf16_to_f64(xp_bits)
    return (np.asarray(c, dtype=np.float32).astype(np.float64) + prod).astype(np.float32)


def layer_forward(x_bits: np.ndarray, w_bits: np.ndarray, p_bits) -> tuple:
    """The layer's forward with its sketch projection: Y = X W^T (T x d) and
    XP = X P (T x r), the activation kept in place of X [RGC, "How it works"].

    W is d x k (out x in), so Y's column j is X times W's row j. Each output is
    the exact float64 sum of the bf16 products, rounded once to fp32 and once to
    bf16 (the layer's output dtype; the pages leave it open). p_bits None gives
    (Y, None).
    """
    y = bf16_to_f64(x_bits) @ bf16_to_f64(w_bits).T
    y_bits = f32_to_bf16_rne(y.astype(np.float32))
    return y_bits, (project(x_bits, p_bits) if p_bits is not None else None)


def layer_backward(d_bits: np.ndarray, w_bits: np.ndarray, xp_bits, c) -> tuple:
    """The layer's backward with its sketch: the input gradient dX = D W (T x k;
    D = dL/dY is T x d) flows on, and C gains D^T (X P) from the saved XP
    [RGC, "How it works"] in place of the weight gradient D^T X. dX rounded as
    Y in layer_forward; C as in accumulate. xp_bits None gives (dX, c).
    """
    dx = bf16_to_f64(d_bits) @ bf16_to_f64(w_bits)
    dx_bits = f32_to_bf16_rne(dx.astype(np.float32))
    return dx_bits, (accumulate(c, d_bits, xp_bits) if xp_bits is not None else c)


def reconstruct(c: np.ndarray, p_bits: np.ndarray) -> np.ndarray:
    """H = C P^T in float64 (rank <= r) [RGC, "How it works"]; [LoGRA-M, low-rank section]."""
    return np.asarray(c, dtype=np.float32).astype(np.float64) @ bf16_to_f64(p_bits).T


# ---------------------------------------------------------------------------
# The update: normalized SGD with stochastic rounding to bf16.
# ---------------------------------------------------------------------------
def rounding_bits(seed: int, rows: int, cols: int, row0: int = 0, col0: int = 0) -> np.ndarray:
    """16 random bits per weight element, keyed on (seed, row, col).

    The pages name no source for the rounding randomness; this reading: one
    Philox call per row i and block of 8 columns (counter (j>>3, i,
    TAG_ROUNDING, 0), key = seed); column j uses word (j & 7) >> 1, its low
    half for even j and its high half for odd j.
    """
    k0, k1 = seed_to_key(seed)
    i = (np.arange(rows, dtype=np.uint64) + np.uint64(row0))[:, None]
    j = (np.arange(cols, dtype=np.uint64) + np.uint64(col0))[None, :]
    w = philox4x32_10(j >> np.uint64(3), i, TAG_ROUNDING, 0, k0, k1)
    w = np.stack([np.broadcast_to(x, (rows, cols)) for x in w], axis=0).astype(np.uint64)
    sel = np.broadcast_to(((j & np.uint64(7)) >> np.uint64(1)).astype(np.int64), (rows, cols))
    word = np.take_along_axis(w, sel[None], axis=0)[0]
    odd = np.broadcast_to((j & np.uint64(1)) == 1, (rows, cols))
    return np.where(odd, word >> np.uint64(16), word & np.uint64(0xFFFF)).astype(np.uint16)


def stochastic_round(v: np.ndarray, r16: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 with stochastic rounding; returns uint16 bits.

    [RGC, "How it works"]: a value lying a fraction f of the way from one bf16
    neighbour to the next must land on the upper one with probability f. Adding
    a uniform 16-bit integer to the dropped low half and keeping the high half
    does exactly that (the carry happens for low16 + r16 >= 2^16, i.e. in
    low16 of the 2^16 cases). NaN becomes a quiet NaN with its sign; +-Inf is
    kept; finite values beyond the largest bf16 may round to +-Inf.
    """
    v = np.asarray(v, dtype=np.float32)
    b = f32_bits(v).astype(np.uint64)
    out = (b + np.asarray(r16, dtype=np.uint64)) >> np.uint64(16)
    out = np.where(np.isinf(v), b >> np.uint64(16), out)
    out = np.where(np.isnan(v), (b >> np.uint64(16)) | np.uint64(0x40), out)
    return out.astype(np.uint16)


def step_scale(tau: float, norm_w: float, norm_h: float) -> tuple[np.float32, int]:
    """s = tau * ||W|| / ||H|| rounded to fp32; (0, 1) when ||H|| = 0 or s is not finite.

    [RGC, "How it works"]: normalized SGD moves each matrix by the same fraction
    tau of its own norm; norms are Frobenius (the plainest reading). A zero
    sketch (e.g. all-equal rewards) gives no direction, so the update is skipped
    and the flag raised.
    """
    t = float(np.float32(tau))
    if norm_h == 0.0 or not np.isfinite(norm_h):
        return np.float32(0.0), 1
    s = np.float32(t * norm_w / norm_h)
    if not np.isfinite(s):
        return np.float32(0.0), 1
    return s, 0


def apply_update(w_bits: np.ndarray, c: np.ndarray, p_bits: np.ndarray, tau: float, seed: int):
    """W <- SR_bf16(W - tau ||W|| H / ||H||), H = C P^T, no fp32 copy of W kept.

    [RGC, "How it works"]. Norms in float64 over the whole matrix; s in fp32;
    the pre-rounding value is two separately rounded fp32 operations,
    v = w - (s * h) with h = fp32(H) (no fused multiply-add); then stochastic
    rounding with the (seed, row, col) stream. When the update is skipped the
    weights are returned unchanged. Returns (new bits, stats) with stats =
    float32 [||W||, ||H||, s, flag].
    """
    w64 = bf16_to_f64(w_bits)
    h64 = reconstruct(c, p_bits)
    norm_w = float(np.sqrt(np.sum(w64 * w64)))
    norm_h = float(np.sqrt(np.sum(h64 * h64)))
    s, flag = step_scale(tau, norm_w, norm_h)
    stats = np.array([norm_w, norm_h, s, flag], dtype=np.float32)
    if flag:
        return np.array(w_bits, dtype=np.uint16, copy=True), stats
    v = pre_round_values(w_bits, h64.astype(np.float32), s)
    d, k = w64.shape
    return stochastic_round(v, rounding_bits(seed, d, k)), stats


def weight_sumsq(w_bits: np.ndarray) -> float:
    """||W||_F^2 of bf16 weights, summed in float64.

    [RGC, "How it works"]: the normalized step scales by norm(W), read as the
    Frobenius norm. An update that carries the norm to the next step hands on
    the squared norm of the weights it wrote, which is this value of them.
    """
    w64 = bf16_to_f64(w_bits)
    return float(np.sum(w64 * w64))


def apply_scaled(w_bits: np.ndarray, c: np.ndarray, p_bits: np.ndarray, alpha, seed: int) -> np.ndarray:
    """W <- SR_bf16(W - alpha H), H = C P^T: the fixed-step update.

    [LoGRA-M, "Minimal Causal Code"]: W -= alpha * eta * (U @ A), with U = S
    for plain SGD on the sketch (C here) and A = P^T; the caller passes the
    product alpha*eta as one fp32 scalar. Readings: the pages do not say how
    LoGRA rounds bf16 weights; the same stochastic rounding and bit stream as
    apply_update are used, and the pre-rounding value is formed exactly as
    there, v = fp32(w - fp32(alpha * h)). No norms, nothing skipped.
    """
    h32 = reconstruct(c, p_bits).astype(np.float32)
    v = pre_round_values(w_bits, h32, np.float32(alpha))
    d, k = np.shape(w_bits)
    return stochastic_round(v, rounding_bits(seed, d, k))


def pre_round_values(w_bits: np.ndarray, h32: np.ndarray, s) -> np.ndarray:
    """v = fp32(w - fp32(s * h)) elementwise, no fused multiply-add."""
    w32 = bf16_to_f64(w_bits).astype(np.float32)
    sh = (np.float32(s) * np.asarray(h32, dtype=np.float32)).astype(np.float32)
    return (w32 - sh).astype(np.float32)


# ---------------------------------------------------------------------------
# One whole update of one matrix, as the pages' loop runs it.
# ---------------------------------------------------------------------------
def sketch_update(kind: str, r: int, p_seed: int, sr_seed: int, w_bits, x_mbs, d_mbs, tau: float):
    """[LoGRA-M, "Minimal Causal Code"] in [RGC]'s normalized form: draw P, zero
    C, add each microbatch's D^T (X P), then apply once.

    Returns (P bits, C, new W bits, stats).
    """
    d, k = w_bits.shape
    p = sample_projection(kind, p_seed, k, r)
    c = np.zeros((d, r), dtype=np.float32)
    for xb, db in zip(x_mbs, d_mbs):
        c = accumulate(c, db, project(xb, p))
    w_new, stats = apply_update(w_bits, c, p, tau, sr_seed)
    return p, c, w_new, stats
