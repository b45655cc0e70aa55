"""Gamma, the DMPQ precision rule and the Temporal Delta Cache (TDC).

Test infrastructure (see the package docstring).

Sources on the 6Bit-Diffusion pages:
  * Fig. 2 caption: DMPQ picks each linear's activation bits from the
    block's input/output relative L1 distance Gamma at the preceding
    timestep; TDC decides to skip a block from the block updates Delta of
    the two preceding timesteps.
  * Fig. 3 caption: E_rel at timestep t is linear in Gamma_{t-1}, fitted as
    y = alpha x + beta for each internal linear layer.
  * Abstract: NVFP4 goes to temporally stable layers and INT8 to volatile
    ones; TDC reuses the block residual (input to output) because it is
    consistent across timesteps, skipping invariant blocks.
  * Fig. 4 caption: the agreement of Delta_t and Delta_{t-1} is measured by
    cosine similarity and relative L2 difference.

Readings taken where the pages are silent:
  * Gamma = sum|out - in| / sum|in| over the whole block hidden state; a
    zero denominator gives 0 if the numerator is 0, else +inf.
  * Predictor p = alpha * Gamma_{t-1} + beta (float64, alpha and beta
    float32); p > tau -> INT8, else NVFP4 (a tie is NVFP4).  No Gamma at
    t = 0: every layer is INT8.
  * Skip at t when t >= 2, the block was computed at t-1, and
    d = ||Delta_{t-1} - Delta_{t-2}||_2 / ||Delta_{t-2}||_2 < delta (strict).
    A skipped block outputs bf16(in + Delta_last) and keeps its cache; the
    next step computes it.  A computed block stores Delta = bf16(out - in)
    and measures d against the cached Delta it replaces.
  * Delta and outputs are bfloat16 rounded once (nearest-even) from the
    exact sum/difference; the norms are square roots of float64 sums.
  * The cosine of Fig. 4 is <Delta_t, Delta_{t-1}> / (||Delta_t|| ||Delta_{t-1}||)
    from float64 sums of exact terms (0 when either norm is 0); its skip
    rule (a variant) is t >= 2, computed at t-1 and cos > threshold.
  * E_rel (the layer-wise relative quantization error of Fig. 3) is the
    relative L2 error ||Y_q - Y||_2 / ||Y||_2 of a linear's bf16 output
    against the bf16 output of the unquantized linear (0/0 = 0, x/0 = inf).
  * The fit of Fig. 3 is ordinary least squares on the time-shifted pairs
    (Gamma_{t-1} of the block, E_rel_t of the linear), t = 1..T-1, pairs
    with a non-finite value dropped; alpha and beta are the exact
    least-squares values rounded to float32 (nearest-even).  Fewer than two
    distinct x: alpha = 0, beta = mean of y (0 without pairs).
"""
from fractions import Fraction
import math

import numpy as np

from .formats import bf16_to_f64, f64_to_bf16_rne


def _fsum(a):
    """Correctly rounded float64 sum."""
    return math.fsum(np.asarray(a, dtype=np.float64).ravel().tolist())


def _psum(a):
    """Pairwise float64 sum (numpy): for n non-negative terms its relative
    error is below ceil(log2 n) * 2^-53 (about 3e-15 for n = 2^25), used
    where the correctly rounded sum is too slow (whole DiT stacks)."""
    return float(np.sum(np.asarray(a, dtype=np.float64)))


_SUM = {"exact": _fsum, "pairwise": _psum}


def ratio(num, den):
    """num / den with 0/0 -> 0 and x/0 -> +inf (float64)."""
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return num / den


def gamma_sums(in_bits, out_bits, summation="exact"):
    """(S1, S2) = (sum|out - in|, sum|in|), each correctly rounded (or
    pairwise, see _psum)."""
    x = bf16_to_f64(in_bits)
    y = bf16_to_f64(out_bits)
    add = _SUM[summation]
    return add(np.abs(y - x)), add(np.abs(x))


def gamma(in_bits, out_bits):
    """Relative L1 distance of a block's output from its input."""
    s1, s2 = gamma_sums(in_bits, out_bits)
    return ratio(s1, s2)


def tdc_update(in_bits, out_bits, delta_prev_bits=None, summation="exact"):
    """Delta_new = bf16(out - in) and the sums S1..S4.

    S1 = sum|out - in|, S2 = sum|in|, S3 = sum (Delta_new - Delta_prev)^2,
    S4 = sum Delta_prev^2; S3 = S4 = 0 without a previous Delta.
    """
    add = _SUM[summation]
    x = bf16_to_f64(in_bits)
    y = bf16_to_f64(out_bits)
    delta_new = f64_to_bf16_rne(y - x)
    s1, s2 = add(np.abs(y - x)), add(np.abs(x))
    if delta_prev_bits is None:
        return delta_new, (s1, s2, 0.0, 0.0)
    dn = bf16_to_f64(delta_new)
    dp = bf16_to_f64(delta_prev_bits)
    return delta_new, (s1, s2, add((dn - dp) ** 2), add(dp ** 2))


def rel_l2(s3, s4):
    """||Delta_new - Delta_prev|| / ||Delta_prev|| from the sums."""
    return ratio(math.sqrt(s3), math.sqrt(s4))


def tdc_apply(in_bits, delta_bits):
    """out = bf16(in + Delta) with one rounding of the exact sum."""
    return f64_to_bf16_rne(bf16_to_f64(in_bits) + bf16_to_f64(delta_bits))


def dmpq_mask(gamma_prev, alpha, beta, tau, n_linears):
    """Per-linear format: 1 = INT8, 0 = NVFP4.

    gamma_prev: [L] float64 or None (no previous timestep: all INT8).
    alpha, beta: [L * n_linears] float32; layer (l, j) is entry l*J + j.
    """
    alpha = np.asarray(alpha, dtype=np.float32).astype(np.float64)
    beta = np.asarray(beta, dtype=np.float32).astype(np.float64)
    if gamma_prev is None:
        return np.ones(alpha.shape, dtype=np.uint8)
    g = np.repeat(np.asarray(gamma_prev, dtype=np.float64), n_linears)
    p = alpha * g + beta
    return (p > float(tau)).astype(np.uint8)


def predictions(gamma_prev, alpha, beta, n_linears):
    """p = alpha * Gamma_{t-1} + beta for every linear (float64)."""
    alpha = np.asarray(alpha, dtype=np.float32).astype(np.float64)
    beta = np.asarray(beta, dtype=np.float32).astype(np.float64)
    g = np.repeat(np.asarray(gamma_prev, dtype=np.float64), n_linears)
    return alpha * g + beta


def tau_for_half(p):
    """Threshold that sends about half of a population of predictions to
    INT8: the midpoint of the two middle values of the sorted population
    (for an odd count, the median itself, which then goes to NVFP4)."""
    s = np.sort(np.asarray(p, dtype=np.float64).ravel())
    n = len(s)
    if n == 0:
        raise ValueError("empty population")
    return 0.5 * (s[(n - 1) // 2] + s[n // 2])


def tdc_decide(t, d_prev, computed_prev, delta):
    """skip[l] = t >= 2 and computed_prev[l] and d_prev[l] < delta."""
    d_prev = np.asarray(d_prev, dtype=np.float64)
    computed_prev = np.asarray(computed_prev).astype(bool)
    if t < 2:
        return np.zeros(d_prev.shape, dtype=np.uint8)
    return (computed_prev & (d_prev < float(delta))).astype(np.uint8)


def rel_err_sums(yq_bits, yref_bits):
    """(sum (y_q - y)^2, sum y^2), each correctly rounded (exact terms)."""
    q = bf16_to_f64(yq_bits).ravel()
    r = bf16_to_f64(yref_bits).ravel()
    return _fsum((q - r) ** 2), _fsum(r ** 2)


def rel_err(s0, s1):
    """E_rel = sqrt(s0) / sqrt(s1) from the two sums."""
    return ratio(math.sqrt(s0), math.sqrt(s1))


def cosine_sums(new_bits, prev_bits):
    """(sum new*prev, sum new^2, sum prev^2), each correctly rounded."""
    a = bf16_to_f64(new_bits).ravel()
    b = bf16_to_f64(prev_bits).ravel()
    return _fsum(a * b), _fsum(a * a), _fsum(b * b)


def cosine(s0, s1, s2):
    """Cosine similarity from the three sums (0 when a norm is 0)."""
    den = math.sqrt(s1) * math.sqrt(s2)
    return 0.0 if den == 0.0 else s0 / den


def tdc_decide_cos(t, cos_prev, computed_prev, threshold):
    """skip[l] = t >= 2 and computed_prev[l] and cos_prev[l] > threshold."""
    c = np.asarray(cos_prev, dtype=np.float64)
    computed_prev = np.asarray(computed_prev).astype(bool)
    if t < 2:
        return np.zeros(c.shape, dtype=np.uint8)
    return (computed_prev & (c > float(threshold))).astype(np.uint8)


def fraction_to_f32(q):
    """A rational rounded to the nearest float32 (ties to even); |q| stays
    well inside the normal float32 range in every use here."""
    q = Fraction(q)
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # a in [2^e, 2^(e+1)): 24 significant bits -> unit 2^(e-23)
    scaled = a / Fraction(2) ** (e - 23)
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    return np.float32(sign * float(Fraction(m) * Fraction(2) ** (e - 23)))


def fit_line(x, y):
    """Least-squares (alpha, beta) of y = alpha x + beta, in exact rational
    arithmetic, rounded to float32."""
    xs = [Fraction(float(v)) for v in np.asarray(x, np.float64).ravel()]
    ys = [Fraction(float(v)) for v in np.asarray(y, np.float64).ravel()]
    n = len(xs)
    if n == 0:
        return np.float32(0.0), np.float32(0.0)
    mx, my = sum(xs) / n, sum(ys) / n
    sxx = sum((a - mx) ** 2 for a in xs)
    sxy = sum((a - mx) * (b - my) for a, b in zip(xs, ys))
    alpha = sxy / sxx if sxx else Fraction(0)
    return fraction_to_f32(alpha), fraction_to_f32(my - alpha * mx)


def calibrate(gamma, erel, n_linears):
    """Per-linear (alpha, beta) from gamma [T, L] and erel [T, L*J]: the
    pairs (gamma[t-1, l], erel[t, l*J + j]) for t >= 1 with both finite."""
    g = np.asarray(gamma, np.float64)
    e = np.asarray(erel, np.float64)
    T, L = g.shape
    J = n_linears
    alpha = np.zeros(L * J, np.float32)
    beta = np.zeros(L * J, np.float32)
    for l in range(L):
        for j in range(J):
            x = g[:T - 1, l]
            y = e[1:, l * J + j]
            ok = np.isfinite(x) & np.isfinite(y)
            alpha[l * J + j], beta[l * J + j] = fit_line(x[ok], y[ok])
    return alpha, beta


class BlockCache:
    """TDC state of one block: two-slot Delta ring, flags and the last d."""

    def __init__(self, summation="exact"):
        self.summation = summation
        self.ring = [None, None]
        self.last = 1            # the first Delta goes to slot 0
        self.n_stored = 0
        self.computed_prev = False
        self.d_prev = math.inf

    def delta_last(self):
        return self.ring[self.last] if self.n_stored else None

    def skip_output(self, in_bits):
        """A skipped step: output from the cached Delta; cache kept."""
        self.computed_prev = False
        return tdc_apply(in_bits, self.ring[self.last])

    def computed(self, in_bits, out_bits):
        """A computed step: store the new Delta, record d; returns sums."""
        delta_new, sums = tdc_update(in_bits, out_bits, self.delta_last(), self.summation)
        d = rel_l2(sums[2], sums[3]) if self.n_stored else math.inf
        self.last ^= 1
        self.ring[self.last] = delta_new
        self.n_stored = min(self.n_stored + 1, 2)
        self.computed_prev = True
        self.d_prev = d
        return delta_new, sums, d
