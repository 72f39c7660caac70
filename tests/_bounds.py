"""Derived error bounds for the bf16 parity checks (test infrastructure).

The bf16 backward takes O from the forward, rounded to bf16, and forms
D_i = sum_c dO_ic O_ic from it ("attention backprop", section "Gradient of
S"); it also rounds P and dS to bf16 before they enter the MFMA products
(dV = P^T dO, dQ = scale dS K, dK = scale dS^T Q, sections "Gradient of V and
P" and "Gradient of Q and K").  At unit-scale inputs these roundings stay
inside the 2e-2 bf16 tolerance.  With larger scores (near one-hot rows) the
exact dS = P (dP - D) cancels while the error that D inherits from the bf16 O
does not, and dK = scale dS^T Q multiplies every dS error by |Q|.

The model (probabilistic rounding-error analysis: every bf16 rounding is an
independent error, uniform within +-u|x|, u = 2^-8 for round-to-nearest-even
with 8 significant bits, variance u^2 x^2 / 3):
  O  : var(O^_ic - O_ic)   = u^2/3 (O_ic^2 + sum_j P_ij^2 V_jc^2)
       (the forward's P rounded for P V, then O rounded on output)
  D  : var(dD_i)           = sum_c dO_ic^2 var(O^_ic - O_ic)
  dQ : var(dQ^_ic - dQ_ic) = scale^2 (var(dD_i) (P K)_ic^2 + u^2/3 sum_j dS_ij^2 K_jc^2)
       (dD_i enters every dS_ij of row i as -P_ij dD_i: fully correlated)
  dK : var(dK^_jc - dK_jc) = scale^2 sum_i (P_ij^2 var(dD_i) + u^2/3 dS_ij^2) Q_ic^2
  dV : var(dV^_jc - dV_jc) = u^2/3 sum_i P_ij^2 dO_ic^2
An element is accepted when |x - r| <= max(tol, tol |r|) (the stated bf16
tolerance) or |x - r| <= 6 sigma + u |r| (the derived bound; u |r| is the
output's own rounding).  tests/test_error_model.py pins the model against a
float64 emulation of the same rounding steps.
"""
import numpy as np

from oracle import causal_blocked, dense_forward

U_BF16 = 2.0 ** -8
N_SIGMA = 6.0


def bf16_backward_parts(q, k, v, dout, scale, causal):
    """float64 P, O and dS of one head (full matrices; small sizes only)."""
    o, lse = dense_forward(q, k, v, scale, causal)
    s = scale * (q @ k.T)
    if causal:
        s = np.where(causal_blocked(s.shape[0], s.shape[1]), -np.inf, s)
    with np.errstate(invalid="ignore"):
        p = np.where(np.isneginf(s), 0.0, np.exp(s - lse[:, None]))
    dp = dout @ v.T
    ds = p * (dp - np.sum(dout * o, axis=1, keepdims=True))
    return p, o, ds


def bf16_backward_sigma(q, k, v, dout, scale, causal):
    """Standard deviation of the bf16 backward's error per element of dQ, dK
    and dV under the model above (float64 inputs of one head)."""
    u2 = U_BF16 ** 2 / 3.0
    p, o, ds = bf16_backward_parts(q, k, v, dout, scale, causal)
    var_o = u2 * (o ** 2 + (p ** 2) @ (v ** 2))
    var_d = np.sum(dout ** 2 * var_o, axis=1, keepdims=True)
    s_dq = np.sqrt(scale ** 2 * (var_d * (p @ k) ** 2 + u2 * (ds ** 2) @ (k ** 2)))
    s_dk = np.sqrt(scale ** 2 * ((p ** 2 * var_d).T @ (q ** 2) + u2 * (ds ** 2).T @ (q ** 2)))
    s_dv = np.sqrt(u2 * (p ** 2).T @ (dout ** 2))
    return s_dq, s_dk, s_dv


def assert_close_or_within_model(name, x, ref, tol, sigma):
    """Element-wise: |x - r| <= max(tol, tol |r|), or within the derived
    bound 6 sigma + u |r|."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(x - ref)
    ok = (d <= tol) | (d <= tol * np.abs(ref)) | (d <= N_SIGMA * sigma + U_BF16 * np.abs(ref))
    ok &= np.isfinite(x)
    assert ok.all(), (f"{name}: {int((~ok).sum())} elements outside both the tolerance {tol} and the derived "
                      f"bound (max abs err {d.max():.3e}, max err / bound "
                      f"{np.max(d / (N_SIGMA * sigma + U_BF16 * np.abs(ref) + 1e-300)):.3f})")


# Per-row magnitude check for rows with many contributing terms: the largest
# error of a row against the row's RMS.  Each element carries one or two bf16
# roundings of its product operands (u/sqrt(3) of the row's RMS each, in the
# model above) and its own output rounding; the largest of a row's 64 or 128
# elements stays within about 3.5 sigma, i.e. about 0.016 of the RMS (a float64
# emulation of one L=4096 causal head and one L=2048 head gives at most 0.020
# over every row with at least 64 terms).  0.06 leaves three times that; a row
# that is off by a factor of 1 +- 0.1 gives at least 0.18.
ROW_REL_BOUND = 0.06
# LSE at full size: fp32 scores from exact bf16 products, a row sum of up to
# 65536 fp32 terms and a log, all well under 1e-5 for these magnitudes (the
# small-size checks measure about 1e-6); the bound allows ten times that.
LSE_ABS_BOUND = 1e-4


def assert_rows_match(name, x, ref, bound=ROW_REL_BOUND):
    """max_c |x_rc - r_rc| <= bound * rms_c(r_rc) for every row r (rows given
    as the leading axis)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref ** 2, axis=1))
    worst = np.max(np.abs(x - ref), axis=1)
    ratio = worst / np.maximum(rms, 1e-300)
    assert np.all(ratio <= bound), (f"{name}: row max|err|/rms(ref) up to {ratio.max():.4f} "
                                    f"(bound {bound}) at row index {int(np.argmax(ratio))} of the checked set")
