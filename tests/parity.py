"""Comparison rules shared by the parity tests.

fp32 state (master, momentum, variance): pass when
    |x - x*| <= 1e-6 * max(|x*|, s)
with s the operand scale of the last update (the sum of the magnitudes of the
terms that produced x*), so that elements where the terms nearly cancel are
judged against the size of the terms rather than the tiny result.
fp16 parameters: at most 1 unit apart in sign-magnitude order.
Integer work (layouts, flags, packed bits): exact.
"""

import numpy as np

RTOL = 1e-6


def fp16_ordered(u16: np.ndarray) -> np.ndarray:
    """Map fp16 bit patterns to integers that are ordered like the values
    (+0 and -0 both map to 0)."""
    u = np.asarray(u16).view(np.uint16).astype(np.int32)
    mag = u & 0x7FFF
    return np.where(u & 0x8000, -mag, mag)


def fp16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return np.abs(fp16_ordered(a) - fp16_ordered(b))


def scaled_close(x: np.ndarray, ref: np.ndarray, scale: np.ndarray, rtol: float = RTOL):
    """Boolean mask of elements within rtol * max(|ref|, scale)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = rtol * np.maximum(np.abs(ref), np.abs(np.asarray(scale, dtype=np.float64)))
    return np.abs(x - ref) <= bound


def assert_scaled_close(x, ref, scale, what: str, rtol: float = RTOL):
    ok = scaled_close(x, ref, scale, rtol)
    if not ok.all():
        bad = np.flatnonzero(~ok)
        i = bad[0]
        raise AssertionError(
            f"{what}: {bad.size} of {ok.size} elements outside {rtol:g} scaled "
            f"tolerance; first at {i}: got {x[i]!r}, want {ref[i]!r}, scale {np.asarray(scale)[i] if np.ndim(scale) else scale!r}")


def assert_fp16_close(a, b, what: str, max_ulp: int = 1):
    d = fp16_ulp_distance(a, b)
    if (d > max_ulp).any():
        bad = np.flatnonzero(d > max_ulp)
        i = bad[0]
        raise AssertionError(
            f"{what}: {bad.size} of {d.size} fp16 values more than {max_ulp} ulp apart; "
            f"first at {i}: got {int(np.asarray(a).view(np.uint16)[i]):#06x}, "
            f"want {int(np.asarray(b).view(np.uint16)[i]):#06x}")


def adam_operand_scales(m_prev, v_prev, p_prev, g_mag, p_new, beta1, beta2,
                        lr=None, t=None, v_new=None, eps=None):
    """Operand scales for the momentum, variance and parameter updates.
    g_mag is the magnitude of the gradient's terms.  When lr, t, v_new and
    eps are given, the parameter scale also carries the momentum's operand
    scale through the update (a momentum that cancels to near zero makes the
    update tiny, but its error is set by the size of the cancelled terms)."""
    f = np.float64
    g_mag = np.abs(np.asarray(g_mag, dtype=f))
    s_m = np.abs(f(beta1) * m_prev.astype(f)) + (1 - f(beta1)) * g_mag
    s_v = np.abs(f(beta2) * v_prev.astype(f)) + (1 - f(beta2)) * g_mag ** 2
    s_p = np.abs(p_prev.astype(f)) + np.abs(p_new.astype(f) - p_prev.astype(f))
    if lr is not None:
        bc1 = 1 - f(beta1) ** t
        bc2 = 1 - f(beta2) ** t
        den = np.sqrt(v_new.astype(f) / bc2) + f(eps)
        s_p = s_p + f(lr) * (s_m / bc1) / den
    return s_m, s_v, s_p
