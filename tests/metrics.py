"""Comparison metrics used by the parity tests (plain numpy, float64)."""
import numpy as np


def rms(x):
    x = np.asarray(x, np.float64)
    return float(np.sqrt(np.mean(x * x))) if x.size else 0.0


def cosine(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(a @ b / (na * nb))


def rel_l2(a, ref):
    a = np.asarray(a, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    return float(np.linalg.norm(a - ref) / np.linalg.norm(ref))


def sqnr_db(a, ref):
    """Signal-to-quantisation-noise ratio of a against ref, in dB."""
    a = np.asarray(a, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    return float(10 * np.log10(np.sum(ref * ref) / max(np.sum((a - ref) ** 2), 1e-300)))


def gate(x_dev, x_ref, allowance, rel_tol=2e-2):
    """Elementwise parity gate |x_dev - x_ref| <= rel_tol * rms(x_ref) + allowance.

    Returns (ok, worst excess over the gate in units of rms, plain max|diff|/rms, number of
    elements with a non-zero allowance).
    """
    x_dev = np.asarray(x_dev, np.float64)
    x_ref = np.asarray(x_ref, np.float64)
    r = rms(x_ref)
    diff = np.abs(x_dev - x_ref)
    excess = diff - (rel_tol * r + allowance)
    plain = float(diff.max() / r) if diff.size and r > 0 else 0.0
    worst = float(excess.max() / r) if diff.size and r > 0 else 0.0
    return bool(np.all(excess <= 0)), worst, plain, int(np.count_nonzero(allowance))
