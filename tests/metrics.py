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


# Bound-free gates. Thresholds: 3 x the largest value the oracle's own uniform perturbation
# inside its budget gave over the calibration cases (tests/test_parity_thresholds.py re-derives
# them on the CPU): rel-L2(dev - oracle) per output, and the fraction of elements with
# |dev - oracle| > 2e-2 rms. A few-percent systematic error fails the rel-L2 gate.
REL_L2_MAX = {"O": 6e-3, "dQ": 6e-3, "dQ16": 2.5e-2, "dK": 1e-2, "dV": 1e-2}
FRAC_MAX = 2e-3
REL = 2e-2


class Gate:
    """Result of the parity gates for one output of one case (see ``gate``)."""

    def __init__(self, name, x_dev, x_ref, B, eta, rounding, rel_tol, rel_l2_max, frac_max):
        x_dev = np.asarray(x_dev, np.float64)
        x_ref = np.asarray(x_ref, np.float64)
        B = np.broadcast_to(np.asarray(B, np.float64), x_ref.shape)
        eta = np.broadcast_to(np.asarray(eta, np.float64), x_ref.shape) + rounding
        self.name = name
        r = rms(x_ref)
        self.rms = r
        diff = np.abs(x_dev - x_ref)
        excess = diff - (rel_tol * r + B + eta)
        n = max(1, diff.size)
        self.elem_ok = bool(np.all(excess <= 0))
        self.worst = float(excess.max() / r) if diff.size and r > 0 else 0.0
        self.plain = float(diff.max() / r) if diff.size and r > 0 else 0.0
        self.rel_l2 = rel_l2(x_dev, x_ref) if diff.size and r > 0 else 0.0
        self.frac = float(np.count_nonzero(diff > rel_tol * r + rounding)) / n
        self.b_count = int(np.count_nonzero(B))
        self.b_density = self.b_count / n
        self.b_med = float(np.median(B) / r) if diff.size and r > 0 else 0.0
        self.allow_med = float(np.median(B + eta) / r) if diff.size and r > 0 else 0.0
        self.rel_l2_max, self.frac_max = rel_l2_max, frac_max
        self.ok = self.elem_ok and self.rel_l2 <= rel_l2_max and self.frac <= frac_max
        i = np.unravel_index(np.argmax(diff), diff.shape) if diff.size else None
        self.where = (tuple(int(t) for t in i), float(x_dev[i]), float(x_ref[i]), float((B + eta)[i] / r)) if i else None

    def __str__(self):
        s = (f"{self.name}: plain max|d|/rms {self.plain:.3e}, rel-L2 {self.rel_l2:.2e} (<= {self.rel_l2_max:.0e}), "
             f"frac>2e-2 {self.frac:.1e} (<= {self.frac_max:.0e}), worst excess {self.worst:.2e}, "
             f"B>0 {self.b_count} ({self.b_density:.3f}), median B/rms {self.b_med:.1e}, "
             f"median allowance/rms {self.allow_med:.1e}")
        if self.where:
            s += f"; worst at {self.where[0]} dev {self.where[1]:.5g} ref {self.where[2]:.5g} allowance/rms {self.where[3]:.2e}"
        return s


def gate(name, x_dev, x_ref, B, eta, out_dtype="bf16", rel_tol=REL, rel_l2_max=None, frac_max=FRAC_MAX, key=None):
    """The parity gates of one output: elementwise |dev - ref| <= rel_tol rms(ref) + B + eta + r
    (B: the oracle's ambiguity bound, eta: its accumulation allowance, r: half an ulp of the
    output storage type at the device value), rel-L2(dev - ref) <= REL_L2_MAX[key or name], and
    the fraction of elements with |dev - ref| > rel_tol rms(ref) + r at most frac_max (the
    storage rounding is not an error of the method). Prints the case line, returns a Gate."""
    from oracle import ulp_of
    rounding = ulp_of(x_dev, out_dtype) / 2
    g = Gate(name, x_dev, x_ref, B, eta, rounding, rel_tol,
             REL_L2_MAX[key or name] if rel_l2_max is None else rel_l2_max, frac_max)
    print("  " + str(g), flush=True)
    return g
