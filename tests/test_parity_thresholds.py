"""The bound-free parity thresholds (tests/metrics.py REL_L2_MAX, FRAC_MAX) against the oracle's
own perturbation runs, CPU only.

A perturbation run replaces every FP32 quantity the oracle budgets (the exponent argument x,
E - D, D, the output products) by a uniform random value inside its budget, which is what
legitimate rounding of a device implementation can produce. The thresholds are 3 x the
largest rel-L2 and over-2e-2-rms fraction such runs produced over the calibration cases (the
cases below, and for FP16 dQ c3 at L = 4096, whose perturbation rel-L2 was 7.7e-3); this test
re-runs the small cases and checks the margin still holds.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.metrics import FRAC_MAX, REL_L2_MAX, rel_l2, rms

CASES = [("c1", 256, 64, True, "f32"), ("c3", 512, 128, True, "f16"), ("c2", 256, 128, True, "f32"),
         ("c5", 256, 128, False, "f32"), ("c3", 200, 128, False, "f32")]
MARGIN = 3.0


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-L{c[1]}-{c[4]}")
def test_thresholds_keep_their_margin_over_perturbation_runs(case):
    cfg, L, d, causal, dqm = case
    x = synth.make_inputs(cfg, batch=1, heads=1, seqlen=L)
    q, k, v, g = (oracle.round_to(np.asarray(x[n][0, 0, :, :d], np.float64), "bf16") for n in "qkvg")
    f = oracle.head_forward(q, k, v, causal)
    b = oracle.head_backward(q, k, v, f["O_out"], f["lse"], g, causal, dq_mode=dqm)
    for seed in range(2):
        r = np.random.default_rng(seed)

        def pert(name, value, budget):
            return value + budget * r.uniform(-1, 1, np.shape(value))

        fp = oracle.head_forward(q, k, v, causal, perturb=pert)
        bp = oracle.head_backward(q, k, v, f["O_out"], f["lse"], g, causal, perturb=pert, dq_mode=dqm)
        for name, ref, per in (("O", f["O"], fp["O"]), ("dQ", b["dQ"], bp["dQ"]), ("dK", b["dK"], bp["dK"]),
                               ("dV", b["dV"], bp["dV"])):
            key = "dQ16" if (name == "dQ" and dqm == "f16") else name
            rl = rel_l2(per, ref)
            frac = np.mean(np.abs(per - ref) > 2e-2 * rms(ref))
            print(f"{cfg} L{L} {dqm} seed {seed} {name}: rel-L2 {rl:.2e} frac {frac:.1e}")
            assert rl * MARGIN <= REL_L2_MAX[key], (name, rl)
            assert frac * MARGIN <= FRAC_MAX, (name, frac)
