"""Host-side logic: work accounting and the seeded input generator (CPU only)."""
import numpy as np

import synth
from block_scaled_mxfp8_amd.flops import attn_flops, visible_pairs, visible_pairs_causal


def test_visible_pairs_worked_examples_flamia_section6():
    # 65,536 tokens: 16 documents of 4096 -> 134,250,496 visible pairs;
    # one 8192-token document plus 224 of 256 tokens -> 40,927,232.
    assert visible_pairs_causal([4096] * 16) == 134_250_496
    assert visible_pairs_causal([8192] + [256] * 224) == 40_927_232
    lens = np.array([5, 17, 300, 1])
    assert visible_pairs_causal(lens) == (lens.sum() + (lens ** 2).sum()) // 2


def test_headline_flop_counts():
    pairs = visible_pairs(4, 32, 4096, causal=True)
    assert pairs == 1_074_003_968
    assert attn_flops(pairs, 128) == 549_890_031_616
    assert attn_flops(pairs, 128, backward=True) == 1_374_725_079_040
    assert visible_pairs(1, 16, 16384, causal=False) == 16 * 16384 ** 2


def test_generator_is_deterministic_and_shaped():
    a = synth.make_inputs("c2", batch=1, heads=2, seqlen=64)
    b = synth.make_inputs("c2", batch=1, heads=2, seqlen=64)
    for t in ("q", "k", "v", "g"):
        assert a[t].shape == (1, 2, 64, 128) and a[t].dtype == np.float32
        assert np.array_equal(a[t], b[t])
    # two outlier channels per (tensor, head) on q/k/v, none on g
    for t in ("q", "k", "v"):
        col = np.abs(a[t][0, 0]).mean(axis=0)
        assert np.sum(col > 10) == 2
    assert np.sum(np.abs(a["g"][0, 0]).mean(axis=0) > 10) == 0


def test_generator_packed_lengths():
    cfg = synth.CONFIGS["c4"]
    lens = synth.doc_lengths(synth.SEED_BASE["c4"], cfg["n_docs"], cfg["median"], cfg["sigma"], cfg["min_len"], cfg["max_len"])
    assert len(lens) == 128 and lens.min() >= 32 and lens.max() <= 2048
    assert 150 < np.median(lens) < 700
    cu = synth.cu_seqlens_of(lens)
    assert cu[0] == 0 and cu[-1] == lens.sum() and cu.dtype == np.int32


def test_generator_magnitude_is_per_token():
    x = synth.make_inputs("c5", seqlen=256, tensors=("q",))["q"]
    # u ~ U(0.5, 4) is shared by all heads and channels of a token
    r = np.abs(x).mean(axis=(1, 3))[0]
    assert r.min() > 0.2 and r.max() < 4.0


def test_backward_step_cursor_matches_the_layout_formulas(tmp_path):
    # The backward producers walk their (head, 64-query step) positions by additions
    # (mx_layout.h step_walk / step_next); a host build of that header checks every step of many
    # batched and packed geometries against the closed address formulas.
    import os
    import shutil
    import subprocess
    import pytest
    hipcc = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)
    if hipcc is None:
        pytest.skip("hipcc not available")
    here = os.path.dirname(os.path.abspath(__file__))
    exe = str(tmp_path / "step_walk_check")
    subprocess.run([hipcc, "-O1", "-std=c++17", os.path.join(here, "host_cpp", "step_walk_check.cpp"), "-o", exe],
                   check=True, capture_output=True)
    out = subprocess.run([exe], capture_output=True, text=True)
    print(out.stdout)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "0 mismatches" in out.stdout
