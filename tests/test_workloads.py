"""The seeded input generator: bf16 rounding and determinism."""
import numpy as np
import torch

import workloads


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 3.0e38, 1e-40,
                                  -0.0, 0.0, np.float32(1.00390625)], dtype=np.float32)])
    ours = workloads.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()


def test_deterministic_and_independent_of_selection():
    a = workloads.layer_inputs(64, 32, 16, 4, "bf16", seed=0)
    b = workloads.layer_inputs(64, 32, 16, 4, "bf16", seed=0, which=("X",))
    c = workloads.layer_inputs(64, 32, 16, 4, "bf16", seed=1)
    assert (a["X"] == b["X"]).all()
    assert not (a["X"] == c["X"]).all()
    assert a["W"].shape == (32, 64) and a["L"].shape == (64, 4) and a["R"].shape == (4, 32)
    assert a["W"].dtype == np.uint16


def test_threading_does_not_change_draws():
    s = np.random.SeedSequence([0, 0])
    a = workloads.draw(s, (3000, 40), 0.02, "bf16", threads=1)
    b = workloads.draw(s, (3000, 40), 0.02, "bf16", threads=8)
    assert (a == b).all()


def test_scales():
    d = workloads.layer_inputs(256, 512, 512, 8, "f32", seed=0)
    assert abs(workloads.bits_to_float32(d["W"]).std() - 0.02) < 0.001
    assert abs(workloads.bits_to_float32(d["X"]).std() - 1.0) < 0.02
