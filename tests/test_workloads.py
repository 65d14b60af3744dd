"""Checks of the seeded input generator (no mLSTM arithmetic involved)."""
import numpy as np
import torch

from workloads import WORKLOADS, WORKLOAD_ORDER, head_inputs, make_inputs, round_to_bf16, sha256_of


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-6, 6, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 3.0e38], np.float32)])
    vals, bits = round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16)
    np.testing.assert_array_equal(vals, ref.to(torch.float32).numpy())
    np.testing.assert_array_equal(bits, ref.view(torch.int16).numpy().view(np.uint16))


def test_generator_is_deterministic_and_per_head():
    w = WORKLOADS["bf16_s2048_d128"].replace(S=64)
    a = make_inputs(w)
    b = make_inputs(w)
    for key in a:
        assert sha256_of(a[key]) == sha256_of(b[key])
    # a single head drawn alone equals the same head inside the full draw
    one = head_inputs(w, 3, 5)
    for key in one:
        np.testing.assert_array_equal(a[key][3, 5], one[key])
    # heads differ
    assert not np.array_equal(a["q"][0, 0], a["q"][0, 1])


def test_workload_shapes_and_distributions():
    names = set(WORKLOAD_ORDER)
    assert names == set(WORKLOADS)
    w = WORKLOADS["bf16_7b_s65536"]
    x = head_inputs(w, 0, 2, S=4096)
    assert x["q"].shape == (4096, 256) and x["v"].shape == (4096, 512)
    assert x["C0"].shape == (256, 512) and x["n0"].shape == (256,)
    assert 0.08 < x["C0"].std() < 0.12
    assert x["n0"].min() >= 0.0 and x["n0"].max() <= 1.0
    assert x["f"].min() >= 2.0 and x["f"].max() <= 6.0
    # bf16 inputs hold bf16-representable values
    np.testing.assert_array_equal(round_to_bf16(x["q"])[0], x["q"])
    w2 = WORKLOADS["bf16_s2048_d128"]
    y = head_inputs(w2, 1, 1)
    spikes = (y["i"] > 6.0).mean()
    assert 0.003 < spikes < 0.03
    assert 1.7 < np.std(y["i"][y["i"] < 6.0]) < 2.3
