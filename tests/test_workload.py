"""The seeded input generator: determinism, codec and the shapes of the workloads."""
import numpy as np
import torch

from workload import WORKLOADS, bf16_bits_to_f32, decode_inputs, f32_to_bf16_bits, make_episode, shape_of
from workload.gen import parents_for, prompt_tokens


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(size=10000).astype(np.float32),
                        np.float32([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 0.0, -0.0, 3.0e38, 1e-40])])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    # ties go to even
    assert bf16_bits_to_f32(f32_to_bf16_bits(np.float32([1 + 2**-8])))[0] == 1.0
    assert bf16_bits_to_f32(f32_to_bf16_bits(np.float32([1 + 3 * 2**-8])))[0] == 1 + 2**-6


def test_decode_inputs_deterministic_and_per_request():
    s = shape_of(0)
    a, b = decode_inputs(s, 0), decode_inputs(s, 0)
    for key in a:
        assert a[key].tobytes() == b[key].tobytes()
    s1 = shape_of(1)
    c = decode_inputs(s1, 0)
    assert c["q"].shape == (3, 256, 16, 128) and c["q"].dtype == np.uint16
    assert c["alpha"].dtype == np.float32
    # unit-norm keys up to bf16 rounding
    kn = np.linalg.norm(bf16_bits_to_f32(c["k"]).astype(np.float64), axis=-1)
    assert np.all(np.abs(kn - 1) < 1e-2)
    assert np.all((c["alpha"] > 0) & (c["alpha"] < 1)) and np.all((c["beta"] > 0) & (c["beta"] < 1))


def test_requests_independent_of_batch():
    s = shape_of(3)
    ep = make_episode(s, reqs=[5])
    one = decode_inputs(s, 5)
    assert ep["q"].tobytes() == one["q"].tobytes()
    assert np.array_equal(ep["parents"][:, 0], parents_for(s, 5))


def test_parent_rules_in_range():
    for cfg in range(len(WORKLOADS)):
        s = WORKLOADS[cfg]
        p = parents_for(s, 0)
        assert p.shape == (s.T, s.W)
        assert np.all(p[0] == -1)
        assert p[1:].min() >= 0 and p[1:].max() < s.W


def test_topw4_clusters():
    s = shape_of(1)
    p = parents_for(s, 0)
    # survivors of "top W of 4W" come from fewer than W distinct parents
    assert len(np.unique(p[1])) < s.W


def test_prompt_tokens_shape():
    s = shape_of(2)
    pt = prompt_tokens(s, 0, length=16)
    assert pt["k"].shape == (16, 16, 128) and pt["alpha"].shape == (16, 16)
