"""The bench's measurement probes compute what they claim to: the copy
copies, and the projection probe's row sums equal S0 times the sum of the
vectors (the projection is linear), within the split-bf16 representation's
error of S0 (2^-17 relative per element)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_harness as gh
    from linear_attention_beam_gdn_amd import probes
    from workload import bf16_bits_to_f32, shape_of


def test_copy_probe():
    src = torch.randn(1 << 20, device=gh.dev())
    dst = torch.empty_like(src)
    probes.copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_mfma_probe_runs():
    out = torch.zeros(4 * 512, device=gh.dev())
    probes.mfma_loop(out, 4, 10)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and out.abs().sum() > 0


def test_projection_probe_equals_s0_times_vector_sum():
    shape = shape_of(1, R=2, H=3, T=1)
    ep, S0 = gh.episode(shape)
    W = shape.W
    colsum = torch.empty((shape.R * shape.H, 128), device=gh.dev())
    pl = probes.planes(gh.to_dev(S0))
    probes.projection(pl, gh.to_dev(ep["k"][0]), gh.to_dev(ep["q"][0]), W, colsum)
    got = colsum.cpu().numpy().reshape(shape.R, shape.H, 128)
    x = (bf16_bits_to_f32(ep["k"][0]).astype(np.float64) + bf16_bits_to_f32(ep["q"][0])).reshape(shape.R, W, shape.H, 128)
    xs = x.sum(axis=1)                                          # [R][H][dk]
    want = np.einsum("rhij,rhj->rhi", S0.astype(np.float64), xs)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-3)
    # operands of pairs 0 and 1 only: workgroup p reproduces pair p mod 2
    probes.projection(pl, gh.to_dev(ep["k"][0]), gh.to_dev(ep["q"][0]), W, colsum, resident_pairs=2)
    res = colsum.cpu().numpy()
    flat = got.reshape(-1, 128)
    for p in range(shape.R * shape.H):
        np.testing.assert_array_equal(res[p], flat[p % 2])
