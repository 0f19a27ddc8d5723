"""Input-side fusion through the C ABI: raw projections in, bf16 o out.

The oracle forms q, k, alpha, beta from the same raw projections
(`oracle.fused_inputs`) and runs the float64 decode step. Bars:
* o (bf16): |o - o_ref| <= 1e-3 + 2^-8 |o_ref| (the step's 1e-3 plus the
  bf16 rounding of o, at most half a unit in the last place, 2^-9 relative);
* delta (float32): 1e-3;
* keys in the records, against the float64 normalisation (`oracle.unit_rows`):
  every element is one of the two bf16 values bracketing the exact value, and
  the exact value's nearest one wherever that is farther from their midpoint
  than the float32 error bound derived in tests/bf16_bounds.py (the kernel
  normalises in float32 before rounding, as the oracle's `fused_inputs` does
  with another summation order);
* alpha in the records: 1e-5 relative (float32 exp/log1p against float64).
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

EPS = 1e-6

if torch.cuda.is_available():
    import gpu_harness as gh
    from linear_attention_beam_gdn_amd import Onela, OnelaError
    from bf16_bounds import check_rounded, fp32_unit_rel_bound
    from oracle import full_state_episode, fused_inputs, unit_rows
    from workload import bf16_bits_to_f32, make_raw_episode, shape_of


def _run_raw(shape, ep):
    n, W, H = len(ep["reqs"]), shape.W, shape.H
    lay = Onela(n, H, shape.dk, shape.dv, W, shape.T)
    for i in range(n):
        lay.init_request(i, gh.to_dev(ep["S0"][i]))
    A, D = gh.to_dev(ep["A_log"]), gh.to_dev(ep["dt_bias"])
    o16 = torch.empty((n * W, H, shape.dv), dtype=torch.int16, device=gh.dev())
    d = torch.empty((n * W, H, shape.dv), dtype=torch.float32, device=gh.dev())
    outs = {"o": [], "delta": []}
    for t in range(shape.T):
        o16.fill_(-1)                  # NaN bits: a skipped write would stay NaN
        d.fill_(float("nan"))
        par = gh.to_dev(ep["parents"][t].astype(np.int32)) if t else None
        lay.step_raw(list(range(n)), *[gh.to_dev(ep[key][t]) for key in ("q_raw", "k_raw", "v", "a_raw", "b_raw")],
                     A, D, par, o16, d, norm_eps=EPS)
        lay.sync()
        outs["o"].append(bf16_bits_to_f32(o16.cpu().numpy().view(np.uint16)))
        outs["delta"].append(d.cpu().numpy().copy())
    outs["layer"] = lay
    return outs


def _oracle(shape, ep, i, h):
    sl = slice(i * shape.W, (i + 1) * shape.W)
    hs = slice(h, h + 1)
    q, k, a, b = fused_inputs(bf16_bits_to_f32(ep["q_raw"][:, sl, hs]), bf16_bits_to_f32(ep["k_raw"][:, sl, hs]),
                              ep["a_raw"][:, sl, hs], ep["b_raw"][:, sl, hs], ep["A_log"][hs], ep["dt_bias"][hs],
                              eps=EPS)
    ref = full_state_episode(ep["S0"][i, h], q[:, :, 0], k[:, :, 0], bf16_bits_to_f32(ep["v"][:, sl, h]),
                             a[:, :, 0], b[:, :, 0], ep["parents"][:, i, :])
    return ref, k[:, :, 0], a[:, :, 0]


def _check(shape, ep, outs, pairs):
    W, T = shape.W, shape.T
    for i, h in pairs:
        ref, kn, an = _oracle(shape, ep, i, h)
        for t in range(T):
            o = outs["o"][t][i * W:(i + 1) * W, h]
            bound = 1e-3 + 2.0 ** -8 * np.abs(ref["o"][t])
            gh.parity_log.record("o_bf16_rel", float(np.max(np.abs(o - ref["o"][t]) / bound)), 1.0)
            assert np.all(np.abs(o - ref["o"][t]) <= bound), (i, h, t)
            ed = gh.nan_max_abs(outs["delta"][t][i * W:(i + 1) * W, h], ref["delta"][t])
            gh.parity_log.record("delta", ed, 1e-3)
            assert ed <= 1e-3, (i, h, t)
        a_rec, _, k_rec = outs["layer"].get_records(i, h, T * W)
        k_gpu = bf16_bits_to_f32(k_rec).reshape(T, W, -1)
        u = unit_rows(bf16_bits_to_f32(ep["k_raw"][:, i * W:(i + 1) * W, h]), eps=EPS)
        bracket, exact, n_band, n_diff = check_rounded(k_gpu, u, fp32_unit_rel_bound(shape.dk))
        gh.parity_log.record("key_elements_off_nearest", float(n_diff), float(n_band))
        assert bracket and exact, (i, h, n_band, n_diff)
        np.testing.assert_allclose(a_rec.reshape(T, W), an, rtol=1e-5)


@pytest.mark.parametrize("cfg,over", [
    (0, {}),
    (1, {"R": 2, "H": 3, "T": 3}),
    (0, {"name": "fused_ragged", "W": 65, "T": 4, "H": 2, "dk": 64, "dv": 64, "R": 2}),
])
def test_fused_matches_oracle(cfg, over):
    shape = shape_of(cfg, **over)
    ep = make_raw_episode(shape)
    print(f"[fused] {shape.name} W={shape.W} T={shape.T} H={shape.H} d={shape.dk}", flush=True)
    outs = _run_raw(shape, ep)
    _check(shape, ep, outs, [(i, h) for i in range(len(ep["reqs"])) for h in range(shape.H)])
    outs["layer"].close()


def test_fused_bench_size_sampled():
    """The 32-request, W = 256, d = 128 workload from raw projections, at full
    size in the bench's launch configuration; three sampled (request, head)
    pairs against the oracle."""
    shape = shape_of(3)
    ep = make_raw_episode(shape)
    print(f"[fused] {shape.name}", flush=True)
    outs = _run_raw(shape, ep)
    _check(shape, ep, outs, [(0, 0), (13, 7), (31, 15)])
    outs["layer"].close()


def test_fused_argument_errors():
    shape = shape_of(0)
    ep = make_raw_episode(shape)
    lay = Onela(1, shape.H, 32, 32, shape.W, shape.T)
    lay.init_request(0, gh.to_dev(ep["S0"][0]))
    ins = [gh.to_dev(ep[key][0]) for key in ("q_raw", "k_raw", "v", "a_raw", "b_raw")]
    o16 = torch.empty((shape.W, shape.H, 32), dtype=torch.int16, device=gh.dev())
    A, D = gh.to_dev(ep["A_log"]), gh.to_dev(ep["dt_bias"])
    with pytest.raises(OnelaError) as e:
        lay.step_raw([0], *ins, A, D, None, o16, norm_eps=-1.0)     # negative epsilon
    assert e.value.status == -1
    lay.step_raw([0], *ins, A, D, None, o16)
    lay.sync()
    assert lay.get_step(0) == 1
    lay.close()
