"""The full-state comparator (a d_v x d_k state per beam) through the C ABI.

It runs the same recurrence the float64 oracle defines, so it must match the
oracle within the same max-abs 1e-3, and match the OneLA path on identical
inputs; its persistent memory must be W*(2 copies) full states per head.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_harness as gh
    from linear_attention_beam_gdn_amd import FullState, OnelaError
    from workload import shape_of


def _run_fs(shape, ep, S0):
    n = len(ep["reqs"])
    fs = FullState(n, shape.H, shape.dk, shape.dv, shape.W, shape.T)
    for i in range(n):
        fs.init_request(i, gh.to_dev(S0[i]))
    o = torch.empty((n * shape.W, shape.H, shape.dv), dtype=torch.float32, device=gh.dev())
    d = torch.empty_like(o)
    out = {"o": [], "delta": []}
    for t in range(shape.T):
        par = gh.to_dev(ep["parents"][t].astype(np.int32)) if t else None
        fs.step(list(range(n)), gh.to_dev(ep["q"][t]), gh.to_dev(ep["k"][t]), gh.to_dev(ep["v"][t]),
                gh.to_dev(ep["alpha"][t]), gh.to_dev(ep["beta"][t]), par, o, d)
        fs.sync()
        out["o"].append(o.cpu().numpy().copy())
        out["delta"].append(d.cpu().numpy().copy())
    return fs, out


@pytest.mark.parametrize("cfg", [0, 1, 2])
def test_fullstate_matches_oracle(cfg):
    shape = shape_of(cfg)
    ep, S0 = gh.episode(shape)
    print(f"[fullstate] {shape.name}", flush=True)
    fs, out = _run_fs(shape, ep, S0)
    worst = 0.0
    for i in range(shape.R):
        for h in range(shape.H):
            ref = gh.oracle_pair(shape, ep, S0, i, h)
            eo, ed = gh.max_err(out, ref, i, h, shape.W)
            worst = max(worst, eo, ed)
            assert eo <= gh.TOL and ed <= gh.TOL, (i, h, eo, ed)
    print(f"[fullstate] {shape.name}: worst max-abs err {worst:.3e}")
    fs.close()


def test_fullstate_agrees_with_onela_at_bench_size():
    shape = shape_of(3)
    ep, S0 = gh.episode(shape)
    print(f"[fullstate] {shape.name} vs the OneLA path", flush=True)
    fs, out = _run_fs(shape, ep, S0)
    fs.close()
    ol = gh.run_episode(shape, ep, S0)
    ol["layer"].close()
    for t in range(shape.T):
        assert np.abs(out["o"][t] - ol["o"][t]).max() <= gh.TOL
        assert np.abs(out["delta"][t] - ol["delta"][t]).max() <= gh.TOL
    ref = gh.oracle_pair(shape, ep, S0, 7, 3)
    eo, ed = gh.max_err(out, ref, 7, 3, shape.W)
    assert eo <= gh.TOL and ed <= gh.TOL


def test_fullstate_bad_parent_and_memory():
    shape = shape_of(0, H=2)
    ep, S0 = gh.episode(shape)
    fs = FullState(1, shape.H, 32, 32, shape.W, shape.T)
    assert fs.memory() == 4 * 32 * 32 * shape.H * (2 * shape.W + 1)
    fs.init_request(0, gh.to_dev(S0[0]))
    o = torch.empty((shape.W, shape.H, 32), dtype=torch.float32, device=gh.dev())
    ins = lambda t: [gh.to_dev(ep[key][t]) for key in ("q", "k", "v", "alpha", "beta")]
    fs.step([0], *ins(0), None, o)
    par = ep["parents"][1].astype(np.int32).copy()
    par[0, 2] = -5
    fs.step([0], *ins(1), gh.to_dev(par), o)
    with pytest.raises(OnelaError) as e:
        fs.sync()
    assert e.value.status == -4
    fs.reset(0)
    fs.sync()
    fs.close()
