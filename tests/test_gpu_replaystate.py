"""The replay comparator (every beam rebuilds its state from S0 and its own
ancestral records at every step) through the C ABI.

It runs the recurrence the float64 oracle defines, so it must match the
oracle within the same max-abs 1e-3 on o and delta, and the OneLA path on
identical inputs; its persistent memory is S0, the records and the parents.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_harness as gh
    from linear_attention_beam_gdn_amd import OnelaError, ReplayState
    from workload import shape_of


def _run_rs(shape, ep, S0, reqs=None):
    n = len(ep["reqs"])
    reqs = list(range(n)) if reqs is None else reqs
    rs = ReplayState(max(reqs) + 1, shape.H, shape.dk, shape.dv, shape.W, shape.T)
    for i, r in enumerate(reqs):
        rs.init_request(r, gh.to_dev(S0[i]))
    o = torch.empty((n * shape.W, shape.H, shape.dv), dtype=torch.float32, device=gh.dev())
    d = torch.empty_like(o)
    out = {"o": [], "delta": []}
    for t in range(shape.T):
        par = gh.to_dev(ep["parents"][t].astype(np.int32)) if t else None
        rs.step(reqs, gh.to_dev(ep["q"][t]), gh.to_dev(ep["k"][t]), gh.to_dev(ep["v"][t]),
                gh.to_dev(ep["alpha"][t]), gh.to_dev(ep["beta"][t]), par, o, d)
        rs.sync()
        out["o"].append(o.cpu().numpy().copy())
        out["delta"].append(d.cpu().numpy().copy())
    return rs, out


def _check_all(shape, ep, S0, out):
    worst = 0.0
    for i in range(len(ep["reqs"])):
        for h in range(shape.H):
            ref = gh.oracle_pair(shape, ep, S0, i, h)
            eo, ed = gh.max_err(out, ref, i, h, shape.W)
            worst = max(worst, eo, ed)
            assert eo <= gh.TOL and ed <= gh.TOL, (i, h, eo, ed)
    return worst


@pytest.mark.parametrize("cfg", [0, 1, 2])
def test_replay_matches_oracle(cfg):
    shape = shape_of(cfg)
    ep, S0 = gh.episode(shape)
    print(f"[replay] {shape.name}", flush=True)
    rs, out = _run_rs(shape, ep, S0)
    print(f"[replay] {shape.name}: worst max-abs err {_check_all(shape, ep, S0, out):.3e}")
    rs.close()


@pytest.mark.parametrize("W,T,H,d", [(65, 12, 2, 64), (8, 40, 1, 32)])
def test_replay_deep_histories_ragged_beams(W, T, H, d):
    """Long ancestor chains (walked through the stored parents of every step)
    and beam counts that are not a multiple of anything; library ids out of
    order."""
    shape = shape_of(0, name=f"replay_t{T}", H=H, dk=d, dv=d, W=W, T=T, R=2)
    ep, S0 = gh.episode(shape)
    print(f"[replay] deep W={W} T={T} H={H} d={d}", flush=True)
    rs, out = _run_rs(shape, ep, S0, reqs=[3, 1])
    _check_all(shape, ep, S0, out)
    rs.close()


def test_replay_agrees_with_onela_at_bench_size():
    shape = shape_of(3)
    ep, S0 = gh.episode(shape)
    print(f"[replay] {shape.name} vs the OneLA path", flush=True)
    rs, out = _run_rs(shape, ep, S0)
    rs.close()
    ol = gh.run_episode(shape, ep, S0)
    ol["layer"].close()
    for t in range(shape.T):
        assert np.abs(out["o"][t] - ol["o"][t]).max() <= gh.TOL
        assert np.abs(out["delta"][t] - ol["delta"][t]).max() <= gh.TOL
    ref = gh.oracle_pair(shape, ep, S0, 30, 9)
    eo, ed = gh.max_err(out, ref, 30, 9, shape.W)
    assert eo <= gh.TOL and ed <= gh.TOL


def test_replay_bad_parent_capacity_and_memory():
    shape = shape_of(0, H=2)
    ep, S0 = gh.episode(shape)
    W, T, d = shape.W, shape.T, 32
    rs = ReplayState(1, shape.H, d, d, W, T)
    assert rs.memory() == shape.H * (4 * d * d + T * W * (4 + 4 * d + 2 * d)) + 4 * T * W
    rs.init_request(0, gh.to_dev(S0[0]))
    o = torch.empty((W, shape.H, d), dtype=torch.float32, device=gh.dev())
    ins = lambda t: [gh.to_dev(ep[key][t]) for key in ("q", "k", "v", "alpha", "beta")]
    with pytest.raises(OnelaError) as e:              # parents are required after the first step
        rs.step([0], *ins(0), None, o)
        rs.step([0], *ins(1), None, o)
    assert e.value.status == -1
    par = ep["parents"][1].astype(np.int32).copy()
    par[0, 2] = W + 3
    rs.step([0], *ins(1), gh.to_dev(par), o)
    with pytest.raises(OnelaError) as e:
        rs.sync()
    assert e.value.status == -4
    rs.reset(0)
    for t in range(T):
        rs.step([0], *ins(t), gh.to_dev(ep["parents"][t].astype(np.int32)) if t else None, o)
    rs.sync()
    with pytest.raises(OnelaError) as e:              # no record slot left
        rs.step([0], *ins(0), gh.to_dev(ep["parents"][1].astype(np.int32)), o)
    assert e.value.status == -3
    rs.close()
