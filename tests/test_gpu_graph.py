"""One decode step of two GDN layers captured once in a HIP graph and replayed.

In graph mode the step counters live on the device, so replaying the same
captured launches advances every request one step per replay. Each replay is
checked against the eager result on the same inputs (bit for bit), with the
program's own eager work and synchronisations between the replays; a replay
past max_steps is reported and writes nothing; a reset outside the graph
starts the next episode.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_harness as gh
    from linear_attention_beam_gdn_amd import Onela, OnelaError
    from workload import make_raw_episode, shape_of

LAYERS = [(4, 128), (2, 64)]   # (heads, head dim); layer 0 owns the ancestry index
KEYS = ("q", "k", "v", "alpha", "beta")


def test_graph_replay_of_a_two_layer_decode_step():
    eps = []
    for H, d in LAYERS:
        shape = shape_of(1, name="graph", R=2, H=H, dk=d, dv=d, T=4)
        eps.append((shape,) + tuple(gh.episode(shape)))
    shape0 = eps[0][0]
    n, W, T = len(eps[0][1]["reqs"]), shape0.W, shape0.T
    print("[graph] two layers, one captured decode step, replayed", flush=True)
    refs = [gh.run_episode(shape, ep, S0) for shape, ep, S0 in eps]   # eager, independent contexts

    s = torch.cuda.Stream()
    owner = Onela(n, shape0.H, shape0.dk, shape0.dv, W, T, stream=s)
    sharer = Onela(n, eps[1][0].H, eps[1][0].dk, eps[1][0].dv, W, T, stream=s, share_index_of=owner)
    layers = [owner, sharer]
    for lay, (shape, ep, S0) in zip(layers, eps):
        lay.set_graph_mode(True)
        for i in range(n):
            lay.init_request(i, gh.to_dev(S0[i]))
    # every step's inputs resident on the device; the graph reads fixed buffers
    src = [{key: [gh.to_dev(ep[key][t]) for t in range(T)] for key in KEYS} for _, ep, _ in eps]
    par_src = [gh.to_dev(np.maximum(eps[0][1]["parents"][t], 0).astype(np.int32)) for t in range(T)]
    buf = [{key: torch.empty_like(src[li][key][0]) for key in KEYS} for li in range(len(layers))]
    par = torch.empty_like(par_src[0])
    outs = [torch.empty((n * W, shape.H, shape.dv), dtype=torch.float32, device=gh.dev()) for shape, _, _ in eps]

    def fill(t):
        with torch.cuda.stream(s):
            for li in range(len(layers)):
                for key in KEYS:
                    buf[li][key].copy_(src[li][key][t])
            par.copy_(par_src[t])

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for li, lay in enumerate(layers):
            lay.step(list(range(n)), *[buf[li][key] for key in KEYS], par, outs[li])

    def replay():
        with torch.cuda.stream(s):                # after the fills and resets on s
            g.replay()
        s.synchronize()

    for t in range(T):
        fill(t)
        replay()
        for li in range(len(layers)):
            assert np.array_equal(outs[li].cpu().numpy(), refs[li]["o"][t]), (li, t)
        torch.cuda.synchronize()
        _ = (torch.ones(1024, device=gh.dev()) * 2).sum().item()      # unrelated eager work between replays
    for lay in layers:
        lay.sync()
        assert lay.get_step(0) == T
    assert np.array_equal(owner.get_ancestry(1), refs[0]["anc"][-1][1])

    replay()                                     # a fifth step: no record slot left
    with pytest.raises(OnelaError) as e:
        owner.sync()
    assert e.value.status == -3
    for lay in layers:                           # the next episode, started outside the graph
        for i in range(n):
            lay.reset(i)
    fill(0)
    replay()
    for li, lay in enumerate(layers):
        lay.sync()
        assert lay.get_step(1) == 1
        assert np.array_equal(outs[li].cpu().numpy(), refs[li]["o"][0])
    del g
    for r in refs:
        r["layer"].close()
    sharer.close()
    owner.close()


def test_graph_mode_switch_keeps_counters():
    """Eager steps, then graph-mode steps (not captured), then eager again:
    the episode continues across the switches."""
    shape = shape_of(1, name="graph_switch", R=1, H=2, T=4)
    ep, S0 = gh.episode(shape)
    ref = gh.run_episode(shape, ep, S0)
    lay = Onela(1, shape.H, 128, 128, shape.W, shape.T)
    lay.init_request(0, gh.to_dev(S0[0]))
    o = torch.empty((shape.W, shape.H, 128), dtype=torch.float32, device=gh.dev())
    for t in range(shape.T):
        lay.set_graph_mode(t in (1, 2))
        par = gh.to_dev(np.maximum(ep["parents"][t], 0).astype(np.int32))
        lay.step([0], *[gh.to_dev(ep[key][t]) for key in KEYS], par, o)
        lay.sync()
        assert lay.get_step(0) == t + 1
        assert np.array_equal(o.cpu().numpy(), ref["o"][t])
    with pytest.raises(OnelaError) as e:         # eager again: the host knows max_steps is reached
        lay.step([0], *[gh.to_dev(ep[key][0]) for key in KEYS], par, o)
    assert e.value.status == -3
    lay.close()
    ref["layer"].close()


def test_graph_replay_of_the_fused_step():
    """onela_step_raw captured once in graph mode and replayed per step equals
    the eager calls bit for bit."""
    shape = shape_of(1, name="graph_fused", R=2, H=3, T=3)
    ep = make_raw_episode(shape)
    n, W, T = 2, shape.W, shape.T
    keys = ("q_raw", "k_raw", "v", "a_raw", "b_raw")
    A, D = gh.to_dev(ep["A_log"]), gh.to_dev(ep["dt_bias"])
    src = {key: [gh.to_dev(ep[key][t]) for t in range(T)] for key in keys}
    par_src = [gh.to_dev(np.maximum(ep["parents"][t], 0).astype(np.int32)) for t in range(T)]

    eager = Onela(n, shape.H, 128, 128, W, T)
    for i in range(n):
        eager.init_request(i, gh.to_dev(ep["S0"][i]))
    o16 = torch.empty((n * W, shape.H, 128), dtype=torch.int16, device=gh.dev())
    want = []
    for t in range(T):
        eager.step_raw([0, 1], *[src[key][t] for key in keys], A, D, par_src[t], o16)
        eager.sync()
        want.append(o16.cpu().numpy().copy())
    eager.close()

    s = torch.cuda.Stream()
    lay = Onela(n, shape.H, 128, 128, W, T, stream=s)
    lay.set_graph_mode(True)
    for i in range(n):
        lay.init_request(i, gh.to_dev(ep["S0"][i]))
    buf = {key: torch.empty_like(src[key][0]) for key in keys}
    par = torch.empty_like(par_src[0])
    out = torch.empty_like(o16)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        lay.step_raw([0, 1], *[buf[key] for key in keys], A, D, par, out)
    for t in range(T):
        with torch.cuda.stream(s):
            for key in keys:
                buf[key].copy_(src[key][t])
            par.copy_(par_src[t])
            g.replay()                            # on s, after the copies
        s.synchronize()
        assert np.array_equal(out.cpu().numpy(), want[t]), t
    lay.sync()
    assert lay.get_step(1) == T
    del g
    lay.close()
