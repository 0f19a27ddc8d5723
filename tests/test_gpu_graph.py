"""One decode step of two GDN layers captured once in a HIP graph and replayed.

In graph mode the step counters live on the device, so replaying the same
captured launches advances every request one step per replay. Each replay is
checked against the float64 oracle (o and delta within 1e-3 for every layer,
request and head; the ancestry rows against a brute-force parent walk) and
against the eager result on the same inputs (bit for bit), with the
program's own eager work and synchronisations between the replays; outputs
are poisoned with NaN before every replay; a replay past max_steps is
reported and writes nothing; a reset outside the graph starts the next
episode. One case runs at the 32-request, 16-head, W = 256 size with
sampled pairs.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_harness as gh
    from linear_attention_beam_gdn_amd import Onela, OnelaError
    from oracle import ancestry_walk, full_state_episode, fused_inputs
    from workload import bf16_bits_to_f32, make_raw_episode, shape_of

LAYERS = [(4, 128), (2, 64)]   # (heads, head dim); layer 0 owns the ancestry index
KEYS = ("q", "k", "v", "alpha", "beta")


@pytest.mark.parametrize("W,order", [(256, -1), (600, 1)])
def test_graph_replay_of_a_two_layer_decode_step(W, order):
    # (600 beams in ancestry order: the captured launches sort them by the radix sort)
    eps = []
    for H, d in LAYERS:
        shape = shape_of(1, name="graph", R=2, H=H, dk=d, dv=d, T=4, W=W)
        eps.append((shape,) + tuple(gh.episode(shape)))
    shape0 = eps[0][0]
    n, W, T = len(eps[0][1]["reqs"]), shape0.W, shape0.T
    print(f"[graph] two layers, one captured decode step, replayed; W={W} beam_order={order}", flush=True)
    refs = [gh.run_episode(shape, ep, S0) for shape, ep, S0 in eps]   # eager, independent contexts

    s = torch.cuda.Stream()
    owner = Onela(n, shape0.H, shape0.dk, shape0.dv, W, T, stream=s)
    sharer = Onela(n, eps[1][0].H, eps[1][0].dk, eps[1][0].dv, W, T, stream=s, share_index_of=owner)
    layers = [owner, sharer]
    owner.set_beam_order(order)
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
    dels = [torch.empty_like(o) for o in outs]
    orc = [gh.oracle_refs(shape, ep, S0, [(i, h) for i in range(n) for h in range(shape.H)])
           for shape, ep, S0 in eps]

    def fill(t):
        with torch.cuda.stream(s):
            for li in range(len(layers)):
                for key in KEYS:
                    buf[li][key].copy_(src[li][key][t])
                outs[li].fill_(float("nan"))
                dels[li].fill_(float("nan"))
            par.copy_(par_src[t])

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for li, lay in enumerate(layers):
            lay.step(list(range(n)), *[buf[li][key] for key in KEYS], par, outs[li], dels[li])

    def replay():
        with torch.cuda.stream(s):                # after the fills and resets on s
            g.replay()
        s.synchronize()

    for t in range(T):
        fill(t)
        replay()
        for li in range(len(layers)):
            o_np = outs[li].cpu().numpy()
            gh.check_step(eps[li][0], orc[li], t, o_np, dels[li].cpu().numpy())
            assert np.array_equal(o_np, refs[li]["o"][t]), (li, t)
        torch.cuda.synchronize()
        _ = (torch.ones(1024, device=gh.dev()) * 2).sum().item()      # unrelated eager work between replays
    for lay in layers:
        lay.sync()
        assert lay.get_step(0) == T
    assert np.array_equal(owner.get_ancestry(1), refs[0]["anc"][-1][1])
    for lay in layers:                           # the sharer reads the owner's rows
        for i in range(n):
            np.testing.assert_array_equal(lay.get_ancestry(i)[:, :T - 1], ancestry_walk(eps[0][1]["parents"][:, i, :], T, W))

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
        gh.check_step(eps[li][0], orc[li], 0, outs[li].cpu().numpy(), dels[li].cpu().numpy())
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
    d = torch.empty_like(o)
    orc = gh.oracle_refs(shape, ep, S0, [(0, h) for h in range(shape.H)])
    for t in range(shape.T):
        lay.set_graph_mode(t in (1, 2))
        par = gh.to_dev(np.maximum(ep["parents"][t], 0).astype(np.int32))
        o.fill_(float("nan"))
        d.fill_(float("nan"))
        lay.step([0], *[gh.to_dev(ep[key][t]) for key in KEYS], par, o, d)
        lay.sync()
        assert lay.get_step(0) == t + 1
        gh.check_step(shape, orc, t, o.cpu().numpy(), d.cpu().numpy())
        assert np.array_equal(o.cpu().numpy(), ref["o"][t])
    with pytest.raises(OnelaError) as e:         # eager again: the host knows max_steps is reached
        lay.step([0], *[gh.to_dev(ep[key][0]) for key in KEYS], par, o)
    assert e.value.status == -3
    lay.close()
    ref["layer"].close()


def _fused_oracle(shape, ep, i, h, eps=1e-6):
    """Oracle episode of (request i, head h) from the raw projections."""
    sl, hs = slice(i * shape.W, (i + 1) * shape.W), slice(h, h + 1)
    q, k, a, b = fused_inputs(bf16_bits_to_f32(ep["q_raw"][:, sl, hs]), bf16_bits_to_f32(ep["k_raw"][:, sl, hs]),
                              ep["a_raw"][:, sl, hs], ep["b_raw"][:, sl, hs], ep["A_log"][hs], ep["dt_bias"][hs],
                              eps=eps)
    return full_state_episode(ep["S0"][i, h], q[:, :, 0], k[:, :, 0], bf16_bits_to_f32(ep["v"][:, sl, h]),
                              a[:, :, 0], b[:, :, 0], ep["parents"][:, i, :])


def test_graph_replay_of_the_fused_step():
    """onela_step_raw captured once in graph mode and replayed per step equals
    the eager calls bit for bit and the oracle (from the same raw projections)
    within the fused path's bounds: o (bf16) 1e-3 + 2^-8 |o|, delta 1e-3."""
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
    dl = torch.empty((n * W, shape.H, 128), dtype=torch.float32, device=gh.dev())
    orc = {(i, h): _fused_oracle(shape, ep, i, h) for i in range(n) for h in range(shape.H)}
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        lay.step_raw([0, 1], *[buf[key] for key in keys], A, D, par, out, dl)
    for t in range(T):
        with torch.cuda.stream(s):
            for key in keys:
                buf[key].copy_(src[key][t])
            par.copy_(par_src[t])
            out.fill_(-1)                         # bf16 NaN bits
            dl.fill_(float("nan"))
            g.replay()                            # on s, after the copies
        s.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got, want[t]), t
        o_f = bf16_bits_to_f32(got.view(np.uint16))
        d_np = dl.cpu().numpy()
        for (i, h), ref in orc.items():
            o_ih, ro = o_f[i * W:(i + 1) * W, h], ref["o"][t]
            assert np.all(np.abs(o_ih - ro) <= 1e-3 + 2.0 ** -8 * np.abs(ro)), (i, h, t)
            gh.parity_log.record("o_bf16_rel", float(np.max(np.abs(o_ih - ro) / (1e-3 + 2.0 ** -8 * np.abs(ro)))), 1.0)
            ed = gh.nan_max_abs(d_np[i * W:(i + 1) * W, h], ref["delta"][t])
            gh.parity_log.record("delta", ed, gh.TOL)
            assert ed <= gh.TOL, (i, h, t, ed)
    lay.sync()
    assert lay.get_step(1) == T
    del g
    lay.close()


def test_graph_replay_full_size_sampled():
    """A captured decode step of two layers at the 32-request, 16-head,
    d = 128, W = 256, T = 5 size (the sharing layer: 8 heads of d = 64),
    replayed five times; every replay's o and delta of sampled (request, head)
    pairs of both layers against the oracle, and the ancestry of sampled
    requests against a brute-force parent walk. Graph mode launches the
    two-body form of the step kernel (the step index is on the device)."""
    shapes = [shape_of(3), shape_of(3, name="graph_full_sharer", H=8, dk=64, dv=64)]
    eps = [(sh,) + tuple(gh.episode(sh)) for sh in shapes]
    n, W, T = shapes[0].R, shapes[0].W, shapes[0].T
    assert np.array_equal(eps[0][1]["parents"], eps[1][1]["parents"])
    print("[graph] full size: 32 requests x (16 + 8) heads, W=256, T=5", flush=True)
    rng = np.random.default_rng(5)
    pairs = [[(0, 0), (n - 1, sh.H - 1)] + [(int(rng.integers(n)), int(rng.integers(sh.H))) for _ in range(2)]
             for sh in shapes]
    orc = [gh.oracle_refs(sh, ep, S0, pr) for (sh, ep, S0), pr in zip(eps, pairs)]

    s = torch.cuda.Stream()
    owner = Onela(n, shapes[0].H, 128, 128, W, T, stream=s)
    sharer = Onela(n, shapes[1].H, 64, 64, W, T, stream=s, share_index_of=owner)
    layers = [owner, sharer]
    for lay, (sh, ep, S0) in zip(layers, eps):
        lay.set_graph_mode(True)
        for i in range(n):
            lay.init_request(i, gh.to_dev(S0[i]))
    src = [{key: [gh.to_dev(ep[key][t]) for t in range(T)] for key in KEYS} for _, ep, _ in eps]
    par_src = [gh.to_dev(np.maximum(eps[0][1]["parents"][t], 0).astype(np.int32)) for t in range(T)]
    buf = [{key: torch.empty_like(src[li][key][0]) for key in KEYS} for li in range(2)]
    par = torch.empty_like(par_src[0])
    outs = [torch.empty((n * W, sh.H, sh.dv), dtype=torch.float32, device=gh.dev()) for sh in shapes]
    dels = [torch.empty_like(o) for o in outs]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for li, lay in enumerate(layers):
            lay.step(list(range(n)), *[buf[li][key] for key in KEYS], par, outs[li], dels[li])
    for t in range(T):
        with torch.cuda.stream(s):
            for li in range(2):
                for key in KEYS:
                    buf[li][key].copy_(src[li][key][t])
                outs[li].fill_(float("nan"))
                dels[li].fill_(float("nan"))
            par.copy_(par_src[t])
            g.replay()
        s.synchronize()
        for li in range(2):
            o_np = outs[li].cpu().numpy()
            assert not np.isnan(o_np).any(), (li, t)
            gh.check_step(shapes[li], orc[li], t, o_np, dels[li].cpu().numpy())
    for lay in layers:
        lay.sync()
        assert lay.get_step(n - 1) == T
    for i in (0, 17, n - 1):
        want = ancestry_walk(eps[0][1]["parents"][:, i, :], T, W)
        for lay in layers:
            np.testing.assert_array_equal(lay.get_ancestry(i)[:, :T - 1], want)
    del g
    sharer.close()
    owner.close()
