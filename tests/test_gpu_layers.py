"""Several GDN layers of the same requests sharing one ancestry index.

One context owns the index and writes it; the others read it. Every step,
layer and head is compared with the float64 oracle (o and delta within 1e-3;
each layer's ancestry rows equal to a brute-force walk of the parents), and
each layer's outputs must also equal those of an independent context on the
same inputs, bit for bit (same kernels, same index contents), including
requests that join at different decode steps; the ordering rules of a shared
index are enforced on the host.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_harness as gh
    from linear_attention_beam_gdn_amd import Onela, OnelaError
    from oracle import ancestry_walk
    from workload import shape_of

# (heads, head dim) of the three layers; the owner is layer 0
LAYERS = [(4, 128), (2, 64), (3, 128)]


def _layer_episodes(T=4, R=2):
    eps = []
    for H, d in LAYERS:
        shape = shape_of(1, name="layers", R=R, H=H, dk=d, dv=d, T=T)
        ep, S0 = gh.episode(shape)
        eps.append((shape, ep, S0))
    # one beam tree per request, whatever the layer
    for _, ep, _ in eps[1:]:
        assert np.array_equal(ep["parents"], eps[0][1]["parents"])
    return eps


def _make_layers(eps, max_requests):
    shape0 = eps[0][0]
    owner = Onela(max_requests, shape0.H, shape0.dk, shape0.dv, shape0.W, shape0.T)
    layers = [owner] + [Onela(max_requests, s.H, s.dk, s.dv, s.W, s.T, share_index_of=owner) for s, _, _ in eps[1:]]
    return layers


def _close(layers):
    for lay in reversed(layers):      # sharing contexts before their owner
        lay.close()


@pytest.mark.parametrize("beam_order", [-1, 1, "alternating"])
def test_shared_index_layers_equal_independent_layers(beam_order):
    # beam_order 1: the owner processes the beams in ancestry order, so every
    # step's records sit at permuted positions that the sharing layers must
    # take from the owner's order; "alternating": ancestry order at odd steps
    # only, so orders and identity positions mix within one history
    eps = _layer_episodes()
    print(f"[layers] 3 layers sharing one index vs independent, beam order {beam_order}", flush=True)
    n = len(eps[0][1]["reqs"])
    layers = _make_layers(eps, n)
    orders = [t % 2 for t in range(eps[0][0].T)] if beam_order == "alternating" else [beam_order] * eps[0][0].T
    for lay, (shape, ep, S0) in zip(layers, eps):
        for i in range(n):
            lay.init_request(i, gh.to_dev(S0[i]))
    outs = [[] for _ in layers]
    deltas = [[] for _ in layers]
    for t in range(eps[0][0].T):
        layers[0].set_beam_order(orders[t])
        for li, (lay, (shape, ep, S0)) in enumerate(zip(layers, eps)):
            par = gh.to_dev(ep["parents"][t].astype(np.int32)) if t else None
            o = torch.full((n * shape.W, shape.H, shape.dv), float("nan"), dtype=torch.float32, device=gh.dev())
            d = torch.full_like(o, float("nan"))
            lay.step(list(range(n)), *[gh.to_dev(ep[key][t]) for key in ("q", "k", "v", "alpha", "beta")], par, o, d)
            outs[li].append(o)
            deltas[li].append(d)
    for li, (lay, (shape, ep, S0)) in enumerate(zip(layers, eps)):
        lay.sync()
        W, T = shape.W, shape.T
        o_np = [o.cpu().numpy() for o in outs[li]]
        d_np = [d.cpu().numpy() for d in deltas[li]]
        for i in range(n):             # every step, head and request against the oracle
            gh.check_request_steps(shape, ep, S0, i, [o[i * W:(i + 1) * W] for o in o_np],
                                   [d[i * W:(i + 1) * W] for d in d_np])
            np.testing.assert_array_equal(lay.get_ancestry(i)[:, :T - 1],
                                          ancestry_walk(ep["parents"][:, i, :], T, W))
        ref = gh.run_episode(shape, ep, S0)
        for t in range(shape.T):
            assert np.array_equal(o_np[t], ref["o"][t]), (li, t)
        for i in range(n):
            assert np.array_equal(lay.get_ancestry(i), ref["anc"][-1][i])
            for h in range(shape.H):    # records by beam, whatever order they were stored in
                got, want = lay.get_records(i, h, T * W), ref["layer"].get_records(i, h, T * W)
                for g, w in zip(got, want):
                    assert np.array_equal(g, w), (li, i, h)
        ref["layer"].close()
    mem = [lay.memory() for lay in layers]
    assert mem[1]["index_bytes"] == 20 * n and mem[2]["index_bytes"] == 20 * n   # per-request words only
    _close(layers)


def test_shared_index_requests_joining_at_different_steps():
    eps = _layer_episodes(T=4, R=2)
    shape0 = eps[0][0]
    W, T = shape0.W, shape0.T
    print("[layers] staggered requests", flush=True)
    layers = _make_layers(eps, 3)
    slots = [2, 0]                  # library ids of workload requests 0 and 1
    start = [0, 2]                  # request i joins at decode call start[i]
    for lay, (shape, ep, S0) in zip(layers, eps):
        for i, s in enumerate(slots):
            lay.init_request(s, gh.to_dev(S0[i]))
    hist = [{i: [] for i in range(2)} for _ in layers]
    for call in range(T + 2):
        active = [i for i in range(2) if start[i] <= call < start[i] + T]
        steps = [call - start[i] for i in active]
        for li, (lay, (shape, ep, S0)) in enumerate(zip(layers, eps)):
            cat = lambda key: np.concatenate([ep[key][steps[j]][i * W:(i + 1) * W] for j, i in enumerate(active)])
            par = gh.to_dev(np.stack([np.maximum(ep["parents"][steps[j]][i], 0)
                                      for j, i in enumerate(active)]).astype(np.int32))
            o = torch.empty((len(active) * W, shape.H, shape.dv), dtype=torch.float32, device=gh.dev())
            lay.step([slots[i] for i in active], *[gh.to_dev(cat(key)) for key in ("q", "k", "v", "alpha", "beta")],
                     par, o)
            lay.sync()
            on = o.cpu().numpy()
            for j, i in enumerate(active):
                hist[li][i].append(on[j * W:(j + 1) * W])
    for li, (shape, ep, S0) in enumerate(eps):
        for i in range(2):             # every step and head of both requests against the oracle
            gh.check_request_steps(shape, ep, S0, i, hist[li][i])
            np.testing.assert_array_equal(layers[li].get_ancestry(slots[i])[:, :T - 1],
                                          ancestry_walk(ep["parents"][:, i, :], T, W))
        ref = gh.run_episode(shape, ep, S0)
        for i in range(2):
            for t in range(T):
                assert np.array_equal(hist[li][i][t], ref["o"][t][i * W:(i + 1) * W]), (li, i, t)
        ref["layer"].close()
    _close(layers)


def test_shared_index_ordering_rules():
    eps = _layer_episodes(T=4, R=1)
    (s0, ep0, S00), (s1, ep1, S01) = eps[0], eps[1]
    owner = Onela(1, s0.H, s0.dk, s0.dv, s0.W, s0.T)
    sharer = Onela(1, s1.H, s1.dk, s1.dv, s1.W, s1.T, share_index_of=owner)
    with pytest.raises(OnelaError) as e:                 # beam width differs from the owner's
        Onela(1, s1.H, s1.dk, s1.dv, s1.W // 2, s1.T, share_index_of=owner)
    assert e.value.status == -1
    with pytest.raises(OnelaError) as e:                 # no chains: a sharer cannot own
        Onela(1, s1.H, s1.dk, s1.dv, s1.W, s1.T, share_index_of=sharer)
    assert e.value.status == -1
    owner.init_request(0, gh.to_dev(S00[0]))
    sharer.init_request(0, gh.to_dev(S01[0]))
    o0 = torch.empty((s0.W, s0.H, s0.dv), device=gh.dev())
    o1 = torch.empty((s1.W, s1.H, s1.dv), device=gh.dev())

    def step(lay, ep, o, t):
        par = gh.to_dev(ep["parents"][t].astype(np.int32)) if t else None
        lay.step([0], *[gh.to_dev(ep[key][t]) for key in ("q", "k", "v", "alpha", "beta")], par, o)

    step(sharer, ep1, o1, 0)            # step 1 reads no index: any order
    with pytest.raises(OnelaError) as e:
        step(sharer, ep1, o1, 1)        # step 2 before the owner's steps 1 and 2
    assert e.value.status == -2
    step(owner, ep0, o0, 0)
    with pytest.raises(OnelaError) as e:
        step(sharer, ep1, o1, 1)        # the owner's step 2 decides where the records of step 2 go
    assert e.value.status == -2
    step(owner, ep0, o0, 1)             # owner at 2, sharer at 1: fine
    with pytest.raises(OnelaError) as e:
        step(owner, ep0, o0, 2)         # owner's step 3 would overwrite what the sharer's step 2 reads
    assert e.value.status == -2
    step(sharer, ep1, o1, 1)
    step(owner, ep0, o0, 2)
    owner.reset(0)                      # restart on the owner: the sharer must restart too
    with pytest.raises(OnelaError) as e:
        step(sharer, ep1, o1, 2)
    assert e.value.status == -2
    sharer.reset(0)
    step(owner, ep0, o0, 0)
    step(sharer, ep1, o1, 0)
    owner.sync()
    sharer.sync()
    with pytest.raises(OnelaError) as e:
        owner.close()                   # the sharer still reads its index
    assert e.value.status == -2
    sharer.close()
    owner.close()
