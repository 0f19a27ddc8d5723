"""Parity of the HIP decode step with the float64 oracle (through the C ABI).

Tolerance: max-abs 1e-3 on o and delta at every step (fp32 state and
accumulation, bf16 inputs); record alpha and key bits, record ids and the
ancestry index must match exactly.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_harness as gh
    from workload import shape_of


def _check_pairs(shape, ep, S0, outs, pairs, tol=None):
    tol = gh.TOL if tol is None else tol
    W, T = shape.W, shape.T
    worst = (0.0, 0.0)
    for (i, h) in pairs:
        ref = gh.oracle_pair(shape, ep, S0, i, h)
        eo, ed = gh.max_err(outs, ref, i, h, W)
        worst = (max(worst[0], eo), max(worst[1], ed))
        assert eo <= tol and ed <= tol, f"pair {(i, h)}: max err o={eo:.3g} delta={ed:.3g}"
        for t in range(T):
            anc = outs["anc"][t][i]
            np.testing.assert_array_equal(anc[:, :t], ref["anc"][t])
            assert np.all(anc[:, t:] == -1)
        a, d, kbits = outs["layer"].get_records(outs["reqs"][i], h, T * W)
        sl = slice(i * W, (i + 1) * W)
        np.testing.assert_array_equal(a.reshape(T, W), ep["alpha"][:, sl, h])
        np.testing.assert_array_equal(kbits.reshape(T, W, -1), ep["k"][:, sl, h, :])
        assert np.abs(d - ref["rec_delta"]).max() <= tol
        # a prefix that ends inside a step: the same records, by beam
        n_part = (T - 1) * W + W // 2 + 1
        for got, full in zip(outs["layer"].get_records(outs["reqs"][i], h, n_part), (a, d, kbits)):
            np.testing.assert_array_equal(got, full[:n_part])
    print(f"{shape.name}: worst max-abs err o={worst[0]:.3e} delta={worst[1]:.3e} over {len(pairs)} pairs")
    return worst


@pytest.mark.parametrize("cfg,order", [(0, -1), (1, -1), (2, -1), (1, 1), (2, 1)])
def test_parity_small_configs(cfg, order):
    """Automatic beam order (index order at these sizes) and ancestry order forced."""
    shape = shape_of(cfg)
    ep, S0 = gh.episode(shape)
    print(f"[parity] cfg={cfg} {shape.name} beam_order={order}", flush=True)
    outs = gh.run_episode(shape, ep, S0, beam_order=order)
    pairs = [(i, h) for i in range(shape.R) for h in range(shape.H)]
    _check_pairs(shape, ep, S0, outs, pairs)
    outs["layer"].close()


def test_parity_r32_full_size_sampled():
    """All 32 requests x 16 heads at W=256, T=5 in the bench's launch shape; sampled pairs vs the oracle."""
    shape = shape_of(3)
    ep, S0 = gh.episode(shape)
    print(f"[parity] {shape.name}", flush=True)
    outs = gh.run_episode(shape, ep, S0, keep_delta=True)
    rng = np.random.default_rng(3)
    pairs = [(0, 0), (31, 15)] + [(int(rng.integers(32)), int(rng.integers(16))) for _ in range(4)]
    _check_pairs(shape, ep, S0, outs, pairs)
    for t in range(shape.T):
        assert np.isfinite(outs["o"][t]).all() and np.isfinite(outs["delta"][t]).all()
    outs["layer"].close()


@pytest.mark.parametrize("W,T,H,d", [(1, 3, 2, 32), (65, 4, 3, 64), (130, 5, 2, 128), (200, 2, 1, 128),
                                     (1100, 3, 1, 32)])
def test_parity_ragged_beams(W, T, H, d):
    """Beam counts that leave partial chunks (and W = 1, a plain GDN chain; W = 1100 is wider
    than the beam sets the kernels process in ancestry order, so its records keep beam order)."""
    shape = shape_of(0, name=f"ragged_w{W}", H=H, dk=d, dv=d, W=W, T=T, R=2)
    ep, S0 = gh.episode(shape)
    print(f"[parity] ragged W={W} T={T} H={H} d={d}", flush=True)
    outs = gh.run_episode(shape, ep, S0)
    pairs = [(i, h) for i in range(2) for h in range(H)]
    _check_pairs(shape, ep, S0, outs, pairs)
    outs["layer"].close()


@pytest.mark.parametrize("W,T,H,d,order", [(40, 12, 2, 64, -1), (16, 20, 1, 128, -1), (8, 64, 1, 32, -1),
                                           (40, 12, 2, 64, 1), (8, 64, 1, 32, 1)])
def test_parity_deep_histories(W, T, H, d, order):
    """Histories longer than the short decode horizons of the pages' workload,
    up to the 64-step maximum: many older blocks of delta gathers per beam,
    long ancestry rows, and (at 64 steps) the largest LDS footprint; in the
    automatic beam order and in ancestry order."""
    shape = shape_of(0, name=f"deep_t{T}", H=H, dk=d, dv=d, W=W, T=T, R=2)
    ep, S0 = gh.episode(shape)
    print(f"[parity] deep history W={W} T={T} H={H} d={d} beam_order={order}", flush=True)
    outs = gh.run_episode(shape, ep, S0, beam_order=order)
    _check_pairs(shape, ep, S0, outs, [(i, h) for i in range(2) for h in range(H)])
    outs["layer"].close()


@pytest.mark.parametrize("W,bpb", [(1100, 0), (1300, 256)])
def test_parity_wide_beam_sets(W, bpb):
    """Beam sets wider than the ancestry-ordered limit (1024) are processed in
    index order; ragged last chunk, several workgroups per (request, head)."""
    shape = shape_of(0, name=f"wide_w{W}", H=2, dk=32, dv=32, W=W, T=3, R=2)
    ep, S0 = gh.episode(shape)
    print(f"[parity] wide beam set W={W} beams_per_block={bpb}", flush=True)
    outs = gh.run_episode(shape, ep, S0, beams_per_block=bpb)
    _check_pairs(shape, ep, S0, outs, [(i, h) for i in range(2) for h in range(2)])
    outs["layer"].close()


def test_parity_extreme_gates():
    """Gates at their ends mixed with ordinary draws: alpha = 0 forgets the
    whole history, S0 included; alpha = 1 keeps it undecayed; beta = 0 writes
    nothing, so delta is exactly zero; beta = 1 writes v back at the key."""
    shape = shape_of(0, name="extreme_gates", R=2, H=3, dk=64, dv=64, W=40, T=6)
    ep, S0 = gh.episode(shape)
    rng = np.random.default_rng(11)
    for key in ("alpha", "beta"):
        pick = rng.integers(0, 3, size=ep[key].shape)
        ep[key] = np.where(pick == 0, 0.0, np.where(pick == 1, 1.0, ep[key])).astype(np.float32)
    print(f"[parity] {shape.name}", flush=True)
    outs = gh.run_episode(shape, ep, S0)
    _check_pairs(shape, ep, S0, outs, [(i, h) for i in range(2) for h in range(3)])
    for t in range(shape.T):
        assert np.all(outs["delta"][t][ep["beta"][t] == 0] == 0)
    outs["layer"].close()


def test_tile_size_invariance_and_determinism():
    """Outputs are bit-identical across launch shapes and across runs."""
    shape = shape_of(1, R=2, T=4)
    ep, S0 = gh.episode(shape)
    runs = [gh.run_episode(shape, ep, S0, beams_per_block=bpb) for bpb in (0, 64, 128, 256, 0)]
    for other in runs[1:]:
        for t in range(shape.T):
            assert np.array_equal(runs[0]["o"][t], other["o"][t])
            assert np.array_equal(runs[0]["delta"][t], other["delta"][t])
    for r in runs:
        r["layer"].close()


def test_beam_order_invariance():
    """The processing order only decides which beams share a chunk: index
    order, ancestry order, and the two alternating from step to step (each
    step then reads the order the previous one wrote, a permutation either
    way) give bit-identical outputs, ancestry and records, equal to the
    oracle's within the tolerance."""
    shape = shape_of(1, R=2, T=5)
    ep, S0 = gh.episode(shape)
    modes = [0, 1, [1, 0, 1, 0, 1], [0, 1, 0, 1, 0], [1, 1, 0, 0, 1]]
    runs = []
    for m in modes:
        print(f"[parity] beam order {m}", flush=True)
        runs.append(gh.run_episode(shape, ep, S0, beam_order=m))
    for other in runs[1:]:
        for t in range(shape.T):
            assert np.array_equal(runs[0]["o"][t], other["o"][t])
            assert np.array_equal(runs[0]["delta"][t], other["delta"][t])
            assert np.array_equal(runs[0]["anc"][t], other["anc"][t])
    _check_pairs(shape, ep, S0, runs[2], [(i, h) for i in range(2) for h in range(0, shape.H, 5)])
    for r in runs:
        r["layer"].close()


def test_requests_at_different_depths():
    """Requests that join later run at their own step index in the same launch."""
    shape = shape_of(1, name="mixed_depth", R=3, H=4, T=4)
    ep, S0 = gh.episode(shape)
    W, H = shape.W, shape.H
    lay = gh.Onela(max_requests=5, num_heads=H, d_k=128, d_v=128, beam_width=W, max_steps=shape.T)
    slots = [4, 0, 2]                                  # library ids of workload requests 0, 1, 2
    for i, s in enumerate(slots):
        lay.init_request(s, gh.to_dev(S0[i]))
    start = [0, 1, 2]                                  # request i joins at call number start[i]
    o_hist = {i: [] for i in range(3)}
    for call in range(shape.T + 2):
        active = [i for i in range(3) if start[i] <= call < start[i] + shape.T]
        if not active:
            continue
        steps = [call - start[i] for i in active]
        cat = lambda key, t_of: np.concatenate(
            [ep[key][t_of[j]][i * W:(i + 1) * W] for j, i in enumerate(active)], axis=0)
        q, k, v = (gh.to_dev(cat(key, steps)) for key in ("q", "k", "v"))
        a, b = gh.to_dev(cat("alpha", steps)), gh.to_dev(cat("beta", steps))
        par = gh.to_dev(np.stack([np.maximum(ep["parents"][steps[j]][i], 0) for j, i in enumerate(active)]).astype(np.int32))
        o = torch.empty((len(active) * W, H, 128), dtype=torch.float32, device=gh.dev())
        lay.step([slots[i] for i in active], q, k, v, a, b, par, o)
        lay.sync()
        on = o.cpu().numpy()
        for j, i in enumerate(active):
            o_hist[i].append(on[j * W:(j + 1) * W])
    for i in range(3):
        for h in range(H):
            ref = gh.oracle_pair(shape, ep, S0, i, h)
            for t in range(shape.T):
                assert np.abs(o_hist[i][t][:, h] - ref["o"][t]).max() <= gh.TOL
    lay.close()
    # requests 1 and 2 took their first step in a launch with a later-step request (the
    # general kernel); all three starting together take it without record gathers: same bits
    together = gh.run_episode(shape_of(1, name="mixed_depth", R=3, H=4, T=1), ep, S0)
    for i in (1, 2):
        assert np.array_equal(o_hist[i][0], together["o"][0][i * W:(i + 1) * W])
    together["layer"].close()


def test_more_requests_than_one_launch():
    """70 requests in one call (two launches per step, 64 + 6) under library
    ids in reverse order; every (request, head) pair against the oracle."""
    shape = shape_of(0, name="many_requests", R=70, H=2, dk=32, dv=32, W=8, T=3)
    ep, S0 = gh.episode(shape)
    reqs = [74 - i for i in range(70)]
    print(f"[parity] {shape.name}: 70 requests, library ids 74..5", flush=True)
    outs = gh.run_episode(shape, ep, S0, reqs=reqs)
    _check_pairs(shape, ep, S0, outs, [(i, h) for i in range(70) for h in range(2)])
    outs["layer"].close()


@pytest.mark.parametrize("W,d,parents,bpb", [(257, 32, "zipf", 0), (500, 64, "topw4", 0), (777, 32, "uniform", 128),
                                            (1024, 128, "zipf", 0), (1024, 32, "topw4", 256)])
def test_parity_wide_beam_sets_in_ancestry_order(W, d, parents, bpb):
    """Ancestry order forced on beam sets wider than 256, which are radix-sorted:
    ragged chunk counts, several chunks per wave, both digit widths."""
    shape = shape_of(0, name=f"wide_w{W}_d{d}", R=2, H=2, dk=d, dv=d, W=W, T=5, parents=parents)
    ep, S0 = gh.episode(shape)
    print(f"[parity] wide W={W} d={d} parents={parents} beams_per_block={bpb} beam_order=1", flush=True)
    outs = gh.run_episode(shape, ep, S0, beams_per_block=bpb, beam_order=1)
    _check_pairs(shape, ep, S0, outs, [(i, h) for i in range(2) for h in range(2)])
    outs["layer"].close()


@pytest.mark.parametrize("seed", range(24))
def test_parity_random_shapes(seed):
    """Seeded random shapes, parent patterns, gate extremes, launch shapes and
    beam orders: every (request, head) pair against the oracle. Parents are
    drawn uniformly, top-W of 4W or Zipf(1.2), or replaced by every beam
    continuing beam 0 (one shared history) or beam b continuing beam b (W
    independent chains)."""
    rng = np.random.default_rng(4242 + seed)
    d = int(rng.choice([32, 64, 128]))
    W, T = int(rng.integers(1, 300)), int(rng.integers(1, 9))
    R, H = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    pattern = str(rng.choice(["uniform", "topw4", "zipf"]))
    shape = shape_of(0, name=f"random{seed}", R=R, H=H, dk=d, dv=d, W=W, T=T, parents=pattern)
    ep, S0 = gh.episode(shape)
    special = int(rng.integers(0, 4))
    if special == 1:
        ep["parents"][1:] = 0
    elif special == 2:
        ep["parents"][1:] = np.arange(W, dtype=ep["parents"].dtype)
    elif special == 3:
        for key in ("alpha", "beta"):
            pick = rng.integers(0, 4, size=ep[key].shape)
            ep[key] = np.where(pick == 0, 0.0, np.where(pick == 1, 1.0, ep[key])).astype(np.float32)
    order, bpb = int(rng.choice([-1, 0, 1])), int(rng.choice([0, 64, 128]))
    print(f"[parity] random seed={seed} R={R} H={H} d={d} W={W} T={T} parents={pattern} special={special} "
          f"beam_order={order} beams_per_block={bpb}", flush=True)
    outs = gh.run_episode(shape, ep, S0, beams_per_block=bpb, beam_order=order)
    _check_pairs(shape, ep, S0, outs, [(i, h) for i in range(R) for h in range(H)])
    outs["layer"].close()
