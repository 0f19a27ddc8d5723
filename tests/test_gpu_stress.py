"""The stress workload at full size: 64 requests x 32 heads, d=128, W=1024, T=7, Zipf(1.2) parents.

All requests run through the C ABI in the automatic launch shape; sampled
(request, head) pairs are compared with the float64 oracle element by element
(max-abs 1e-3 on o and delta at every step), ancestry rows of sampled requests
must equal a brute-force parent walk, and every output must be finite.
"""
import numpy as np
import pytest
import torch

import parity_log

pytestmark = pytest.mark.gpu

TOL = 1e-3


def test_stress_r64_h32_w1024_t7_sampled():
    from linear_attention_beam_gdn_amd import Onela
    from oracle import ancestry_walk, full_state_episode
    from workload import bf16_bits_to_f32, shape_of
    from workload.gen_device import all_parents, s0_device, step_inputs

    shape = shape_of(4)
    R, H, W, T, d = shape.R, shape.H, shape.W, shape.T, shape.dk
    dev = torch.device("cuda:0")
    print(f"[stress] {shape.name}", flush=True)
    parents = all_parents(shape)
    S0 = s0_device(shape, dev)
    lay = Onela(R, H, d, d, W, T)
    for r in range(R):
        lay.init_request(r, S0[r].contiguous())
    pairs = [(0, 0), (R - 1, H - 1), (37, 11)]
    keep = {p: {key: [] for key in ("q", "k", "v", "alpha", "beta", "o", "delta")} for p in pairs}
    o = torch.empty((R * W, H, d), dtype=torch.float32, device=dev)
    dl = torch.empty_like(o)
    for t in range(T):
        o.fill_(float("nan"))          # a skipped write would stay NaN
        dl.fill_(float("nan"))
        inp = step_inputs(shape, t, dev)
        par = torch.from_numpy(parents[t].astype(np.int32)).to(dev) if t else None
        lay.step(list(range(R)), inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], par, o, dl)
        lay.sync()
        assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(dl).all()), f"non-finite output at step {t + 1}"
        for (r, h) in pairs:
            sl = slice(r * W, (r + 1) * W)
            for key in ("q", "k", "v"):
                keep[(r, h)][key].append(inp[key][sl, h].cpu().numpy().view(np.uint16))
            for key in ("alpha", "beta"):
                keep[(r, h)][key].append(inp[key][sl, h].cpu().numpy())
            keep[(r, h)]["o"].append(o[sl, h].cpu().numpy())
            keep[(r, h)]["delta"].append(dl[sl, h].cpu().numpy())
        del inp
    for r in sorted({p[0] for p in pairs}):
        anc = lay.get_ancestry(r)
        np.testing.assert_array_equal(anc[:, : T - 1], ancestry_walk(parents[:, r, :], T, W))
        assert np.all(anc[:, T - 1:] == -1)
    s0_host = {p: S0[p[0], p[1]].cpu().numpy() for p in pairs}
    lay.close()
    for (r, h) in pairs:
        kp = keep[(r, h)]
        f = lambda key: bf16_bits_to_f32(np.stack(kp[key]))
        ref = full_state_episode(s0_host[(r, h)], f("q"), f("k"), f("v"), np.stack(kp["alpha"]),
                                 np.stack(kp["beta"]), parents[:, r, :])
        eo = float(np.abs(np.stack(kp["o"]) - ref["o"]).max())
        ed = float(np.abs(np.stack(kp["delta"]) - ref["delta"]).max())
        print(f"[stress] pair {(r, h)}: max-abs err o={eo:.3e} delta={ed:.3e}", flush=True)
        parity_log.record("o", eo, TOL)
        parity_log.record("delta", ed, TOL)
        assert eo <= TOL and ed <= TOL
