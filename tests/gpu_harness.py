"""Helpers that drive the HIP library through its C ABI for the GPU tests."""
from __future__ import annotations

import numpy as np
import torch

from linear_attention_beam_gdn_amd import Onela
from oracle import full_state_episode, prompt_state
from workload import bf16_bits_to_f32, make_episode, prompt_tokens

TOL = 1e-3   # max-abs bound on o and delta against the float64 oracle


def dev():
    return torch.device("cuda:0")


def s0_for(shape, ep, reqs):
    """S0 [n][H][dv][dk] float32 for the requests: drawn, or folded from the prompt by the oracle."""
    if shape.s0 == "normal":
        return ep["S0"]
    out = []
    for r in reqs:
        pt = prompt_tokens(shape, r)
        S = prompt_state(bf16_bits_to_f32(pt["k"]), bf16_bits_to_f32(pt["v"]), pt["alpha"], pt["beta"])
        out.append(S.astype(np.float32))
    return np.stack(out)


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.int16)
    return t.to(dev())


def run_episode(shape, ep, S0, beams_per_block=0, keep_delta=True, reqs=None):
    """Run all T steps of the episode on the GPU. Returns per-step host arrays.

    o[t], delta[t]: [n*W][H][dv] float32; anc[t]: [n][W][max_steps] int32.
    """
    n = len(ep["reqs"])
    reqs = list(range(n)) if reqs is None else reqs
    lay = Onela(max_requests=max(reqs) + 1, num_heads=shape.H, d_k=shape.dk, d_v=shape.dv,
                beam_width=shape.W, max_steps=shape.T)
    if beams_per_block:
        lay.set_beams_per_block(beams_per_block)
    for i, r in enumerate(reqs):
        lay.init_request(r, to_dev(S0[i]))
    outs = {"o": [], "delta": [], "anc": []}
    rows = n * shape.W
    o = torch.empty((rows, shape.H, shape.dv), dtype=torch.float32, device=dev())
    d = torch.empty_like(o) if keep_delta else None
    for t in range(shape.T):
        par = to_dev(ep["parents"][t].astype(np.int32)) if t > 0 else None
        lay.step(reqs, to_dev(ep["q"][t]), to_dev(ep["k"][t]), to_dev(ep["v"][t]),
                 to_dev(ep["alpha"][t]), to_dev(ep["beta"][t]), par, o, d)
        lay.sync()
        outs["o"].append(o.cpu().numpy().copy())
        if keep_delta:
            outs["delta"].append(d.cpu().numpy().copy())
        outs["anc"].append(np.stack([lay.get_ancestry(r) for r in reqs]))
    outs["layer"] = lay
    outs["reqs"] = reqs
    return outs


def oracle_pair(shape, ep, S0, i, h):
    """Oracle episode of call-local request i, head h."""
    W = shape.W
    sl = slice(i * W, (i + 1) * W)
    f = lambda key: bf16_bits_to_f32(ep[key][:, sl, h, :])
    return full_state_episode(S0[i, h], f("q"), f("k"), f("v"), ep["alpha"][:, sl, h], ep["beta"][:, sl, h],
                              ep["parents"][:, i, :])


def max_err(gpu_steps, ref, i, h, W):
    """Max |gpu - oracle| over all steps for (i, h) of o and delta."""
    eo = max(float(np.abs(gpu_steps["o"][t][i * W:(i + 1) * W, h] - ref["o"][t]).max())
             for t in range(len(gpu_steps["o"])))
    ed = max(float(np.abs(gpu_steps["delta"][t][i * W:(i + 1) * W, h] - ref["delta"][t]).max())
             for t in range(len(gpu_steps["delta"])))
    return eo, ed


def episode(shape, reqs=None):
    ep = make_episode(shape, reqs=reqs)
    return ep, s0_for(shape, ep, ep["reqs"])
