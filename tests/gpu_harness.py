"""Helpers that drive the HIP library through its C ABI for the GPU tests."""
from __future__ import annotations

import numpy as np
import torch

from linear_attention_beam_gdn_amd import Onela
from oracle import full_state_episode, prompt_state
from workload import bf16_bits_to_f32, make_episode, prompt_tokens

import parity_log

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


def run_episode(shape, ep, S0, beams_per_block=0, keep_delta=True, reqs=None, beam_order=-1):
    """Run all T steps of the episode on the GPU. Returns per-step host arrays.

    o[t], delta[t]: [n*W][H][dv] float32; anc[t]: [n][W][max_steps] int32.
    beam_order: -1 automatic, 0 index order, 1 ancestry order, or a list with
    one of these per step.
    """
    n = len(ep["reqs"])
    reqs = list(range(n)) if reqs is None else reqs
    lay = Onela(max_requests=max(reqs) + 1, num_heads=shape.H, d_k=shape.dk, d_v=shape.dv,
                beam_width=shape.W, max_steps=shape.T)
    if beams_per_block:
        lay.set_beams_per_block(beams_per_block)
    orders = beam_order if isinstance(beam_order, (list, tuple)) else [beam_order] * shape.T
    for i, r in enumerate(reqs):
        lay.init_request(r, to_dev(S0[i]))
    outs = {"o": [], "delta": [], "anc": []}
    rows = n * shape.W
    o = torch.empty((rows, shape.H, shape.dv), dtype=torch.float32, device=dev())
    d = torch.empty_like(o) if keep_delta else None
    for t in range(shape.T):
        # outputs poisoned before every step: a write the kernel skips shows as NaN
        o.fill_(float("nan"))
        if d is not None:
            d.fill_(float("nan"))
        par = to_dev(ep["parents"][t].astype(np.int32)) if t > 0 else None
        lay.set_beam_order(orders[t])
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
    """Max |gpu - oracle| over all steps for (i, h) of o and delta (NaN counts
    as an infinite error); recorded in the session's error log."""
    eo = max(nan_max_abs(gpu_steps["o"][t][i * W:(i + 1) * W, h], ref["o"][t]) for t in range(len(gpu_steps["o"])))
    ed = max(nan_max_abs(gpu_steps["delta"][t][i * W:(i + 1) * W, h], ref["delta"][t])
             for t in range(len(gpu_steps["delta"])))
    parity_log.record("o", eo, TOL)
    parity_log.record("delta", ed, TOL)
    return eo, ed


def nan_max_abs(a, b) -> float:
    """max |a - b|, infinite if either holds a NaN."""
    e = np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))
    return float("inf") if np.isnan(e).any() else float(e.max())


def check_request_steps(shape, ep, S0, i, o_req, d_req=None, tol=TOL, heads=None):
    """Every step and head (or the listed heads) of call-local request i against the oracle.

    o_req[t] (and d_req[t]): the request's [W][H][dv] outputs of step t.
    Errors go to the session's error log; returns the worst over o and delta."""
    worst = 0.0
    for h in range(shape.H) if heads is None else heads:
        ref = oracle_pair(shape, ep, S0, i, h)
        for t in range(len(o_req)):
            eo = nan_max_abs(o_req[t][:, h], ref["o"][t])
            parity_log.record("o", eo, tol)
            assert eo <= tol, (i, h, t, eo)
            worst = max(worst, eo)
            if d_req is not None:
                ed = nan_max_abs(d_req[t][:, h], ref["delta"][t])
                parity_log.record("delta", ed, tol)
                assert ed <= tol, (i, h, t, ed)
                worst = max(worst, ed)
    return worst


def episode(shape, reqs=None):
    ep = make_episode(shape, reqs=reqs)
    return ep, s0_for(shape, ep, ep["reqs"])


def oracle_refs(shape, ep, S0, pairs):
    """Oracle episodes of the listed (call-local request, head) pairs."""
    return {(i, h): oracle_pair(shape, ep, S0, i, h) for (i, h) in pairs}


def check_step(shape, refs, t, o_np, d_np=None, tol=TOL):
    """Step t's outputs ([n*W][H][dv] in call-local request order) of every
    pair in refs against the oracle; errors go to the session's error log."""
    W = shape.W
    for (i, h), ref in refs.items():
        eo = nan_max_abs(o_np[i * W:(i + 1) * W, h], ref["o"][t])
        parity_log.record("o", eo, tol)
        assert eo <= tol, (i, h, t, eo)
        if d_np is not None:
            ed = nan_max_abs(d_np[i * W:(i + 1) * W, h], ref["delta"][t])
            parity_log.record("delta", ed, tol)
            assert ed <= tol, (i, h, t, ed)
