"""Seeded synthetic inputs generated on the GPU, for workloads too large to draw on the host.

Same distributions as `workload.gen` (q, k ~ N(0,1) L2-normalised over the head
dimension then rounded to bf16; v ~ N(0,1) in bf16; alpha = sigmoid(N(2, 0.5)),
beta = sigmoid(N(0, 1)) in float32; S0 ~ N(0, sigma^2)), drawn with torch's
device generator and normalised in float32. Every stream is seeded from
(1729, config, step or request, stream), so a step's inputs do not depend on
the other steps. Holds none of the decode step's arithmetic.
"""
from __future__ import annotations

import numpy as np
import torch

from .gen import SEED_ROOT, Shape, parents_for


def _gen(device, *key) -> torch.Generator:
    seed = int(np.random.SeedSequence([SEED_ROOT, *key]).generate_state(1, dtype=np.uint64)[0] >> 1)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def step_inputs(shape: Shape, t: int, device) -> dict:
    """Inputs of step t (0-based) for all R requests, on `device`.

    q, k: int16 bf16 bits [R*W][H][dk]; v: [R*W][H][dv]; alpha, beta: float32 [R*W][H].
    """
    n = shape.R * shape.W
    g = _gen(device, shape.cfg, 1000 + t, 0)

    def unit(d):
        x = torch.randn((n, shape.H, d), generator=g, device=device, dtype=torch.float32)
        x = x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)
        return x.to(torch.bfloat16).view(torch.int16)

    q = unit(shape.dk)
    k = unit(shape.dk)
    v = torch.randn((n, shape.H, shape.dv), generator=g, device=device, dtype=torch.float32)
    v = v.to(torch.bfloat16).view(torch.int16)
    alpha = torch.sigmoid(torch.randn((n, shape.H), generator=g, device=device) * 0.5 + 2.0)
    beta = torch.sigmoid(torch.randn((n, shape.H), generator=g, device=device))
    return {"q": q, "k": k, "v": v, "alpha": alpha.float().contiguous(), "beta": beta.float().contiguous()}


def s0_device(shape: Shape, device) -> torch.Tensor:
    """S0 [R][H][dv][dk] float32 ~ N(0, sigma^2) on `device`."""
    g = _gen(device, shape.cfg, 0, 1)
    return torch.randn((shape.R, shape.H, shape.dv, shape.dk), generator=g, device=device) * shape.s0_sigma


def prompt_tokens_device(shape: Shape, device, length: int | None = None, reqs=None) -> dict:
    """Prompt tokens of the requests, on `device`, for a prompt-derived S0.

    k: int16 bf16 bits [n][L][H][dk] (L2-normalised); v: [n][L][H][dv];
    alpha, beta: float32 [n][L][H]. Seeded per request, so a request's
    prompt does not depend on which other requests are drawn.
    """
    L = shape.prompt_len if length is None else length
    reqs = range(shape.R) if reqs is None else reqs
    ks, vs, als, bes = [], [], [], []
    for r in reqs:
        g = _gen(device, shape.cfg, 3000 + r, 3)
        x = torch.randn((L, shape.H, shape.dk), generator=g, device=device, dtype=torch.float32)
        x = x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)
        ks.append(x.to(torch.bfloat16).view(torch.int16))
        v = torch.randn((L, shape.H, shape.dv), generator=g, device=device, dtype=torch.float32)
        vs.append(v.to(torch.bfloat16).view(torch.int16))
        als.append(torch.sigmoid(torch.randn((L, shape.H), generator=g, device=device) * 0.5 + 2.0))
        bes.append(torch.sigmoid(torch.randn((L, shape.H), generator=g, device=device)))
    return {"k": torch.stack(ks), "v": torch.stack(vs),
            "alpha": torch.stack(als).float().contiguous(), "beta": torch.stack(bes).float().contiguous()}


def all_parents(shape: Shape) -> np.ndarray:
    """Parents [T][R][W] int32 (row 0 = -1), drawn on the host like `workload.gen`."""
    return np.stack([parents_for(shape, r) for r in range(shape.R)], axis=1)
