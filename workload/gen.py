"""Seeded synthetic workloads for the OneLA large-beam GDN decode step.

The OneLA pages evaluate a 0.8B Qwen3.5 generative-recommendation model at beam
width 256 with 1K/5K-token prompts and 3-7 output tokens (OneLA review,
evolve.pub, "Summary"). Neither that model nor its prompts are available, so
every input here is drawn from fixed distributions with the same shapes:

* q, k ~ N(0, 1) per component, L2-normalised over the head dimension in
  float64, rounded to float32 and then to bf16 (round to nearest even);
* v ~ N(0, 1), rounded the same way to bf16;
* alpha = sigmoid(N(2, 0.5)), beta = sigmoid(N(0, 1)), stored as float32;
* S0 ~ N(0, sigma^2) float32 per head, or the state a prompt of L synthetic
  tokens leaves behind (the prompt tokens are drawn here; folding them into a
  state is the decode arithmetic itself and is done by the caller);
* parents: uniform, beam-search-like "top W of 4W" or Zipf(1.2) rank skew.

Every stream is seeded by SeedSequence([1729, config, request, stream]), so a
request's inputs do not depend on how many other requests are generated.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

SEED_ROOT = 1729
STREAM_S0 = 0
STREAM_PROMPT = 1
STREAM_DECODE = 2
STREAM_PARENTS = 3
STREAM_RAW = 4         # raw projections of the decode step (input-side fusion)
STREAM_GATES = 5       # per-head gate parameters


@dataclass(frozen=True)
class Shape:
    cfg: int
    name: str
    R: int            # concurrent requests
    H: int            # heads
    dk: int
    dv: int
    W: int            # beam width
    T: int            # decode steps per episode
    s0: str           # "normal" or "prompt"
    s0_sigma: float   # std of S0 entries when s0 == "normal"
    prompt_len: int   # tokens folded into S0 when s0 == "prompt"
    parents: str      # "uniform", "topw4" or "zipf"
    zipf_s: float = 1.2


WORKLOADS = (
    Shape(0, "tiny_r1_h1_d32_w8_t3", 1, 1, 32, 32, 8, 3, "normal", 0.1, 0, "uniform"),
    Shape(1, "r1_h16_d128_w256_t3", 1, 16, 128, 128, 256, 3, "normal", 0.05, 0, "topw4"),
    Shape(2, "r1_h16_d128_w256_t7_prompt1024", 1, 16, 128, 128, 256, 7, "prompt", 0.0, 1024, "topw4"),
    Shape(3, "r32_h16_d128_w256_t5", 32, 16, 128, 128, 256, 5, "normal", 0.05, 0, "topw4"),
    Shape(4, "r64_h32_d128_w1024_t7_zipf1.2", 64, 32, 128, 128, 1024, 7, "normal", 0.05, 0, "zipf"),
)


def shape_of(cfg: int, **overrides) -> Shape:
    """The shape of workload `cfg`, optionally with fields replaced."""
    s = WORKLOADS[cfg]
    return replace(s, **overrides) if overrides else s


def _rng(cfg: int, req: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([SEED_ROOT, cfg, req, stream]))


# ---------------------------------------------------------------- bf16 codec
def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Exact float32 value of bf16 bit patterns."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _unit_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.standard_normal(shape)
    x = x / np.linalg.norm(x, axis=-1, keepdims=True)
    return f32_to_bf16_bits(x.astype(np.float32))


def _sigmoid32(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


# ----------------------------------------------------------------- streams
def decode_inputs(shape: Shape, req: int) -> dict:
    """q, k, v bits and alpha, beta of one request for all T steps.

    Layout: q, k [T][W][H][dk] uint16; v [T][W][H][dv] uint16; alpha, beta
    [T][W][H] float32.
    """
    rng = _rng(shape.cfg, req, STREAM_DECODE)
    T, W, H = shape.T, shape.W, shape.H
    q = _unit_bf16(rng, (T, W, H, shape.dk))
    k = _unit_bf16(rng, (T, W, H, shape.dk))
    v = f32_to_bf16_bits(rng.standard_normal((T, W, H, shape.dv)).astype(np.float32))
    alpha = _sigmoid32(rng.normal(2.0, 0.5, (T, W, H)))
    beta = _sigmoid32(rng.normal(0.0, 1.0, (T, W, H)))
    return {"q": q, "k": k, "v": v, "alpha": alpha, "beta": beta}


def s0_normal(shape: Shape, req: int) -> np.ndarray:
    """S0 [H][dv][dk] float32 ~ N(0, sigma^2)."""
    rng = _rng(shape.cfg, req, STREAM_S0)
    return rng.normal(0.0, shape.s0_sigma, (shape.H, shape.dv, shape.dk)).astype(np.float32)


def prompt_tokens(shape: Shape, req: int, length: int | None = None) -> dict:
    """Synthetic prompt tokens k, v, alpha, beta [L][H][...] for a prompt-derived S0."""
    L = shape.prompt_len if length is None else length
    rng = _rng(shape.cfg, req, STREAM_PROMPT)
    H = shape.H
    k = _unit_bf16(rng, (L, H, shape.dk))
    v = f32_to_bf16_bits(rng.standard_normal((L, H, shape.dv)).astype(np.float32))
    alpha = _sigmoid32(rng.normal(2.0, 0.5, (L, H)))
    beta = _sigmoid32(rng.normal(0.0, 1.0, (L, H)))
    return {"k": k, "v": v, "alpha": alpha, "beta": beta}


def parents_for(shape: Shape, req: int) -> np.ndarray:
    """Parent beam of every beam at every step, [T][W] int32; row 0 is -1 (no parent)."""
    rng = _rng(shape.cfg, req, STREAM_PARENTS)
    T, W = shape.T, shape.W
    par = np.full((T, W), -1, dtype=np.int32)
    if shape.parents == "uniform":
        for t in range(1, T):
            par[t] = rng.integers(0, W, size=W)
    elif shape.parents == "topw4":
        # Beam-search-like selection: beam p carries a running score s_p;
        # candidate c = 4p + j scores s_p + g_c with g ~ N(0, 1); the W best
        # candidates (score descending, lower c first on ties) survive in rank
        # order, and each survivor's parent is c // 4.
        score = np.zeros(W)
        cand_ids = np.arange(4 * W)
        for t in range(1, T):
            cand = np.repeat(score, 4) + rng.standard_normal(4 * W)
            order = np.lexsort((cand_ids, -cand))[:W]
            par[t] = order // 4
            score = cand[order]
    elif shape.parents == "zipf":
        # Beams are indexed best-first; rank r is chosen with P(r) ~ (r+1)^-s.
        p = (np.arange(1, W + 1, dtype=np.float64)) ** (-shape.zipf_s)
        p /= p.sum()
        for t in range(1, T):
            par[t] = rng.choice(W, size=W, p=p)
    else:
        raise ValueError(f"unknown parent rule {shape.parents!r}")
    return par


def raw_decode_inputs(shape: Shape, req: int) -> dict:
    """Raw projections of one request for all T steps (input-side fusion).

    q_raw, k_raw [T][W][H][dk] uint16 bf16 bits of N(0, 1) draws (not
    normalised); v [T][W][H][dv] as in `decode_inputs`; a_raw, b_raw
    [T][W][H] float32 ~ N(0, 1).
    """
    rng = _rng(shape.cfg, req, STREAM_RAW)
    T, W, H = shape.T, shape.W, shape.H
    q = f32_to_bf16_bits(rng.standard_normal((T, W, H, shape.dk)).astype(np.float32))
    k = f32_to_bf16_bits(rng.standard_normal((T, W, H, shape.dk)).astype(np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((T, W, H, shape.dv)).astype(np.float32))
    a = rng.standard_normal((T, W, H)).astype(np.float32)
    b = rng.standard_normal((T, W, H)).astype(np.float32)
    return {"q_raw": q, "k_raw": k, "v": v, "a_raw": a, "b_raw": b}


def gate_params(shape: Shape) -> dict:
    """Per-head gate parameters: A_log ~ U[0, ln 16], dt_bias ~ U[-6.9, -2.3]
    (the range that puts a layer's decay near 0.45-0.95 for N(0, 1) inputs)."""
    rng = _rng(shape.cfg, 0, STREAM_GATES)
    return {"A_log": rng.uniform(0.0, np.log(16.0), shape.H).astype(np.float32),
            "dt_bias": rng.uniform(-6.9, -2.3, shape.H).astype(np.float32)}


def make_raw_episode(shape: Shape, reqs=None) -> dict:
    """Like `make_episode` with raw projections instead of q, k, alpha, beta:
    q_raw, k_raw, v, a_raw, b_raw stacked over requests, parents [T][n][W],
    S0 [n][H][dv][dk] (drawn), and the per-head A_log, dt_bias [H]."""
    reqs = list(range(shape.R)) if reqs is None else list(reqs)
    parts = [raw_decode_inputs(shape, r) for r in reqs]
    out = {key: np.concatenate([p[key] for p in parts], axis=1) for key in parts[0]}
    out["parents"] = np.stack([parents_for(shape, r) for r in reqs], axis=1)
    out["S0"] = np.stack([s0_normal(shape, r) for r in reqs], axis=0)
    out.update(gate_params(shape))
    out["reqs"] = reqs
    return out


def make_episode(shape: Shape, reqs=None, with_s0: bool = True) -> dict:
    """All inputs of one episode for the given requests (default: all R).

    Returns q, k [T][n*W][H][dk] uint16, v [T][n*W][H][dv] uint16,
    alpha, beta [T][n*W][H] float32, parents [T][n][W] int32 (row 0 = -1) and,
    when S0 is drawn (not prompt-derived) and with_s0 is set, S0 [n][H][dv][dk]
    float32. Requests are stacked in the order given.
    """
    reqs = list(range(shape.R)) if reqs is None else list(reqs)
    parts = [decode_inputs(shape, r) for r in reqs]
    out = {key: np.concatenate([p[key] for p in parts], axis=1) for key in parts[0]}
    out["parents"] = np.stack([parents_for(shape, r) for r in reqs], axis=1)
    if with_s0 and shape.s0 == "normal":
        out["S0"] = np.stack([s0_normal(shape, r) for r in reqs], axis=0)
    out["reqs"] = reqs
    return out
