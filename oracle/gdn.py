"""Float64 reference of the OneLA GDN decode step (test infrastructure only).

Sources (the OneLA pages):
* OneLA abstract (readsearch.ai page): all beams of a request share one
  prompt-derived state and differ by append-only transition records; an
  ancestry index lists the records that make up each beam's history, and beams
  advance without moving or copying records.
* OneLA review (evolve.pub), "Summary", "Key claims", "Strengths" and "Scope &
  Claims": the Gated DeltaNet recurrence (paper Eq. 2), the record
  (alpha_t, delta_t, k_t) with delta_t computed when the record is written, and
  projection replay (paper Eq. 3-4), which right-multiplies the recurrence by
  q_t and k_t and expands it over the ancestry with two d_v-long accumulators.

The pages name the equations without printing them. The reading used here
(standard GDN delta rule, post-update output):
    delta_t = beta_t * (v_t - alpha_t * S_{t-1} k_t)
    S_t     = alpha_t * S_{t-1} + delta_t k_t^T
    o_t     = S_t q_t
with S of shape (d_v, d_k), no query scaling and no normalisation inside.

Step and record conventions: steps are t = 1..T. At t = 1 every beam starts
from S0 and parents are ignored; at t >= 2 beam b continues from the state
beam parents[t-1][b] held after step t-1. The record written by beam b at
step t has id rid(t, b) = (t-1)*W + b. The ancestry of beam b at step t lists
the ids of the records its state is built from, oldest first (t-1 of them).
"""
from __future__ import annotations

import numpy as np


def rid(t: int, b: int, W: int) -> int:
    """Id of the record beam b appends at step t (t >= 1)."""
    return (t - 1) * W + b


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def full_state_episode(S0, q, k, v, alpha, beta, parents, return_states=False):
    """Run T decode steps for one (request, head) with a full state per beam.

    S0: (dv, dk); q, k: (T, W, dk); v: (T, W, dv); alpha, beta: (T, W);
    parents: (T, W) integers, row 0 ignored, rows t >= 1 in [0, W).

    Returns a dict with
      o, delta       (T, W, dv)   output S_t q_t and delta_t of every beam/step
      rec_alpha      (T*W,)       record store indexed by record id
      rec_delta      (T*W, dv)
      rec_k          (T*W, dk)
      anc            list of T int arrays (W, t-1): record ids of each beam's
                     history at step t (oldest first)
      states         (T, W, dv, dk) S_t of every beam (only if return_states)
    """
    S0 = _f64(S0)
    q, k, v = _f64(q), _f64(k), _f64(v)
    alpha, beta = _f64(alpha), _f64(beta)
    parents = np.asarray(parents)
    T, W, dk = k.shape
    dv = v.shape[2]
    assert S0.shape == (dv, dk)

    o = np.empty((T, W, dv))
    delta = np.empty((T, W, dv))
    rec_alpha = np.empty(T * W)
    rec_delta = np.empty((T * W, dv))
    rec_k = np.empty((T * W, dk))
    anc_tables = []
    states = np.empty((T, W, dv, dk)) if return_states else None

    S_prev = None
    anc_prev = None
    for t in range(1, T + 1):
        i = t - 1
        if t == 1:
            P = np.broadcast_to(S0, (W, dv, dk))
            anc = np.zeros((W, 0), dtype=np.int64)
        else:
            p = parents[i].astype(np.int64)
            if p.min() < 0 or p.max() >= W:
                raise ValueError(f"parent index out of range at step {t}")
            P = S_prev[p]
            # A beam's history is its parent's history plus the parent's own
            # record of step t-1; only ids are copied, never records.
            anc = np.concatenate([anc_prev[p], (rid(t - 1, 0, W) + p)[:, None]], axis=1)
        a = alpha[i][:, None]
        u = np.einsum("bij,bj->bi", P, k[i])                       # S_{t-1} k_t
        d = beta[i][:, None] * (v[i] - a * u)                        # delta_t
        S_new = a[:, :, None] * P + d[:, :, None] * k[i][:, None, :]  # S_t
        o[i] = np.einsum("bij,bj->bi", S_new, q[i])                  # S_t q_t
        delta[i] = d
        ids = rid(t, 0, W) + np.arange(W)
        rec_alpha[ids] = alpha[i]
        rec_delta[ids] = d
        rec_k[ids] = k[i]
        anc_tables.append(anc)
        if return_states:
            states[i] = S_new
        S_prev, anc_prev = S_new, anc

    out = {"o": o, "delta": delta, "rec_alpha": rec_alpha, "rec_delta": rec_delta,
           "rec_k": rec_k, "anc": anc_tables}
    if return_states:
        out["states"] = states
    return out


def prompt_state(k, v, alpha, beta, S_init=None):
    """Fold a prompt of L tokens into one state with the same recurrence (W = 1).

    k: (L, H, dk); v: (L, H, dv); alpha, beta: (L, H). Returns S (H, dv, dk)
    in float64; callers that need the float32 S0 round it themselves.
    """
    k, v = _f64(k), _f64(v)
    alpha, beta = _f64(alpha), _f64(beta)
    L, H, dk = k.shape
    dv = v.shape[2]
    S = np.zeros((H, dv, dk)) if S_init is None else _f64(S_init).copy()
    for s in range(L):
        a = alpha[s][:, None]
        u = np.einsum("hij,hj->hi", S, k[s])
        d = beta[s][:, None] * (v[s] - a * u)
        S = a[:, :, None] * S + d[:, :, None] * k[s][:, None, :]
    return S


def ancestry_walk(parents, t: int, W: int) -> np.ndarray:
    """Record ids of every beam's history at step t by walking parent pointers.

    Independent of `full_state_episode`: starts at beam b of step t and follows
    parents back to step 1, collecting the id of each ancestor's record.
    Returns (W, t-1) ids, oldest first.
    """
    out = np.zeros((W, t - 1), dtype=np.int64)
    for b in range(W):
        cur = b
        for s in range(t, 1, -1):          # the parent of step s lives at step s-1
            p = int(parents[s - 1][cur])
            out[b, s - 2] = rid(s - 1, p, W)
            cur = p
    return out


def replay_episode(S0, q, k, v, alpha, beta, parents):
    """The same T steps by projection replay, without any per-beam matrix.

    For x in {k_t, q_t}: y <- S0 x, then for each ancestral record
    (alpha_j, delta_j, k_j), oldest first, y <- alpha_j * y + (k_j . x) * delta_j,
    which leaves y = S_{t-1} x. Then delta_t = beta_t (v_t - alpha_t y_k) and
    o_t = alpha_t y_q + (k_t . q_t) delta_t, which is S_t q_t. Histories come
    from `ancestry_walk`; records are the ones this routine itself wrote.
    Returns o, delta (T, W, dv).
    """
    S0 = _f64(S0)
    q, k, v = _f64(q), _f64(k), _f64(v)
    alpha, beta = _f64(alpha), _f64(beta)
    T, W, dk = k.shape
    dv = v.shape[2]
    rec_a = np.empty(T * W)
    rec_d = np.empty((T * W, dv))
    rec_k = np.empty((T * W, dk))
    o = np.empty((T, W, dv))
    delta = np.empty((T, W, dv))
    for t in range(1, T + 1):
        i = t - 1
        hist = ancestry_walk(parents, t, W)
        for b in range(W):
            kt, qt = k[i, b], q[i, b]
            yk = S0 @ kt
            yq = S0 @ qt
            for r in hist[b]:
                yk = rec_a[r] * yk + (rec_k[r] @ kt) * rec_d[r]
                yq = rec_a[r] * yq + (rec_k[r] @ qt) * rec_d[r]
            d = beta[i, b] * (v[i, b] - alpha[i, b] * yk)
            o[i, b] = alpha[i, b] * yq + (kt @ qt) * d
            delta[i, b] = d
        ids = rid(t, 0, W) + np.arange(W)
        rec_a[ids] = alpha[i]
        rec_d[ids] = delta[i]
        rec_k[ids] = k[i]
    return {"o": o, "delta": delta}


# ------------------------------------------------------ input-side fusion
# The pages do not describe how a layer forms q, k, alpha and beta from its
# projections. The reading used here is the usual gated DeltaNet layer: q and
# k are L2-normalised per head, alpha = exp(-exp(A_log) * softplus(a + dt_bias))
# with per-head parameters A_log and dt_bias, and beta = sigmoid(b).

def _bf16_round(x32) -> np.ndarray:
    """float32 values rounded to the nearest bf16 (ties to even), as float32."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32)


def unit_rows(x, eps=1e-6) -> np.ndarray:
    """x / sqrt(sum of squares + eps) over the last axis, in float64: the
    plain definition of the per-head L2 normalisation of q and k, before the
    step rounds them to the bf16 it consumes."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def fused_inputs(q_raw, k_raw, a_raw, b_raw, A_log, dt_bias, eps=1e-6):
    """Decode-step inputs from raw projections.

    q_raw, k_raw: [..., H, d] float values; a_raw, b_raw: [..., H];
    A_log, dt_bias: [H]. Returns (q, k, alpha, beta): q and k divided by
    sqrt(sum of squares + eps) per head in float32 and rounded to bf16 (the
    precision the step consumes them in, so both sides take that rounding
    decision in the same precision; `unit_rows` is the float64 definition it
    is pinned against), alpha and beta in float64.
    """
    def unit(x):
        x = np.asarray(x, dtype=np.float32)
        s = np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32) + np.float32(eps)
        return _bf16_round(x / np.sqrt(s))

    a = _f64(a_raw) + _f64(dt_bias)
    softplus = np.where(a > 20.0, a, np.log1p(np.exp(np.minimum(a, 20.0))))
    alpha = np.exp(-np.exp(_f64(A_log)) * softplus)
    beta = 1.0 / (1.0 + np.exp(-_f64(b_raw)))
    return unit(q_raw), unit(k_raw), alpha, beta
