"""The prefill (prompt -> S0) through the C ABI, against the float64 oracle.

The states are compared with max-abs S_TOL = 5e-5: o = S q with a unit q
moves by at most ||dS||_max * ||q||_1 <= 5e-5 * sqrt(128) < 6e-4, inside the
decode step's 1e-3 budget; the end-to-end test checks that budget directly.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

S_TOL = 5e-5

if torch.cuda.is_available():
    import gpu_harness as gh
    from linear_attention_beam_gdn_amd import Onela, OnelaError, load_library, prefill
    from oracle import prompt_state
    from workload import bf16_bits_to_f32, f32_to_bf16_bits, prompt_tokens, shape_of
    from workload.gen_device import prompt_tokens_device


def _host_tokens(shape, n, L):
    toks = [prompt_tokens(shape, r, L) for r in range(n)]
    return {key: np.stack([t[key] for t in toks]) for key in ("k", "v", "alpha", "beta")}


def _dev(tok):
    return [gh.to_dev(tok[key]) for key in ("k", "v", "alpha", "beta")]


def _oracle(tok, i, heads=None):
    sl = slice(None) if heads is None else heads
    return prompt_state(bf16_bits_to_f32(tok["k"][i][:, sl]), bf16_bits_to_f32(tok["v"][i][:, sl]),
                        tok["alpha"][i][:, sl], tok["beta"][i][:, sl])


@pytest.mark.parametrize("d,L,H,n", [(32, 37, 2, 2), (64, 16, 3, 1), (128, 1, 2, 1), (128, 100, 2, 3),
                                     (32, 300, 2, 2), (64, 200, 3, 1)])
def test_prefill_matches_oracle(d, L, H, n):
    shape = shape_of(0, name=f"prefill_d{d}", H=H, dk=d, dv=d)
    tok = _host_tokens(shape, n, L)
    print(f"[prefill] d={d} L={L} H={H} n={n}", flush=True)
    out = prefill(*_dev(tok)).cpu().numpy()
    for i in range(n):
        err = np.abs(out[i] - _oracle(tok, i)).max()
        gh.parity_log.record("S", err, S_TOL)
        assert err <= S_TOL, (i, err)


def test_prefill_prompt_config():
    """The 1024-token prompt of the W = 256, T = 7 workload (all 16 heads)."""
    shape = shape_of(2)
    tok = _host_tokens(shape, 1, shape.prompt_len)
    print(f"[prefill] {shape.name}", flush=True)
    out = prefill(*_dev(tok)).cpu().numpy()
    err = np.abs(out[0] - _oracle(tok, 0)).max()
    print(f"[prefill] {shape.name}: max-abs err {err:.3e}")
    gh.parity_log.record("S", err, S_TOL)
    assert err <= S_TOL


def test_prefill_zero_length_and_split_prompts():
    shape = shape_of(0, name="prefill_split", H=3, dk=64, dv=64)
    L = 100
    tok = _host_tokens(shape, 2, L)
    k, v, a, b = _dev(tok)
    # no tokens: the initial state (or zero) comes back unchanged
    init = torch.randn((2, 3, 64, 64), device=gh.dev())
    empty = lambda x: x[:, :0].contiguous()
    assert torch.equal(prefill(empty(k), empty(v), empty(a), empty(b), S_init=init), init)
    assert torch.count_nonzero(prefill(empty(k), empty(v), empty(a), empty(b))) == 0
    # 100 tokens at once == 32 then 68, or 64 then 36 (in place), bit for bit (the
    # 32-token chunk pairs are the same); a split inside a pair (45 + 55) agrees to 1e-5
    whole = prefill(k, v, a, b)
    part = lambda x, s: x[:, s].contiguous()

    def two_calls(n1):
        first = prefill(part(k, slice(0, n1)), part(v, slice(0, n1)), part(a, slice(0, n1)), part(b, slice(0, n1)))
        return prefill(part(k, slice(n1, L)), part(v, slice(n1, L)), part(a, slice(n1, L)),
                       part(b, slice(n1, L)), S_init=first, out=first)

    assert torch.equal(whole, two_calls(32))
    assert torch.equal(whole, two_calls(64))
    assert (whole - two_calls(45)).abs().max().item() <= 1e-5


def test_prefill_extreme_gates_and_repeated_keys():
    """Gates at their ends and keys that repeat, where the chunk's triangular
    system is least benign (unit entries below the diagonal)."""
    shape = shape_of(0, name="prefill_gates", H=2, dk=64, dv=64)
    L = 45
    tok = _host_tokens(shape, 1, L)
    gen = torch.Generator().manual_seed(5)
    init = (0.05 * torch.randn((1, 2, 64, 64), generator=gen)).to(gh.dev())

    # alpha = 1, beta = 0 on every token: nothing is written and the initial
    # state comes back bit for bit
    t1 = dict(tok, alpha=np.ones_like(tok["alpha"]), beta=np.zeros_like(tok["beta"]))
    assert torch.equal(prefill(*_dev(t1), S_init=init), init)

    # one unit key (four entries of 1/2, exact in bf16) on every token with
    # alpha = beta = 1: each token overwrites the value stored at k, so the fold
    # is S_init (I - k k^T) + v_L k^T
    kvec = np.zeros((2, 64))
    kvec[0, [3, 17, 40, 63]] = 0.5
    kvec[1, [0, 1, 2, 3]] = 0.5
    t2 = dict(tok, k=np.broadcast_to(f32_to_bf16_bits(kvec), tok["k"].shape).copy(),
              alpha=np.ones_like(tok["alpha"]), beta=np.ones_like(tok["beta"]))
    out = prefill(*_dev(t2), S_init=init).cpu().numpy()[0]
    S_in = init.cpu().numpy()[0].astype(np.float64)
    v_last = bf16_bits_to_f32(tok["v"][0, L - 1]).astype(np.float64)
    for h in range(2):
        kk = kvec[h]
        want = S_in[h] @ (np.eye(64) - np.outer(kk, kk)) + np.outer(v_last[h], kk)
        assert np.abs(out[h] - want).max() <= S_TOL, h

    # alpha = 0 at token 20 (inside the second chunk) forgets everything before
    # it: the fold equals that of tokens 20.. alone, from a zero state
    t3 = dict(tok, alpha=tok["alpha"].copy())
    t3["alpha"][:, 20] = 0.0
    whole = prefill(*_dev(t3), S_init=init)
    tail = {key: np.ascontiguousarray(val[:, 20:]) for key, val in t3.items()}
    assert (whole - prefill(*_dev(tail))).abs().max().item() <= 1e-5
    assert np.abs(whole.cpu().numpy()[0] - _oracle(tail, 0)).max() <= S_TOL

    # gates drawn from {0, 1, ordinary} and keys drawn from three per head
    # (each also negated) over 100 tokens at d = 128, against the oracle
    shape = shape_of(0, name="prefill_gates128", H=2, dk=128, dv=128)
    t4 = _host_tokens(shape, 2, 100)
    rng = np.random.default_rng(9)
    pool = t4["k"][:, :3]
    pick = rng.integers(0, 3, size=t4["k"].shape[:3])
    n_, L_, H_ = pick.shape
    keys = pool[np.arange(n_)[:, None, None], pick, np.arange(H_)[None, None, :]]
    sign = np.where(rng.random(pick.shape) < 0.5, 0, 0x8000).astype(np.uint16)
    t4["k"] = keys ^ sign[..., None]
    for key in ("alpha", "beta"):
        pick = rng.integers(0, 3, size=t4[key].shape)
        t4[key] = np.where(pick == 0, 0.0, np.where(pick == 1, 1.0, t4[key])).astype(np.float32)
    print("[prefill] extreme gates d=128 L=100", flush=True)
    out = prefill(*_dev(t4)).cpu().numpy()
    for i in range(2):
        err = np.abs(out[i] - _oracle(t4, i)).max()
        gh.parity_log.record("S", err, S_TOL)
        assert err <= S_TOL, (i, err)


def test_prompt_init_equals_float32_init_and_decodes_within_budget():
    """S0 folded into the planes on the GPU == onela_init_request of the
    prefill's float32 state (bit-identical decode), and the decode outputs
    match the oracle run from the oracle's own S0 within 1e-3."""
    shape = shape_of(2, name="prompt_e2e", H=4, T=3, prompt_len=300)
    ep, S0_oracle = gh.episode(shape)
    tok = _host_tokens(shape, 1, shape.prompt_len)
    k, v, a, b = _dev(tok)
    print(f"[prefill] {shape.name}", flush=True)
    S_gpu = prefill(k, v, a, b)
    ref = gh.run_episode(shape, ep, S_gpu.cpu().numpy())
    lay = Onela(2, shape.H, 128, 128, shape.W, shape.T)
    lay.init_requests_from_prompts([1], k, v, a, b)
    o = torch.empty((shape.W, shape.H, 128), dtype=torch.float32, device=gh.dev())
    for t in range(shape.T):
        par = gh.to_dev(ep["parents"][t].astype(np.int32)) if t else None
        lay.step([1], *[gh.to_dev(ep[key][t]) for key in ("q", "k", "v", "alpha", "beta")], par, o)
        assert np.array_equal(o.cpu().numpy(), ref["o"][t])
    lay.close()
    ref["layer"].close()
    for h in range(shape.H):
        want = gh.oracle_pair(shape, ep, S0_oracle, 0, h)
        eo, ed = gh.max_err(ref, want, 0, h, shape.W)
        assert eo <= gh.TOL and ed <= gh.TOL, (h, eo, ed)


def test_prefill_bench_size_sampled():
    """32 prompts of 5120 tokens, 16 heads, d = 128 in one launch (the S0 of
    the 32-request bench workload); three (request, head) pairs against the
    oracle on the same seeded tokens."""
    shape = shape_of(3, s0="prompt", prompt_len=5120)
    print(f"[prefill] {shape.name} prompt {shape.prompt_len}", flush=True)
    toks = prompt_tokens_device(shape, gh.dev())
    out = prefill(toks["k"], toks["v"], toks["alpha"], toks["beta"])
    torch.cuda.synchronize()
    for r, h in [(0, 0), (17, 9), (31, 15)]:
        host = {key: toks[key][r:r + 1, :, h:h + 1].cpu().numpy() for key in toks}
        host["k"] = host["k"].view(np.uint16)
        host["v"] = host["v"].view(np.uint16)
        want = _oracle(host, 0)[0]
        err = np.abs(out[r, h].cpu().numpy() - want).max()
        print(f"[prefill] pair ({r}, {h}): max-abs err {err:.3e}", flush=True)
        gh.parity_log.record("S", err, S_TOL)
        assert err <= S_TOL


def test_prompt_init_more_requests_than_one_launch():
    """70 requests (more than one launch carries) folded into the planes; each
    equals the float32 fold of its own prompt put through onela_init_request."""
    shape = shape_of(0, name="prompt_many", H=2, dk=32, dv=32, W=8, T=2, R=70)
    toks = prompt_tokens_device(shape, gh.dev(), length=20)
    args = [toks[key] for key in ("k", "v", "alpha", "beta")]
    S = prefill(*args)
    a = Onela(70, 2, 32, 32, 8, 2)
    b = Onela(70, 2, 32, 32, 8, 2)
    a.init_requests_from_prompts(list(range(70)), *args)
    for r in range(70):
        b.init_request(r, S[r].contiguous())
    ep, _ = gh.episode(shape_of(0, name="prompt_many", H=2, dk=32, dv=32, W=8, T=2, R=70))
    o_a = torch.empty((70 * 8, 2, 32), dtype=torch.float32, device=gh.dev())
    o_b = torch.empty_like(o_a)
    for t in range(2):
        par = gh.to_dev(ep["parents"][t].astype(np.int32)) if t else None
        ins = [gh.to_dev(ep[key][t]) for key in ("q", "k", "v", "alpha", "beta")]
        a.step(list(range(70)), *ins, par, o_a)
        b.step(list(range(70)), *ins, par, o_b)
        assert torch.equal(o_a, o_b)
    a.close()
    b.close()


def test_prefill_bad_arguments():
    shape = shape_of(0, name="prefill_bad", H=2, dk=32, dv=32)
    tok = _host_tokens(shape, 1, 8)
    k, v, a, b = _dev(tok)
    lib = load_library()
    out = torch.empty((1, 2, 32, 32), device=gh.dev())
    ptr = lambda t: t.data_ptr()
    call = lambda n, dk, L, kk=ptr(k), o=ptr(out): lib.onela_prefill(n, 2, dk, dk, L, kk, ptr(v), ptr(a), ptr(b),
                                                                     None, o, None)
    assert call(0, 32, 8) == -1                 # no sequences
    assert call(1, 32, -1) == -1                # negative length
    assert call(1, 48, 8) == -7                 # no kernel for d = 48
    assert call(1, 32, 8, kk=ptr(k) + 2) == -1  # misaligned k
    assert call(1, 32, 8, o=0) == -1            # no output
    lay = Onela(2, 2, 32, 32, 8, 3)
    with pytest.raises(OnelaError):
        lay.init_requests_from_prompts([0, 0], torch.cat([k, k]), torch.cat([v, v]), torch.cat([a, a]),
                                       torch.cat([b, b]))   # duplicate request id
    with pytest.raises(OnelaError):
        lay.init_requests_from_prompts([2], k, v, a, b)     # request id out of range
    lay.close()
