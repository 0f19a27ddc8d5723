"""Error paths and lifecycle of the C ABI, forced from the host.

Every misuse here is rejected by the host before anything is enqueued, except
the out-of-range parent, which the kernel's own range check turns into the
request's error word (it clamps the index, so nothing is read out of bounds).
"""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_harness as gh
    from linear_attention_beam_gdn_amd import Onela, OnelaError
    from linear_attention_beam_gdn_amd.onela import _Config, load_library
    from workload import shape_of


def _small():
    shape = shape_of(0, H=2, R=1)
    ep, S0 = gh.episode(shape)
    return shape, ep, S0


def _inputs(shape, ep, t):
    return (gh.to_dev(ep["q"][t]), gh.to_dev(ep["k"][t]), gh.to_dev(ep["v"][t]),
            gh.to_dev(ep["alpha"][t]), gh.to_dev(ep["beta"][t]))


def _status(exc_info):
    return exc_info.value.status


def test_create_rejects_bad_configs():
    lib = load_library()
    out = ctypes.c_void_p()
    bad = [(0, 1, 32, 32, 8, 3), (1, 1, 48, 48, 8, 3), (1, 1, 32, 64, 8, 3), (1, 1, 32, 32, 0, 3),
           (1, 1, 32, 32, 8, 0), (1, 1, 32, 32, 8, 65),
           (1, 64, 32, 32, 1 << 20, 3),      # W*H*d reaches 2^31: 32-bit offsets would overflow
           (1, 1, 128, 128, 1 << 18, 64)]    # T*W*d reaches 2^31
    expect = [-1, -7, -7, -1, -1, -7, -7, -7]
    for cfg, e in zip(bad, expect):
        c = _Config(*cfg)
        assert lib.onela_create(ctypes.byref(c), None, ctypes.byref(out)) == e, cfg
        assert not out.value
    assert lib.onela_create(None, None, ctypes.byref(out)) == -1
    assert lib.onela_status_string(-4) == b"parent index outside [0, W)"


def test_host_misuse_is_rejected_without_side_effects():
    shape, ep, S0 = _small()
    lay = Onela(2, shape.H, 32, 32, shape.W, shape.T)
    o = torch.empty((shape.W, shape.H, 32), dtype=torch.float32, device=gh.dev())
    q, k, v, a, b = _inputs(shape, ep, 0)
    with pytest.raises(OnelaError) as e:          # never initialised
        lay.step([0], q, k, v, a, b, None, o)
    assert _status(e) == -2
    lay.init_request(0, gh.to_dev(S0[0]))
    for reqs, st in (([2], -1), ([-1], -1)):
        with pytest.raises(OnelaError) as e:
            lay.step(reqs, q, k, v, a, b, None, o)
        assert _status(e) == st
    with pytest.raises(OnelaError) as e:
        lay.init_request(5, gh.to_dev(S0[0]))
    assert _status(e) == -1
    # raw ABI: NULL pointers and duplicate ids
    lib = lay.lib
    arr = (ctypes.c_int32 * 2)(0, 0)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    assert lib.onela_step(lay._ctx, 2, arr, p(q), p(k), p(v), p(a), p(b), None, p(o), None) == -1
    arr1 = (ctypes.c_int32 * 1)(0)
    assert lib.onela_step(lay._ctx, 1, arr1, None, p(k), p(v), p(a), p(b), None, p(o), None) == -1
    assert lib.onela_step(lay._ctx, 1, arr1, p(q), p(k), p(v), p(a), p(b), None, None, None) == -1
    # no requests, or more than the context holds
    assert lib.onela_step(lay._ctx, 0, arr1, p(q), p(k), p(v), p(a), p(b), None, p(o), None) == -1
    arr3 = (ctypes.c_int32 * 3)(0, 1, 0)
    assert lib.onela_step(lay._ctx, 3, arr3, p(q), p(k), p(v), p(a), p(b), None, p(o), None) == -1
    assert lay.get_step(0) == 0                    # nothing above advanced the request
    # tuning knobs: values outside their ranges
    assert lib.onela_set_beam_order(lay._ctx, 2) == -1
    assert lib.onela_set_beam_order(lay._ctx, -2) == -1
    assert lib.onela_set_beam_order(None, 0) == -1
    assert lib.onela_set_beams_per_block(lay._ctx, 100) == -1
    # step 1 works, step 2 needs parents
    lay.step([0], q, k, v, a, b, None, o)
    q, k, v, a, b = _inputs(shape, ep, 1)
    with pytest.raises(OnelaError) as e:
        lay.step([0], q, k, v, a, b, None, o)
    assert _status(e) == -1
    assert lay.get_step(0) == 1
    lay.close()


def test_capacity_reset_and_rerun_identical():
    shape, ep, S0 = _small()
    lay = Onela(1, shape.H, 32, 32, shape.W, shape.T)
    lay.init_request(0, gh.to_dev(S0[0]))
    o = torch.empty((shape.W, shape.H, 32), dtype=torch.float32, device=gh.dev())

    def episode():
        res = []
        for t in range(shape.T):
            par = gh.to_dev(ep["parents"][t].astype(np.int32)) if t else None
            lay.step([0], *_inputs(shape, ep, t), par, o)
            res.append(o.cpu().numpy().copy())
        return res

    first = episode()
    with pytest.raises(OnelaError) as e:
        lay.step([0], *_inputs(shape, ep, 0), gh.to_dev(ep["parents"][1].astype(np.int32)), o)
    assert _status(e) == -3
    lay.reset(0)
    assert lay.get_step(0) == 0
    second = episode()
    for a_, b_ in zip(first, second):
        assert np.array_equal(a_, b_)
    # re-init with another S0 changes the outputs; re-init with the first restores them
    lay.init_request(0, gh.to_dev(S0[0] * 2))
    third = episode()
    assert not np.array_equal(third[0], first[0])
    lay.init_request(0, gh.to_dev(S0[0]))
    fourth = episode()
    assert all(np.array_equal(a_, b_) for a_, b_ in zip(first, fourth))
    lay.close()


@pytest.mark.parametrize("order,bad", [(-1, "W"), (1, "W"), (1, -7)])
def test_parent_out_of_range_poisons_request(order, bad):
    # (order 1: the bad parent also enters the ancestry-order sort, which clamps it)
    shape, ep, S0 = _small()
    lay = Onela(2, shape.H, 32, 32, shape.W, shape.T)
    lay.set_beam_order(order)
    for r in (0, 1):
        lay.init_request(r, gh.to_dev(S0[0]))
    W = shape.W
    o = torch.empty((2 * W, shape.H, 32), dtype=torch.float32, device=gh.dev())
    cat = lambda key, t: gh.to_dev(np.concatenate([ep[key][t], ep[key][t]], axis=0))
    ins = lambda t: (cat("q", t), cat("k", t), cat("v", t), cat("alpha", t), cat("beta", t))
    lay.step([0, 1], *ins(0), None, o)
    par = np.stack([ep["parents"][1][0], ep["parents"][1][0]]).astype(np.int32)
    par[1, 3] = W if bad == "W" else bad            # request 1: one parent out of range
    lay.step([0, 1], *ins(1), gh.to_dev(par), o)
    with pytest.raises(OnelaError) as e:
        lay.sync()
    assert _status(e) == -4
    assert lay.get_step(0) == 2                     # request 0 is unaffected
    with pytest.raises(OnelaError) as e:
        lay.get_step(1)
    assert _status(e) == -4
    with pytest.raises(OnelaError) as e:            # poisoned request refuses to step
        lay.step([1], *_inputs(shape, ep, 2), gh.to_dev(par[1:2]), o[:W])
    assert _status(e) == -2
    lay.reset(1)
    lay.sync()                                      # poison cleared
    assert lay.get_step(1) == 0
    lay.close()


def test_memory_accounting():
    shape = shape_of(1)
    lay = Onela(1, shape.H, 128, 128, shape.W, shape.T)
    m = lay.memory()
    assert m["s0_bytes"] == shape.H * 128 * 128 * 4
    assert m["record_bytes"] == shape.H * shape.T * shape.W * (4 + 4 * 128 + 2 * 128)
    # ancestry rows (two parities), the order (two parities) and the order of
    # every step, + 5 words per request
    assert m["index_bytes"] == 2 * shape.W * shape.T * 4 + 2 * shape.W * 4 + shape.T * shape.W * 4 + 5 * 4
    lay.close()
    wide = Onela(1, 1, 32, 32, 2048, 2)                 # wider than the ordered beam sets: no order history
    assert wide.memory()["index_bytes"] == 2 * 2048 * 2 * 4 + 2 * 2048 * 4 + 5 * 4
    wide.close()
