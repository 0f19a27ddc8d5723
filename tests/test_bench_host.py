"""Host-side accounting of bench.py that the reported roofline rests on: the
distinct ancestral records a step reads (against a brute-force parent walk),
the algorithmic bytes per launch (against the byte counts written out by
hand for a small case), and the counter summary (against synthetic counter
files with known values). No GPU needed."""
import csv
import os

import numpy as np
import pytest

import bench
from oracle import ancestry_walk
from workload import shape_of
from workload.gen import parents_for


def _brute_unique(parents_req, t, W):
    """Record ids every beam of step t reads, as a set, from the oracle's walk."""
    if t < 2:
        return 0
    return len(set(ancestry_walk(parents_req, t, W).ravel().tolist()))


@pytest.mark.parametrize("cfg,W,T", [(0, 8, 3), (1, 64, 5), (4, 128, 7)])
def test_unique_ancestors_matches_parent_walk(cfg, W, T):
    shape = shape_of(cfg, W=W, T=T)
    for r in range(2):
        par = parents_for(shape, r)
        for t in range(1, T + 1):
            assert bench.unique_ancestors(par, t) == _brute_unique(par, t, W), (cfg, r, t)


def test_step_bytes_small_case_by_hand():
    # 1 request, 1 head, d = 32, W = 2, T = 3; both step-2 beams descend from step-1
    # beam 0, step-3 beams from step-2 beams 0 and 1
    shape = shape_of(0, R=1, H=1, dk=32, dv=32, W=2, T=3)
    par = np.array([[-1, -1], [0, 0], [0, 1]], dtype=np.int32)[:, None, :]     # [T][R][W]
    rec = 4 + 4 * 32 + 2 * 32                                                   # alpha, delta, k
    s0 = 4 * 32 * 32
    inputs = 2 * (2 * 32 + 2 * 32 + 2 * 32 + 8)
    append = 2 * rec
    o = 2 * 4 * 32
    b1, b2, b3 = (bench.step_bytes(shape, par, t) for t in (1, 2, 3))
    assert b1["unique_records"] == 0 and b1["total"] == s0 + inputs + append + o
    # step 2: one distinct record (step 1, beam 0); ancestry rows 1 entry x 2 beams, read and written
    assert b2["unique_records"] == 1
    assert b2["total"] == s0 + inputs + append + o + rec + 2 * 4 * 2
    # step 3: records (2, 0), (2, 1) and (1, 0)
    assert b3["unique_records"] == 3
    assert b3["total"] == s0 + inputs + append + o + 3 * rec + 2 * 4 * 4


def _write_counter_run(d, rows, agent):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for disp, name, counters in rows:
            for cn, cv in counters.items():
                w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": cn, "Counter_Value": cv})
    with open(os.path.join(d, "run_agent_info.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Simd_Count", "Cu_Count", "Num_Xcc"])
        w.writeheader()
        w.writerow({"Name": "gfx950", **agent})


def test_counter_summary_arithmetic(tmp_path, monkeypatch):
    agent = {"Simd_Count": 1024, "Cu_Count": 256, "Num_Xcc": 8}
    name = "void onela::(anonymous namespace)::step_kernel<128, 128, false, 1>(onela::StepParams)"
    gui = 8 * 1000.0                                  # 1000 cycles per XCD
    # MFMA busy cycles summed over SIMDs: 25% of 1024 SIMDs x 1000 cycles
    c1 = {"SQ_WAVES": 100.0, "SQ_WAVE_CYCLES": 1e6, "SQ_WAIT_ANY": 6e5, "SQ_ACTIVE_INST_ANY": 1e5,
          "GRBM_GUI_ACTIVE": gui}
    c2 = {"SQ_INSTS_VALU": 2e5 + 1e4, "SQ_INSTS_MFMA": 1e4, "SQ_VALU_MFMA_BUSY_CYCLES": 0.25 * 1024 * 1000,
          "SQ_INSTS_LDS": 5e3, "SQ_INSTS_VMEM_RD": 1e3, "SQ_INSTS_VMEM_WR": 5e2, "SQ_INSTS_SALU": 1.0,
          "SQ_INSTS_VALU_MFMA_MOPS_BF16": 1e6, "GRBM_GUI_ACTIVE": gui}
    c3 = {"SQ_LDS_BANK_CONFLICT": 2e4, "SQ_LDS_IDX_ACTIVE": 1e5, "SQ_WAVES": 100.0, "GRBM_GUI_ACTIVE": gui}
    dirs = []
    for i, c in enumerate((c1, c2, c3)):
        d = str(tmp_path / f"c{i}")
        _write_counter_run(d, [(7, name, c)], agent)
        dirs.append(d)
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(tmp_path / "counters.txt"))
    text = bench.counters_from(dirs, "test")
    row = next(line for line in text.splitlines() if line.startswith("| step_kernel<128, 128, false, *>"))
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[2] == "25.0%"                        # MFMA busy
    assert cells[3] == "78%"                          # 4 x 2e5 non-MFMA VALU / (1024 x 1000)
    assert cells[4] == "39.1%"                        # LDS 1e5 / (256 x 1000)
    assert cells[5] == "20.0%"                        # bank conflicts 2e4 / 1e5
    assert cells[6] == "60%" and cells[7] == "10%"    # wait / issue over wave cycles
    assert cells[8] == "2100"                         # VALU per wave (2.1e5 / 100)


def test_profile_by_depth_arithmetic(tmp_path):
    """Per-depth traffic summary of the 4-layer leg from synthetic FETCH_SIZE /
    WRITE_SIZE runs: every layer-step of depth t reports (100 + t) MB fetched
    and 50 MB written as counted, a 64 MiB copy counts half its bytes as fetched
    and all as written, so the scaled bytes are 2 (100 + t) MB and 50 MB."""
    agent = {"Simd_Count": 1024, "Cu_Count": 256, "Num_Xcc": 8}
    name = "void onela::(anonymous namespace)::step_kernel<128, 128, false, 1, 64>(onela::StepParams)"
    T, layers, episodes = 5, 4, 2
    copy = 64 * 2.0 ** 20
    runs = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        rows = [(0, "__amd_rocclr_copyBuffer", {counter: (copy / 2 if counter == "FETCH_SIZE" else copy) / 1024})]
        i = 1
        for _ in range(episodes):
            for t in range(T):
                for _ in range(layers):
                    mb = (100 + t + 1) * 1e6 if counter == "FETCH_SIZE" else 50e6
                    rows.append((i, name, {counter: mb / 1024}))
                    i += 1
        d = str(tmp_path / counter)
        _write_counter_run(d, rows, agent)
        runs[counter] = d
    text = bench.profile_by_depth("multi_layer", runs["FETCH_SIZE"], runs["WRITE_SIZE"], [], 64, "test",
                                  out_dir=str(tmp_path))
    assert os.path.exists(tmp_path / "step_kernel_4layers_r32_h16_w256_t5_by_depth.txt")
    lines = [line for line in text.splitlines() if line.startswith("| ") and line[2].isdigit()]
    assert len(lines) == T
    shape = shape_of(3)
    par = np.stack([parents_for(shape, r) for r in range(shape.R)], axis=1)
    for t, line in enumerate(lines):
        cells = [c.strip() for c in line.strip("|").split("|")]
        assert int(cells[0]) == t + 1 and int(cells[1]) == episodes * layers
        assert float(cells[2]) == pytest.approx(2 * (100 + t + 1), abs=0.05)      # fetch MB, scaled
        assert float(cells[3]) == pytest.approx(50.0, abs=0.05)                   # write MB
        alg = bench.step_bytes(shape, par, t + 1)["total"]
        assert float(cells[5]) == pytest.approx(alg / 1e6, abs=0.05)
        assert float(cells[6]) == pytest.approx((2 * (100 + t + 1) + 50) * 1e6 / alg, abs=5e-4)


def test_depth_stats_percentiles():
    per = np.array([[float(i), 10.0 * i] for i in range(1, 11)])   # 10 episodes, 2 depths
    st = bench.depth_stats(per)
    assert st["episodes"] == 10
    assert st["median"] == [5.5, 55.0]
    assert st["p10"] == [round(float(np.percentile(per[:, 0], 10)), 2), round(float(np.percentile(per[:, 1], 10)), 2)]
    assert st["p90"][1] == round(float(np.percentile(per[:, 1], 90)), 2)


def test_cpu_baseline_error_check(monkeypatch):
    """The CPU baseline's check of the GPU outputs: outputs equal to the
    oracle's give zero error; an output moved by a known amount in one element
    gives exactly that error, on o or delta alone; pairs without outputs are
    timed but not checked."""
    from oracle import full_state_episode
    from workload import bf16_bits_to_f32, make_episode

    monkeypatch.setenv("OMP_NUM_THREADS", "2")
    shape = shape_of(0, R=2, H=2, W=8, T=3)
    ep = make_episode(shape)
    pairs = bench.baseline_pairs(shape, 3)
    W = shape.W

    def ref(r, h):
        sl = slice(r * W, (r + 1) * W)
        f = lambda key: bf16_bits_to_f32(ep[key][:, sl, h, :])
        return full_state_episode(ep["S0"][r, h], f("q"), f("k"), f("v"), ep["alpha"][:, sl, h],
                                  ep["beta"][:, sl, h], ep["parents"][:, r, :])

    r0, h0 = pairs[0]
    out = ref(r0, h0)
    exact = {(r0, h0): (out["o"].copy(), out["delta"].copy())}
    res = bench.cpu_baseline(shape, ep, 3, gpu_outputs=exact)
    assert res["max_abs_err_vs_gpu"]["o"] == 0.0 and res["max_abs_err_vs_gpu"]["delta"] == 0.0
    assert res["max_abs_err_vs_gpu"]["pairs"] == 1              # distinct pairs checked
    moved = (out["o"].copy(), out["delta"].copy())
    moved[1][2, 5, 7] += 3e-4
    res = bench.cpu_baseline(shape, ep, 3, gpu_outputs={(r0, h0): moved})
    assert res["max_abs_err_vs_gpu"]["o"] == 0.0
    assert abs(res["max_abs_err_vs_gpu"]["delta"] - 3e-4) < 1e-12
    assert bench.cpu_baseline(shape, ep, 3)["max_abs_err_vs_gpu"] is None
