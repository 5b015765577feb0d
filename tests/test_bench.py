"""Host logic of bench.py (no GPU): the algorithmic bytes and flops each stage
is priced at, the roofline bound chosen from the expert MLP's arithmetic
intensity, and the scaling of hardware counters into HBM bytes.

The expected figures are written out term by term from the shapes of the
operands (the per-expert gate, up and down matrices of the SiLU-gated MLP,
the token rows, the index and weight arrays), independently of the single
expression bench.py evaluates."""
import csv
import json
import os

import pytest

import bench
from combine_router_softmax_top_amd.workloads import CONFIGS


def _mlp_terms(cfg, n_loc):
    """Bytes of the expert MLP as named operands: weights once, x read, h
    written by the gate/up pass and read by the down pass, y written."""
    b = 2 if cfg.dtype == "bf16" else 4
    d, i_ = cfg.hidden, cfg.intermediate
    experts = (cfg.expert_end - cfg.expert_begin) + cfg.num_shared
    rows = n_loc + cfg.num_shared * cfg.num_tokens
    w_gate = w_up = w_down = i_ * d * b
    x_read = rows * d * b
    h_write = h_read = rows * i_ * b
    y_write = rows * d * b
    return experts * (w_gate + w_up + w_down) + x_read + h_write + h_read + y_write


def _mlp_flops(cfg, n_loc):
    """Three GEMMs per row (gate, up: d -> I; down: I -> d), 2 flops per MAC."""
    rows = n_loc + cfg.num_shared * cfg.num_tokens
    return 3 * 2 * rows * cfg.hidden * cfg.intermediate


@pytest.mark.parametrize("name,n_loc", [("dsv3_prefill_ep", 30896), ("mixtral_bf16", 8192),
                                        ("dsv2lite_decode", 768), ("tiny_f32", 128)])
def test_expert_mlp_bytes_and_flops(name, n_loc):
    cfg = CONFIGS[name]
    alg = bench.algorithmic(cfg, n_loc, cfg.num_tokens)
    assert alg["gemm_bytes"] == _mlp_terms(cfg, n_loc)
    assert alg["gemm_flops"] == _mlp_flops(cfg, n_loc)


def test_dsv3_share_figures():
    """The DeepSeek-V3-shaped share with 30 896 local rows: 2.72 TFLOP and
    3.96 GB for the MLP; 1.004 GB for dispatch plus combine when every token
    routes to at least one local expert."""
    cfg = CONFIGS["dsv3_prefill_ep"]
    alg = bench.algorithmic(cfg, 30896, 4096)
    assert alg["gemm_flops"] == 2721331544064
    assert alg["gemm_bytes"] == 3957522432
    row = 7168 * 2
    # dispatch: token rows read once, x_sorted rows written, row -> token map,
    # ids read and positions written per assignment, per-expert counts/offsets.
    assert alg["dispatch"] == 4096 * row + 30896 * row + 30896 * 4 + 4096 * 8 * 4 * 2 + 256 * 4 * 2
    # combine: expert outputs gathered, (weight, position) per assignment, output rows.
    assert alg["combine"] == 30896 * row + 4096 * 8 * 8 + 4096 * row
    assert alg["dispatch"] + alg["combine"] == 1003940544


def test_decode_weights_dominate():
    """64 routed + 2 shared experts of width 1408 at d=2048: 761.3 MB of gate
    and up weights and 380.6 MB of down weights, against 12.6 MB of rows."""
    cfg = CONFIGS["dsv2lite_decode"]
    alg = bench.algorithmic(cfg, 768, 128)
    w = 66 * 3 * 1408 * 2048 * 2
    assert round(66 * 2 * 1408 * 2048 * 2 / 1e6, 1) == 761.3
    assert round(66 * 1408 * 2048 * 2 / 1e6, 1) == 380.6
    assert alg["gemm_bytes"] - w == (768 + 256) * (2 * 2048 + 2 * 1408) * 2


@pytest.mark.parametrize("name,n_loc,bound", [("dsv3_prefill_ep", 30896, "mfma"),
                                              ("mixtral_bf16", 8192, "mfma"),
                                              ("dsv2lite_decode", 768, "hbm"),
                                              ("tiny_f32", 128, "hbm")])
def test_roofline_bound_by_intensity(name, n_loc, bound):
    cfg = CONFIGS[name]
    alg = bench.algorithmic(cfg, n_loc, cfg.num_tokens)
    ms = 1.5
    eg, rf = bench.mlp_roofline(cfg, alg, ms)
    peak = 2500.0 if cfg.dtype == "bf16" else 157.3
    assert eg["ridge_flop_per_byte"] == pytest.approx(peak * 1e12 / 8e12)
    assert rf["bound"] == bound
    if bound == "hbm":
        assert eg["flop_per_byte"] < eg["ridge_flop_per_byte"]
        assert rf["unit"] == "GB/s" and rf["peak"] == 8000.0
        assert rf["achieved"] == pytest.approx(alg["gemm_bytes"] / 1.5e-3 / 1e9)
    else:
        assert eg["flop_per_byte"] >= eg["ridge_flop_per_byte"]
        assert rf["unit"] == "TFLOP/s" and rf["peak"] == peak
        assert rf["achieved"] == pytest.approx(alg["gemm_flops"] / 1.5e-3 / 1e12)
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"])


def test_fp32_above_ridge_reports_alu():
    """An fp32 shape with enough rows per weight crosses the fp32 ridge
    (157.3 TFLOP/s over 8 TB/s) and is priced against the vector ALUs."""
    cfg = CONFIGS["tiny_f32"]
    alg = {"gemm_flops": 1e12, "gemm_bytes": 1e9}
    _, rf = bench.mlp_roofline(cfg, alg, 10.0)
    assert rf["bound"] == "alu" and rf["peak"] == 157.3
    assert rf["achieved"] == pytest.approx(100.0)


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (k, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": "X", "Counter_Value": v})


def test_traffic_record_scaling(tmp_path):
    """Counter values in KiB per dispatch, averaged over dispatches of one
    kernel and scaled so that a 1 GiB device copy reads and writes 1 GiB."""
    g1 = "void gemm_bf16_kernel<1>(GemmArgs)"
    g0 = "void gemm_bf16_kernel<0>(GemmArgs)"
    cp = "__amd_rocclr_copyBuffer"
    d = str(tmp_path)
    _write_csv(os.path.join(d, "pmc_FETCH_SIZE", "h", "run_counter_collection.csv"),
               [(g1, 1000.0), (g1, 3000.0), (g0, 500.0), ("void combine_kernel<8>(A)", 7.0)])
    _write_csv(os.path.join(d, "pmc_WRITE_SIZE", "h", "run_counter_collection.csv"),
               [(g1, 100.0), (g1, 100.0), (g0, 40.0)])
    _write_csv(os.path.join(d, "pmc_copy_FETCH_SIZE", "h", "run_counter_collection.csv"),
               [(cp, float(1 << 19))])  # the copy's reads counted at half: factor 2
    _write_csv(os.path.join(d, "pmc_copy_WRITE_SIZE", "h", "run_counter_collection.csv"),
               [(cp, float(1 << 20))])  # writes counted exactly: factor 1
    out = os.path.join(d, "rec.json")
    rec = bench.write_traffic_record(d, out)
    assert rec["fetch_factor"] == 2.0 and rec["write_factor"] == 1.0
    assert rec["gate_up_bytes"] == (2000.0 * 2 + 100.0) * 1024
    assert rec["down_bytes"] == (500.0 * 2 + 40.0) * 1024
    assert rec["hbm_bytes_per_launch"] == rec["gate_up_bytes"] + rec["down_bytes"]
    assert rec["per_kernel_hbm_mb"]["combine_kernel<8>"] == {"read": 7.0 * 2 * 1024 / 1e6, "write": 0.0}
    assert cp not in rec["per_kernel_hbm_mb"]
    assert json.load(open(out)) == rec
    assert rec["source_digest"] == bench.source_digest()


def test_committed_traffic_record_is_plausible():
    """The committed counter record names its workload and the source digest it
    was counted on (bench.py reports it only while that digest is current),
    and counts at least the algorithmic bytes."""
    rec = json.load(open(bench.TRAFFIC_FILE))
    assert rec["workload"] == "dsv3_prefill_ep"
    assert len(rec["source_digest"]) == len(bench.source_digest())
    assert rec["hbm_bytes_per_launch"] > bench.algorithmic(CONFIGS["dsv3_prefill_ep"], 30896, 4096)["gemm_bytes"]


def test_multi_gpu_refused(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err
