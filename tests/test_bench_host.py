"""bench.py's host-side arithmetic (CPU only): percentiles, the layer
roofline, the algorithmic FLOPs and the rule that a committed traffic figure
is used only while the kernel source it was measured on is unchanged."""
import hashlib

import pytest

import bench
import workloads as W


def test_quantiles_median_and_tails():
    q = bench.quantiles([5.0, 1.0, 3.0, 2.0, 4.0])
    assert q == {"median": 3.0, "p10": 1.0, "p90": 5.0}
    q = bench.quantiles(list(range(101)))
    assert q["median"] == 50 and q["p10"] == 10 and q["p90"] == 90


def test_algorithmic_flops_dsv3():
    cfg = W.CONFIGS["dsv3"]
    fl = bench.algorithmic_flops(cfg, n_kept=cfg.T * cfg.top_k)
    d, N, T = cfg.d_model, cfg.n_experts, cfg.T
    assert fl["router"] == 2.0 * T * d * N
    assert fl["experts"] == 6.0 * d * cfg.d_ff * T * cfg.top_k
    assert fl["shared"] == 6.0 * T * d * cfg.d_ff_shared
    assert fl["total"] == fl["router"] + fl["experts"] + fl["shared"]


def test_layer_roofline_bounds():
    # decode: weight bytes dominate -> HBM-bound; the floor is bytes / 8 TB/s
    cfg = W.CONFIGS["decode"]
    r = bench.layer_roofline(cfg, touched=51, n_kept=512, ms=0.150)
    esz = 2
    nbytes = 4 * cfg.n_experts * cfg.d_model + esz * (3 * cfg.d_model * 51 * cfg.d_ff
                                                      + 2 * cfg.T * cfg.d_model)
    assert r["bound"] == "hbm" and r["algorithmic_bytes"] == nbytes
    assert r["min_ms_at_peaks"] == pytest.approx(nbytes / 8e12 * 1e3, abs=1e-4)
    assert r["frac"] == pytest.approx(r["min_ms_at_peaks"] / 0.150, abs=1e-3)
    # mixtral: ~1024 rows per expert -> MFMA-bound at the bf16 peak
    cfg = W.CONFIGS["mixtral"]
    r = bench.layer_roofline(cfg, touched=8, n_kept=cfg.T * cfg.top_k, ms=2.7)
    assert r["bound"] == "mfma"
    fl = bench.algorithmic_flops(cfg, cfg.T * cfg.top_k)["total"]
    assert r["min_ms_at_peaks"] == pytest.approx(fl / 2.5e15 * 1e3, abs=1e-4)


def test_committed_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    root = tmp_path
    (root / "profiles").mkdir()
    src = root / "sparse_mixture_experts_18_amd" / "csrc"
    src.mkdir(parents=True)
    (src / "grouped_gemm.hip").write_text("// kernel source A\n")
    sha = hashlib.sha256(b"// kernel source A\n").hexdigest()
    (root / "profiles" / "gemm_gate_up_wl_hbm_traffic.md").write_text(
        "# x\n\n- hbm bytes per launch: 1234\n- grouped_gemm.hip sha256: `%s`\n" % sha)
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench.committed_traffic("wl") == 1234
    assert bench.committed_traffic("wl", "down") is None  # no summary for it
    (src / "grouped_gemm.hip").write_text("// kernel source B\n")
    assert bench.committed_traffic("wl") is None  # stale once the source changes


def test_multi_gpu_request_exits(capsys, monkeypatch):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().out
