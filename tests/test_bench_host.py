"""Host-side pieces of bench.py that need no GPU."""
import bench


def test_sensor_sampler_never_fails_the_bench():
    # without a GPU driver the SMI library refuses to start: the bench records why
    r = bench.GpuSensors(0, 0.01).start().stop()
    assert isinstance(r, dict) and "readable" in r
    if not r["readable"]:
        assert r["reason"]


def test_sensor_spread_is_min_median_max():
    s = bench.GpuSensors(0, 0.01)
    s.samples = [(1700.0, 80.0, 1200.0), (1800.0, None, 1300.0), (1750.0, 82.0, None)]
    r = s.stop()
    assert r["readable"] and r["samples"] == 3
    assert r["gfx_clock_mhz_min_median_max"] == [1700.0, 1750.0, 1800.0]
    assert r["hotspot_temp_c_min_median_max"] == [80.0, 82.0, 82.0]
    assert r["socket_power_w_min_median_max"] == [1200.0, 1300.0, 1300.0]


def _res(chunk, n_valid=8192, kernels=None, accum="f32"):
    BT, H, V = 8192, 4096, 128256
    chunks = -(-n_valid // chunk)
    return dict(BT=BT, H=H, V=V, n_valid=n_valid, chunks_run=chunks, chunk_size=chunk,
                dx_splits=16, kernels=kernels or {},
                timed_kernel=dict(name="dw_gemm", launches=chunks, ms_per_launch=1.0))


def test_roofline_bound_follows_the_chunk():
    """grad_weight with fp32 dW: MFMA-bound at 2048 rows per chunk (2.15 TFLOP
    against 4.7 GB), HBM-bound at 256 rows (0.27 TFLOP against 4.3 GB)."""
    import bench
    cfg = dict(dtype="bf16", accum="f32")
    big = bench.roofline(_res(2048), cfg)
    assert big["bound"] == "mfma" and big["unit"] == "TFLOP/s"
    assert abs(big["achieved"] - 2 * 2048 * 4096 * 128256 / 1e-3 / 1e12) < 1e-6
    small = bench.roofline(_res(256), cfg)
    assert small["bound"] == "hbm" and small["unit"] == "GB/s"
    f, b = bench.kernel_work("dw_gemm", _res(256), cfg)
    # G and the gathered rows, plus dW written once and read-modified-written 31 times
    want = 256 * 128256 * 2 + 256 * 4096 * 2 + 128256 * 4096 * 4 * (2 * 32 - 1) / 32
    assert f == 2 * 256 * 4096 * 128256 and abs(b - want) < 1
    assert abs(small["achieved"] - b / 1e-3 / 1e9) < 1e-6


def test_kernel_rates_cover_every_timed_kind():
    import bench
    kinds = ["mask_scan", "zero_ignored_rows", "logits_gemm", "softmax_grad", "dx_gemm",
             "dx_reduce", "dw_gemm", "loss_finalize", "gather_rows"]
    k = {n: dict(launches=4, ms_per_launch=0.5, ms_per_step=2.0) for n in kinds}
    rates = bench.kernel_rates(_res(2048, kernels=k), dict(dtype="bf16", accum="f32"))
    assert set(rates) == set(kinds)
    assert rates["mask_scan"]["hbm_gbs"] == (8 * 8192 + 4 * 8192) / 0.5e-3 / 1e9
    assert rates["logits_gemm"]["bound"] == "mfma" and rates["softmax_grad"]["bound"] == "hbm"


def test_extra_summaries():
    import bench
    e = {f"masked_sft_{p}_trained": dict(ms_per_step_unbracketed=40.0 * n / 8192, n_valid=n,
                                         chunks_run=-(-n // 128))
         for p, n in ((100, 8192), (75, 6144), (50, 4096), (10, 819))}
    e["long_seq_8k_c256"] = dict(BT=8192, peak_transient_bytes=1 << 21, workspace_bytes=1000)
    e["long_seq_32k_c256"] = dict(BT=32768, peak_transient_bytes=1 << 21,
                                  workspace_bytes=1000 + 8 * 24576)
    s = bench.extra_summaries(e)
    rows = s["ignored_token_speedup"]["rows"]
    assert [r["labelled_share"] for r in rows] == [0.75, 0.5, 0.1]
    assert abs(rows[1]["speedup"] - 2.0) < 1e-12 and rows[2]["chunk_ratio"] == 64 / 7
    f = s["flat_transient_c256"]
    assert f["workspace_difference_bytes"] == f["row_index_and_loss_bytes"] == 8 * 24576


def test_ceiling_fraction_follows_the_bound():
    ceil = {"mfma_loop_bf16_random_tflops": 1600.0, "mfma_loop_bf16_zero_tflops": 2400.0,
            "mfma16_loop_bf16_random_tflops": 2000.0, "mfma16_loop_bf16_zero_tflops": 2400.0,
            "hbm_read_stream_gbs": 6000.0, "hbm_copy_gbs": 5000.0}
    rl = dict(bound="mfma", achieved=800.0)
    bench.add_ceiling(rl, ceil, "bf16")
    assert rl["frac_of_ceiling"] == 0.5 and rl["ceiling"]["unit"] == "TFLOP/s"
    # grad_input of large chunks runs on 16x16x32 MFMAs: that loop is its ceiling
    for rows, frac in ((bench.DX_SUB16_ROWS, 0.4), (bench.DX_SUB16_ROWS - 1, 0.5)):
        rl = dict(kernel="dx_gemm", bound="mfma", achieved=800.0, rows_per_launch=rows)
        bench.add_ceiling(rl, ceil, "f16")
        assert rl["frac_of_ceiling"] == frac
    # logits and grad_weight on their large tiles (more than 128 rows) run on 16x16x32
    for kern in ("dw_gemm", "logits_gemm"):
        rl = dict(kernel=kern, bound="mfma", achieved=800.0, rows_per_launch=2048)
        bench.add_ceiling(rl, ceil, "bf16", 4096, 128256)
        assert rl["frac_of_ceiling"] == 0.4 and "16x16x32" in rl["ceiling"]["kind"]
        rl = dict(kernel=kern, bound="mfma", achieved=800.0, rows_per_launch=128)
        bench.add_ceiling(rl, ceil, "bf16", 4096, 128256)
        assert rl["frac_of_ceiling"] == 0.5 and "32x32x16" in rl["ceiling"]["kind"]
    rl = dict(kernel="softmax_grad", bound="mfma", achieved=800.0, rows_per_launch=2048)
    bench.add_ceiling(rl, ceil, "bf16")
    assert rl["frac_of_ceiling"] == 0.5
    rl = dict(bound="hbm", achieved=4500.0)
    bench.add_ceiling(rl, ceil, "bf16")
    assert rl["frac_of_ceiling"] == 0.75 and rl["ceiling"]["unit"] == "GB/s"
    # an fp32 contraction has no bf16 loop to compare with; no probes, no fields
    rl = dict(bound="mfma", achieved=100.0)
    bench.add_ceiling(rl, ceil, "f32")
    assert "frac_of_ceiling" not in rl
    bench.add_ceiling(rl, None, "bf16")
    assert "frac_of_ceiling" not in rl
