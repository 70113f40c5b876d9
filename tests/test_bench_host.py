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
