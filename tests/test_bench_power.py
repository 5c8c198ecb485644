"""The benchmark's power figures (bench.py, PowerSampler.window) from synthetic counter tables:
average power from the energy counter over the device's own time base, the power-limited
fraction from the residency ticks, and only refresh intervals wholly inside the window."""
import bench


def _sampler(tables, energy_j=1e-3):
    s = object.__new__(bench.PowerSampler)  # no amdsmi: only the arithmetic over kept tables
    s.tables, s.energy_j = tables, energy_j
    return s


def _table(host_s, fw_s, energy, ppt, ticks, watts=0, clk=2000.0, clk_min=1900):
    return (host_s, int(fw_s * 1e9), energy, ppt, ticks, watts, clk, clk_min)


def test_window_uses_the_counters_over_whole_intervals():
    # one table a second; 1,000 W (1e6 energy units of 1 mJ a second) and half of the ticks
    # power-limited from t = 2 s on, 300 W and none before
    tables = []
    e = ppt = 0
    for i in range(8):
        tables.append(_table(10.0 + i + 0.003, 500.0 + i, e, ppt, 1000 * i, watts=1000 if i > 2 else 300,
                             clk=1700.0 if i > 2 else 2400.0, clk_min=1650 if i > 2 else 2390))
        w, lim = (1000, 500) if i >= 2 else (300, 0)
        e += w * 1000
        ppt += lim
    s = _sampler(tables)
    r = s.window(12.0, 17.5)  # tables at 12.003 ... 17.003: five whole intervals
    assert r["intervals"] == 5 and r["s"] == 5.0
    assert r["avg_w"] == 1000.0 and r["ppt_limited"] == 0.5
    assert r["reported_w"] == [1000] * 5 and r["gfxclk_mhz"] == 1700.0 and r["gfxclk_min_xcd_mhz"] == 1650.0
    r = s.window(10.5, 13.5)  # tables at 11.003, 12.003, 13.003: 300 W, then 1,000 W
    assert r["intervals"] == 2 and r["avg_w"] == 650.0 and r["ppt_limited"] == 0.25
    assert s.window(12.5, 13.2) == {"intervals": 0}  # one table: no whole interval
