#!/usr/bin/env python3
"""Replay-attention benchmark: fwd+bwd TFLOP/s and % of bf16 matrix-core peak.

One step is one group of the workload replayed in full through the library: G members
one after another, each member's response in reverse blocks of B rows, every block a
forward (split-prefix partials + LSE merge) and a backward (prep, dK/dV pages, dQ parts,
part sum), with the prompt K/V gradient pages accumulated across the whole group.  The
prompt pages are captured once before timing and every member's inputs are resident in
HBM before the timed region starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c2m]

Prints one JSON line.  Counted work per member is 14 * Hq * d * pairs (4 forward + 10
backward multiply-add units over visible (row, key) pairs); masked pairs and the second
recompute of the two-pass backward are not counted.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from suffix_attention_amd import api, configs, datagen, driver  # noqa: E402

METRIC = "replay-attention fwd+bwd TFLOP/s and % bf16 MFMA peak at P=2M, G=8"


def replay_metric(cfg) -> str:
    """The headline metric names the 2M-token, G = 8 workload as configured; any other
    configuration (another config, or c2m with G, B or S overridden) names its own sizes."""
    if cfg == configs.CONFIGS["c2m"]:
        return METRIC
    return f"replay-attention fwd+bwd TFLOP/s and % bf16 MFMA peak at P={cfg.P}, G={cfg.G}, B={cfg.B}, S={cfg.S}"
# --workload fused: the same step with the fused forward + dQ pass (dO known before the forward)
FUSED_METRIC = ("replay-attention fwd+bwd TFLOP/s and % bf16 MFMA peak with the fused forward + dQ pass "
                "(dO known before the forward) at P={P}, G={G}, B={B}, S={S}")
# --workload score: the pre-step scoring pass (forward only, all G members batched)
SCORE_METRIC = "pre-step scoring (forward-only, G members batched) TFLOP/s and % bf16 MFMA peak at P=2M, G=8"
# --workload prefill: capture-side prefill (the prompt's causal attention, chunked, pages written)
PREFILL_METRIC = "capture-side prefill (no-grad causal attention, chunked) TFLOP/s and % bf16 MFMA peak"
# --workload blocksweep: small response blocks, where the replay turns HBM-bound
SWEEP_METRIC = ("replay block-size sweep at P=2M: algorithmic HBM GB/s per replayed block (K/V pools read by the "
                "forward and the backward, fp32 K/V gradient pages read and written)")
# --workload reuse: consecutive optimizer cycles over one capture
REUSE_METRIC = "prefix-reuse fwd+bwd TFLOP/s over consecutive G=8 cycles on one capture at P=4,456,448"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 matrix-core peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)

# Algorithmic matrix work per visible (row, key) pair and query head, in units of 2*d flops
# (one multiply-add GEMM over the head dimension), for each kernel that does it.
KERNEL_UNITS = {"fwd_mfma": 2, "dkdv_mfma": 4, "dq_mfma": 3, "dqs_mfma": 1, "fwd_dq_mfma": 5}

# Measured HBM traffic of the dominant kernel (rocprofv3 FETCH_SIZE / WRITE_SIZE per dispatch,
# scaled by the same counters on a copy of known size), written by --ingest-counters.  It is
# reported only while the kernel sources still hash to the digest it was measured on.
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "suffix_attention_amd", "csrc")
COPY_BYTES = 1 << 30  # --calibrate-copy: bytes read and bytes written per copy launch


def source_digest() -> str:
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.hpp"))
                    + glob.glob(os.path.join(CSRC, "*.cpp"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_file(cfg_name: str) -> str:
    return os.path.join(PROFILES, f"hbm_traffic_{cfg_name}.json")


def measured_traffic(cfg_name: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None if absent or
    taken on other kernel sources."""
    path = traffic_file(cfg_name)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("kernel") != kernel or t.get("source_sha256") != source_digest():
        return None
    return t["hbm_bytes_per_launch"]


def _counter_sums(d: str, counter: str) -> dict:
    """{kernel name: [per-dispatch values]} from a rocprofv3 --pmc csv directory."""
    out = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        per = {}
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Kernel_Name"], r.get("Dispatch_Id", r.get("Correlation_Id", "")))
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        for (name, _), v in per.items():
            out.setdefault(name, []).append(v)
    return out


def ingest_counters(cfg_name: str, kernel: str, fetch_dir: str, write_dir: str, cal_fetch: str, cal_write: str):
    """Turn four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE on the benchmark and on
    --calibrate-copy) into the traffic summary that the benchmark reports."""
    def per_launch(d, counter, match):
        # one library call of the kernel may dispatch several instantiations (the matrix
        # passes launch masked and unmasked parts separately): sum them per call
        sums = {name: vs for name, vs in _counter_sums(d, counter).items() if match(name)}
        assert sums, (d, counter)
        calls = max(len(vs) for vs in sums.values())
        return sum(v for vs in sums.values() for v in vs) / calls, calls

    def biggest(d, counter):
        sums = _counter_sums(d, counter)
        name = max(sums, key=lambda k: max(sums[k]))
        return max(sums[name])

    fetch_kib, n_f = per_launch(fetch_dir, "FETCH_SIZE", lambda n: kernel in n)
    write_kib, n_w = per_launch(write_dir, "WRITE_SIZE", lambda n: kernel in n)
    cal_f = COPY_BYTES / (biggest(cal_fetch, "FETCH_SIZE") * 1024)   # true bytes per counted byte
    cal_w = COPY_BYTES / (biggest(cal_write, "WRITE_SIZE") * 1024)
    out = {"kernel": kernel, "config": cfg_name, "source_sha256": source_digest(),
           "fetch_kib_per_launch": fetch_kib, "write_kib_per_launch": write_kib, "launches": [n_f, n_w],
           "copy_calibration": {"bytes": COPY_BYTES, "fetch_factor": cal_f, "write_factor": cal_w},
           "hbm_bytes_per_launch": fetch_kib * 1024 * cal_f + write_kib * 1024 * cal_w}
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_file(cfg_name), "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def calibrate_copy():
    """A plain device copy of COPY_BYTES (read COPY_BYTES, write COPY_BYTES), three launches."""
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": COPY_BYTES, "launches": 3}))


def log(msg):
    print(msg, file=sys.stderr, flush=True)


MICROBENCH = os.path.join(ROOT, "bench", "libmicrobench.so")


def measured_ceilings() -> dict:
    """The chip's matrix-core and HBM ceilings as the committed microbenchmarks reach them
    (bench/hip/mfma_peak.hip, bench/hip/hbm_bw.hip): best of a few timed launches each."""
    import ctypes as C
    lib = C.CDLL(MICROBENCH)
    lib.mb_mfma_peak.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.POINTER(C.c_double)]
    lib.mb_hbm.argtypes = [C.c_int, C.c_size_t, C.c_int, C.c_int, C.c_int, C.POINTER(C.c_double)]
    out = {}
    v = C.c_double(0)
    # random operands: launches of about 130 ms, as long as the library's own, since the
    # clock keeps falling for tens of milliseconds under that load
    for key, rand, iters in (("mfma_bf16_tflops", 0, 100000), ("mfma_bf16_random_operands_tflops", 1, 400000)):
        best = 0.0
        for blocks in (256, 512):  # one and two waves on every SIMD
            rc = lib.mb_mfma_peak(blocks, iters if blocks == 256 else iters // 2, 3, rand, C.byref(v))
            assert rc == 0, rc
            best = max(best, v.value)
        out[key] = round(best, 1)
    for name, mode, fill in (("hbm_read_gbs", 0, 1), ("hbm_read_zeros_gbs", 0, 0), ("hbm_write_gbs", 1, 1),
                             ("hbm_copy_gbs", 2, 1)):
        best = 0.0
        for blocks in (2048, 8192):
            rc = lib.mb_hbm(mode, 4 << 30, fill, blocks, 5, C.byref(v))
            assert rc == 0, rc
            best = max(best, v.value)
        out[name] = round(best, 1)
    lib.mb_lds.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.POINTER(C.c_double)]
    for name, mode in (("lds_read_b128_tbs", 0), ("lds_read_tr_b64_tbs", 1),
                       ("mfma_lds_fed_1kib_per_mfma_tflops", 2), ("mfma_lds_fed_1kib_per_2mfma_tflops", 3),
                       ("mfma_lds_fed_2tr_per_mfma_tflops", 4)):
        for waves in (4, 8):
            rc = lib.mb_lds(mode, 256, waves, 100000, 3, C.byref(v))
            assert rc == 0, rc
            out[f"{name}_{waves}w"] = round(v.value, 1)
    out["source"] = ("bench/hip/mfma_peak.hip (32x32x16 bf16 chains, every SIMD), bench/hip/hbm_bw.hip (4 GiB), "
                     "bench/hip/lds_bw.hip (one workgroup of 4 or 8 waves per CU)")
    return out


class PowerSampler:
    """GPU 0's power-management counters through amdsmi (read-only queries), polled on a
    background thread.  The device refreshes its metrics table about once a second; every new
    table is kept: the firmware's time base (ns), its energy counter, the count of its
    accumulation ticks and of those ticks in which the package power limit (PPT) held the
    clock down, the socket power it reports and the graphics clock of every XCD at that moment.
    Between two consecutive tables, the energy and tick differences give the average power
    and the fraction of time the chip was power-limited over that interval."""

    def __init__(self, poll_s: float = 0.005):
        import threading

        import amdsmi
        self.smi = amdsmi
        amdsmi.amdsmi_init()
        hs = amdsmi.amdsmi_get_processor_handles()
        self.h = hs[0] if len(hs) == 1 else self._match(hs)
        self.cap_w = amdsmi.amdsmi_get_power_cap_info(self.h)["power_cap"] / 1e6
        self.energy_j = float(amdsmi.amdsmi_get_energy_count(self.h)["counter_resolution"]) * 1e-6
        self.poll = poll_s
        self.tables = []  # (host time, fw ns, energy, ppt ticks, ticks, socket W, mean XCD MHz, min XCD MHz)
        self._stop = threading.Event()
        self._thr = threading.Thread(target=self._run, daemon=True)

    def _match(self, hs):
        bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
        for h in hs:
            if bus is not None and int(self.smi.amdsmi_get_gpu_device_bdf(h).split(":")[1], 16) == bus:
                return h
        raise RuntimeError("no amdsmi device matches cuda:0")

    def _run(self):
        last = None
        while not self._stop.is_set():
            m = self.smi.amdsmi_get_gpu_metrics_info(self.h)
            # a table read while the device rewrites it can come back empty: skip it
            if m["system_clock_counter"] not in (last, 0, "N/A") and m["energy_accumulator"] not in (0, "N/A"):
                last = m["system_clock_counter"]
                clks = [c for c in m["current_gfxclks"] if isinstance(c, int)]
                self.tables.append((time.perf_counter(), m["system_clock_counter"], m["energy_accumulator"],
                                    m["ppt_residency_acc"], m["accumulation_counter"], m["current_socket_power"],
                                    sum(clks) / len(clks), min(clks)))
            time.sleep(self.poll)

    def start(self):
        self._thr.start()
        return self

    def stop(self):
        self._stop.set()
        self._thr.join()
        self.smi.amdsmi_shut_down()

    def window(self, t0: float, t1: float) -> dict:
        """Averages over the refresh intervals that lie wholly inside host times [t0, t1]."""
        tb = [x for x in self.tables if t0 <= x[0] <= t1]
        if len(tb) < 2:
            return {"intervals": 0}
        ns = tb[-1][1] - tb[0][1]
        ticks = tb[-1][4] - tb[0][4]
        return {"intervals": len(tb) - 1, "s": round(ns * 1e-9, 3),
               "avg_w": round((tb[-1][2] - tb[0][2]) * self.energy_j / (ns * 1e-9), 1) if ns > 0 else None,
               "ppt_limited": round((tb[-1][3] - tb[0][3]) / ticks, 3) if ticks > 0 else None,
               "reported_w": [x[5] for x in tb[1:]],
               "gfxclk_mhz": round(float(np.mean([x[6] for x in tb[1:]])), 0),
               "gfxclk_min_xcd_mhz": round(float(np.mean([x[7] for x in tb[1:]])), 0)}


def power_phases(prefix, members, cfg, dump: str | None = None) -> dict:
    """Average power, graphics clock and the fraction of time the package power limit held the
    clock down, while the chip runs, one after another for several seconds each: nothing
    (idle); chains of the matrix instruction on constant and on random operands and an HBM read
    stream (the committed microbenchmarks); whole steps; the forward and the backward of one
    block (the member's last rows, the first replayed), each called repeatedly.  The device's
    counters advance once a second, so each figure covers the whole seconds inside its phase."""
    import ctypes as C
    lib = C.CDLL(MICROBENCH)
    lib.mb_mfma_peak.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.POINTER(C.c_double)]
    lib.mb_mfma_peak_16x16x32.argtypes = [C.c_int, C.c_int, C.c_int, C.POINTER(C.c_double)]
    lib.mb_hbm.argtypes = [C.c_int, C.c_size_t, C.c_int, C.c_int, C.c_int, C.POINTER(C.c_double)]
    v = C.c_double(0)
    smp = PowerSampler().start()
    out = {"source": "amdsmi GPU metrics of the device (read-only), refreshed about once a second",
           "power_cap_w": smp.cap_w, "phases": []}
    min_s = 5.0  # at least four whole refresh intervals per phase

    def phase(name, fn):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        r = {}
        while time.perf_counter() - t0 < min_s:
            r = fn() or {}
            torch.cuda.synchronize()
        row = {"phase": name, **r}
        row.update(smp.window(t0, time.perf_counter()))
        out["phases"].append(row)
        log(f"[bench] power: {row}")
        return row

    def mfma(rand):
        rc = lib.mb_mfma_peak(256, 400000, 8, rand, C.byref(v))
        assert rc == 0, rc
        return {"tflops": round(v.value, 1)}

    def mfma16(blocks):
        rc = lib.mb_mfma_peak_16x16x32(blocks, 400000 * 256 // blocks, 8, C.byref(v))
        assert rc == 0, rc
        return {"tflops": round(v.value, 1)}

    def hbm():
        rc = lib.mb_hbm(0, 4 << 30, 1, 8192, 1000, C.byref(v))
        assert rc == 0, rc
        return {"gbs": round(v.value, 1)}

    phase("idle", lambda: time.sleep(0.5))
    phase("matrix-instruction chains, constant operands", lambda: mfma(0))
    phase("matrix-instruction chains, random operands", lambda: mfma(1))
    # the smaller matrix instruction on the same data, one and two waves per SIMD
    phase("16x16x32 chains, random operands, 1 wave per SIMD", lambda: mfma16(256))
    phase("16x16x32 chains, random operands, 2 waves per SIMD", lambda: mfma16(512))
    phase("HBM read stream", hbm)
    phase("whole steps", lambda: run_steps(prefix, members, cfg, 1) and None)

    # one block, the member's last rows (the first replayed), forward and backward on their own
    dev = prefix.k_pages.device
    m = members[0]
    a, e = max(0, cfg.R - cfg.B), cfg.R
    q, do = m["q"][a:e], m["do"][a:e]
    o, lse, ws_f = api.replay_fwd(prefix, q, a, m["kr"], m["vr"])
    dk_r = torch.zeros(m["kr"].shape, dtype=torch.float32, device=dev)
    dv_r = torch.zeros_like(dk_r)
    dk_p = torch.zeros(prefix.k_pages.shape, dtype=torch.float32, device=dev)
    dv_p = torch.zeros_like(dk_p)
    need = api.bwd_ds_workspace_bytes(prefix, e - a, e)
    store = prefix.dtype == torch.bfloat16 and api.ds_fits(need, dev)
    ws_b = torch.empty(((need if store else api.bwd_workspace_bytes(prefix, e - a)) + 3) // 4,
                       dtype=torch.float32, device=dev)

    def fwd_loop():
        for _ in range(10):
            api.replay_fwd(prefix, q, a, m["kr"], m["vr"], workspace=ws_f, o=o, lse=lse)

    def bwd_loop():
        for _ in range(4):
            api.replay_bwd(prefix, q, a, m["kr"], m["vr"], o, lse, do, dk_r, dv_r, False, dk_p, dv_p,
                           shard_first_touch=[False] * prefix.n_shards, workspace=ws_b)
        return {"dq_form": "stored dS" if store else "recompute"}

    phase(f"forward of rows [{a}, {e})", fwd_loop)
    phase(f"backward of rows [{a}, {e})", bwd_loop)
    smp.stop()
    del ws_b, dk_p, dv_p
    if dump:
        with open(dump, "w") as f:
            json.dump({"tables": smp.tables, "phases": out["phases"]}, f)
    return out


def build_prefix(cfg, dev):
    table = datagen.page_table(cfg.n_pages, datagen.seed(cfg.cfg_id, datagen.TAG_PERM), dev)
    kp, vp = datagen.prefix_kv(cfg, dev)
    k_pages, v_pages = api.capture_pages(kp, vp, table, cfg.n_pages)
    torch.cuda.synchronize()
    return api.Prefix(cfg.hq, cfg.hkv, cfg.d, cfg.dtype, cfg.P, table, k_pages, v_pages,
                      api.even_shard_bounds(cfg.n_pages, cfg.S)), kp, vp


def block_pairs(cfg):
    """Visible pairs per head of every block of one member (reverse order irrelevant)."""
    out = []
    for b in range(cfg.n_blocks):
        a = b * cfg.B
        n = min(cfg.R, a + cfg.B) - a
        out.append(configs.pairs(n, a, cfg.P))
    return out


# Backward: None lets the driver keep dS for the dQ pass when it fits in device memory (or in
# DS_BUDGET bytes), all kv heads at once or in chunks; True / False force either dQ pass.
STORE_DS = None
DS_BUDGET = None


FUSED = False  # --workload fused: every group runs the fused forward + dQ pass


def run_steps(prefix, members, cfg, n, cycle_log=None, store_ds="default"):
    """n optimizer cycles: each a fresh group (gradient pages allocated at its first backward,
    released at its end) replaying every member, every member's peak device memory recorded.
    cycle_log, if given, receives (ms, peak bytes) per cycle (events on the stream; each cycle
    ends with a synchronisation)."""
    last = None
    store_ds = STORE_DS if store_ds == "default" else store_ds
    for _ in range(n):
        last = None  # release the previous group's gradient pages before allocating anew
        if cycle_log is not None:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        grp = driver.GroupReplay(prefix, store_ds=store_ds, ds_budget=DS_BUDGET, track_peak=True, fused=FUSED)
        results = [grp.replay_member(m["q"], m["kr"], m["vr"], m["do"], cfg.B, keep="none") for m in members]
        last = (grp, results)
        if cycle_log is not None:
            e1.record()
            torch.cuda.synchronize()
            cycle_log.append((e0.elapsed_time(e1), grp.peak_bytes))
    return last


def memory_vs_g(prefix, members, cfg, timed_peak: int, timed_form: str) -> dict:
    """Peak device memory of a group at G = 2 and at the config's G, with the backward of the
    timed run and with the recomputing one (untimed runs, each a fresh group after the previous
    one's gradient pages are released; the timed run itself is the timed form's figure at the
    config's G)."""
    out = {}
    for label, store in (("timed_form", STORE_DS), ("recompute", False)):
        row = {}
        for g_ in sorted({2, cfg.G}):
            if label == "timed_form" and g_ == cfg.G:
                peak = timed_peak
            else:
                grp, _ = run_steps(prefix, members[:g_], cfg, 1, store_ds=store)
                peak = grp.peak_bytes
                del grp
            row[f"G={g_}"] = round(peak / 1e9, 3)
        out[label] = row
    out["timed_form"]["form"] = timed_form
    return out


def blas_library() -> str:
    try:
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        return f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:  # noqa: BLE001
        return "unknown"


def cpu_baseline(cfg, kp, vp, member, n_tok=64):
    """The oracle, untuned, on a bounded sample: the last n_tok response rows of member 0
    (all heads) against prompt shard 0 and the response keys those rows see; with the time the
    whole step would take at the sample's rate (extrapolated by counted work)."""
    from oracle import attention as orc  # test infrastructure; used only for this baseline leg

    shard_tokens = min(cfg.P, (cfg.n_pages // cfg.S) * 64)
    q_start = cfg.R - n_tok
    to_np = lambda t: t.to("cpu", torch.float32).numpy()  # noqa: E731
    kps, vps = to_np(kp[:shard_tokens]), to_np(vp[:shard_tokens])
    kr, vr = to_np(member["kr"]), to_np(member["vr"])
    q, do = to_np(member["q"][q_start:]), to_np(member["do"][q_start:])
    t0 = time.perf_counter()
    O, L = orc.forward(q, kps, vps, kr, vr, q_start)
    orc.backward(q, kps, vps, kr, vr, do, q_start, o=O, lse=L, prefix_grad_sink=lambda *a: None)
    dt = time.perf_counter() - t0
    flops = configs.counted_flops(n_tok, q_start, shard_tokens, cfg.hq, cfg.d)
    cores = len(os.sched_getaffinity(0))
    step_flops = cfg.G * configs.member_flops(cfg)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds": round(dt, 3), "blas_threads": int(os.environ.get("OMP_NUM_THREADS", cores)),
            "blas": blas_library(),
            "extrapolated_step_s": round(dt * step_flops / flops, 1),
            "extrapolated": "time of one whole step (every member, every block, all keys) at the sample's rate: "
                            "sample seconds x counted step work / counted sample work",
            "sample": f"float64 numpy oracle fwd+bwd of the last {n_tok} response rows (all {cfg.hq} heads) of "
                      f"member 0 over prompt shard 0 ({shard_tokens} keys) plus their {cfg.R} causal response "
                      f"keys; counted with the same 14*Hq*d*pairs convention"}


def cpu_baseline_score(cfg, kp, vp, member, n_tok=64):
    """The oracle forward, untuned, on a bounded sample: the last n_tok response rows of member 0
    (all heads) against prompt shard 0 and the response keys those rows see."""
    from oracle import attention as orc  # test infrastructure; used only for this baseline leg

    shard_tokens = min(cfg.P, (cfg.n_pages // cfg.S) * 64)
    q_start = cfg.R - n_tok
    to_np = lambda t: t.to("cpu", torch.float32).numpy()  # noqa: E731
    kps, vps = to_np(kp[:shard_tokens]), to_np(vp[:shard_tokens])
    kr, vr = to_np(member["kr"]), to_np(member["vr"])
    q = to_np(member["q"][q_start:])
    t0 = time.perf_counter()
    orc.forward(q, kps, vps, kr, vr, q_start)
    dt = time.perf_counter() - t0
    flops = 4 * cfg.hq * cfg.d * configs.pairs(n_tok, q_start, shard_tokens)
    cores = len(os.sched_getaffinity(0))
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds": round(dt, 3), "blas_threads": int(os.environ.get("OMP_NUM_THREADS", cores)),
            "sample": f"float64 numpy oracle forward of the last {n_tok} response rows (all {cfg.hq} heads) of "
                      f"member 0 over prompt shard 0 ({shard_tokens} keys) plus their {cfg.R} causal response "
                      f"keys; counted as 4*Hq*d*pairs"}


def bench_blocksweep(ns, cfg, dev, prefix, members):
    """Small response blocks.  Per block the replay reads the K/V pools twice (forward and
    backward, 2 x 4 bytes per key, kv head and element) and reads and writes the fp32 K/V
    gradient pages (16 bytes), 24 bytes in all, while its matrix work shrinks with the block:
    below about 90 rows a block is bound by HBM.  Member 0 is replayed in full at each block
    size of --sweep-B (one untimed replay first, then --steps timed ones, each a fresh group);
    the rate is those algorithmic bytes over the measured time (the first block of a group
    only writes the gradient pages, so the figure slightly overstates the bytes)."""
    sizes = [int(x) for x in ns.sweep_B.split(",")]
    m = members[0]
    alg_block = 24 * cfg.P * cfg.hkv * cfg.d
    rows = []
    for b in sizes:
        c = cfg.with_(B=b, G=1)
        run_steps(prefix, [m], c, 1)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        api.profile_begin()
        ev0.record()
        run_steps(prefix, [m], c, ns.steps)
        ev1.record()
        torch.cuda.synchronize()
        kstats = api.profile_end()
        ms = ev0.elapsed_time(ev1)
        n_blocks = ns.steps * c.n_blocks
        gbs = alg_block * n_blocks / (ms / 1e3) / 1e9
        tflops = configs.member_flops(c) * ns.steps / (ms / 1e3) / 1e12
        row = {"B": b, "blocks": c.n_blocks, "ms_per_block": round(ms / n_blocks, 3),
               "alg_gb_per_block": round(alg_block / 1e9, 2), "alg_gbs": round(gbs, 1),
               "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2), "counted_tflops": round(tflops, 1),
               "kernels_ms_per_block": {k: round(v[1] / n_blocks, 3) for k, v in sorted(kstats.items())}}
        log(f"[bench] B={b}: {row}")
        rows.append(row)
    first = rows[0]
    out = {"metric": SWEEP_METRIC, "value": first["alg_gbs"], "unit": "GB/s", "n_gpus": 1, "steps": ns.steps,
           "warmup": 1, "ms_per_step": first["ms_per_block"] * first["blocks"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"{cfg.name}: member 0 replayed in blocks of {ns.sweep_B} rows, P={cfg.P} prompt "
                                  f"tokens in 64-token pages, S={cfg.S} shards, R={cfg.R}, Hq={cfg.hq}, Hkv={cfg.hkv}, "
                                  f"d={cfg.d}, N(0,1) inputs; value is the smallest block size",
                      "P": cfg.P, "R": cfg.R, "S": cfg.S, "hq": cfg.hq, "hkv": cfg.hkv, "d": cfg.d},
           "roofline": {"bound": "hbm", "kernel": "whole block", "achieved": first["alg_gbs"], "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(first["alg_gbs"] / PEAK_HBM_GBS, 4), "traffic": None,
                        "bytes_per_unit": "24 B per (prompt key, kv head, element) per block"},
           "sweep": rows}
    print(json.dumps(out), flush=True)


def bench_score(ns, cfg, dev, prefix, kp, vp, members):
    """Pre-step scoring: every member's whole response, forward only, in one batched call per
    step (ls_score_fwd)."""
    q = torch.stack([m["q"] for m in members])
    kr = torch.stack([m["kr"] for m in members])
    vr = torch.stack([m["vr"] for m in members])
    o, lse, ws = api.score_fwd(prefix, q, kr, vr)  # allocates outputs and workspace once
    for _ in range(ns.warmup):
        api.score_fwd(prefix, q, kr, vr, workspace=ws, o=o, lse=lse)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    api.profile_begin()
    ev0.record()
    for _ in range(ns.steps):
        api.score_fwd(prefix, q, kr, vr, workspace=ws, o=o, lse=lse)
    ev1.record()
    torch.cuda.synchronize()
    kstats = api.profile_end()
    ms = ev0.elapsed_time(ev1)
    pairs = configs.pairs(cfg.R, 0, cfg.P)
    flops_step = cfg.G * 4 * cfg.hq * cfg.d * pairs
    tflops = flops_step * ns.steps / (ms / 1e3) / 1e12
    kern = {k: {"launches": v[0], "total_ms": round(v[1], 3), "mean_ms": round(v[1] / max(1, v[0]), 4)}
            for k, v in kstats.items()}
    achieved = ns.steps * flops_step / (kern["fwd_mfma"]["total_ms"] / 1e3) / 1e12
    out = {
        "metric": SCORE_METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": ns.steps,
        "warmup": ns.warmup,
        "ms_per_step": round(ms / ns.steps, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} scoring: one attention layer, P={cfg.P} prompt tokens in 64-token pages "
                               f"with a seeded permuted page table, S={cfg.S} shards, G={cfg.G} members x R={cfg.R} "
                               f"response rows scored forward-only in one batched call, Hq={cfg.hq}, "
                               f"Hkv={cfg.hkv}, d={cfg.d}, N(0,1) inputs",
                   "P": cfg.P, "R": cfg.R, "G": cfg.G, "S": cfg.S, "hq": cfg.hq, "hkv": cfg.hkv, "d": cfg.d},
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "counted_tflop_per_step": round(flops_step / 1e12, 3),
        "roofline": {"bound": "mfma", "kernel": "fwd_mfma", "achieved": round(achieved, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "flops_per_unit": "4*d per visible (row, key) pair and query head",
                     "mean_launch_ms": kern["fwd_mfma"]["mean_ms"]},
        "kernels": kern,
        "peak_mem_gb": round(torch.cuda.max_memory_allocated(dev) / 1e9, 3),
    }
    if not ns.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_score(cfg, kp, vp, members[0])
    print(json.dumps(out), flush=True)


def bench_prefill(ns, cfg, dev):
    """Capture-side prefill of a P-token prompt in chunks (driver.prefill_capture): counted as
    4*Hq*d per causal (row, key) pair."""
    P, chunk = ns.prefill_tokens, ns.prefill_chunk
    q = datagen.normal((P, cfg.hq, cfg.d), datagen.seed(cfg.cfg_id, 900), cfg.dtype, dev)
    k = datagen.normal((P, cfg.hkv, cfg.d), datagen.seed(cfg.cfg_id, 901), cfg.dtype, dev)
    v = datagen.normal((P, cfg.hkv, cfg.d), datagen.seed(cfg.cfg_id, 902), cfg.dtype, dev)
    n_pages = api.n_logical_pages(P)
    table = datagen.page_table(n_pages, datagen.seed(cfg.cfg_id, 903), dev)
    for _ in range(ns.warmup):
        driver.prefill_capture(q, k, v, table, n_pages, chunk, n_shards=cfg.S, keep_o=False)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    api.profile_begin()
    ev0.record()
    for _ in range(ns.steps):
        pre, _, _ = driver.prefill_capture(q, k, v, table, n_pages, chunk, n_shards=cfg.S, keep_o=False)
    ev1.record()
    torch.cuda.synchronize()
    kstats = api.profile_end()
    ms = ev0.elapsed_time(ev1)
    flops_step = 4 * cfg.hq * cfg.d * configs.pairs(P, 0, 0)
    tflops = flops_step * ns.steps / (ms / 1e3) / 1e12
    kern = {k_: {"launches": v_[0], "total_ms": round(v_[1], 3), "mean_ms": round(v_[1] / max(1, v_[0]), 4)}
            for k_, v_ in kstats.items()}
    achieved = ns.steps * flops_step / (kern["fwd_mfma"]["total_ms"] / 1e3) / 1e12
    out = {"metric": PREFILL_METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": ns.steps,
           "warmup": ns.warmup, "ms_per_step": round(ms / ns.steps, 2), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16" if cfg.dtype == torch.bfloat16 else "f32", "data": "synthetic",
           "config": {"workload": f"prefill: P={P} prompt tokens of one attention layer in chunks of {chunk}, each "
                                  f"attending to the pages captured so far ({cfg.S} shards) plus itself causally, "
                                  f"then captured; Hq={cfg.hq}, Hkv={cfg.hkv}, d={cfg.d}, N(0,1) inputs",
                      "P": P, "chunk": chunk, "S": cfg.S, "hq": cfg.hq, "hkv": cfg.hkv, "d": cfg.d},
           "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
           "counted_tflop_per_step": round(flops_step / 1e12, 3),
           "roofline": {"bound": "mfma", "kernel": "fwd_mfma", "achieved": round(achieved, 1),
                        "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                        "traffic": None, "flops_per_unit": "4*d per visible (row, key) pair and query head",
                        "mean_launch_ms": kern["fwd_mfma"]["mean_ms"]},
           "kernels": kern}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="c2m", choices=sorted(configs.CONFIGS))
    ap.add_argument("--G", type=int, default=None, help="override the group size")
    ap.add_argument("--B", type=int, default=None, help="override the response block size")
    ap.add_argument("--S", type=int, default=None, help="override the number of prompt shards")
    ap.add_argument("--sweep-B", default="16,64,256", help="block sizes of --workload blocksweep")
    ap.add_argument("--workload", default="replay", choices=["replay", "score", "prefill", "reuse", "blocksweep",
                                                             "fused"],
                    help="replay: the fwd+bwd step (the headline); score: batched forward-only scoring; "
                         "prefill: chunked capture-side prefill; reuse: consecutive G=8 cycles on one capture "
                         "at P=4,456,448 (--steps cycles, per-cycle times and peaks); blocksweep: member 0 at "
                         "the block sizes of --sweep-B, algorithmic HBM GB/s; fused: the replay step with the "
                         "fused forward + dQ pass (dO known before the forward) and a backward without dQ")
    ap.add_argument("--prefill-tokens", type=int, default=524288)
    ap.add_argument("--prefill-chunk", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--store-ds", default="auto", choices=["auto", "on", "off"],
                    help="dQ from the dS stored by the dK/dV pass (auto: when it fits in device memory or in "
                         "--ds-budget-gb, all kv heads at once or in chunks)")
    ap.add_argument("--ds-budget-gb", type=float, default=None,
                    help="device-memory budget for the backward workspace (auto picks the largest dS chunking "
                         "that fits)")
    ap.add_argument("--no-memory-sweep", action="store_true",
                    help="skip the untimed G=2 / recompute runs that report peak memory versus G")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the matrix-core and HBM microbenchmarks")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a device copy of known size (for HBM counter calibration)")
    ap.add_argument("--ingest-counters", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR"),
                    help="write the dominant kernel's HBM traffic summary from rocprofv3 --pmc output")
    ap.add_argument("--kernel", default="dkdv_mfma", help="kernel for --ingest-counters")
    ap.add_argument("--no-power", action="store_true",
                    help="skip the power phases run after the timed steps (average power, clock and power-limit "
                         "residency from the device's counters, read through amdsmi, for idle, the microbenchmarks, "
                         "a step and one block's forward and backward)")
    ap.add_argument("--power-dump", default=None, help="write the power phases' raw counter tables to this JSON file")
    ns = ap.parse_args()
    if ns.ingest_counters:
        ingest_counters(ns.config, ns.kernel, *ns.ingest_counters)
        return
    if ns.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (--gpus {ns.gpus} requested)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if ns.calibrate_copy:
        calibrate_copy()
        return
    if ns.workload == "reuse" and ns.config == "c2m":
        ns.config = "reuse4m"
    cfg = configs.CONFIGS[ns.config]
    if ns.G:
        cfg = cfg.with_(G=ns.G)
    if ns.B:
        cfg = cfg.with_(B=ns.B)
    if ns.S:
        cfg = cfg.with_(S=ns.S)
    global STORE_DS, DS_BUDGET, FUSED
    STORE_DS = {"auto": None, "on": True, "off": False}[ns.store_ds]
    FUSED = ns.workload == "fused"
    DS_BUDGET = None if ns.ds_budget_gb is None else int(ns.ds_budget_gb * 1e9)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    log(f"[bench] config {cfg}")
    if ns.workload == "prefill":
        bench_prefill(ns, cfg, dev)
        return
    prefix, kp, vp = build_prefix(cfg, dev)
    members = [datagen.member_inputs(cfg, i, dev) for i in range(cfg.G)]
    torch.cuda.synchronize()
    log(f"[bench] prefix captured ({cfg.n_pages} pages), {cfg.G} members resident")
    if ns.workload == "score":
        bench_score(ns, cfg, dev, prefix, kp, vp, members)
        return
    if ns.workload == "blocksweep":
        bench_blocksweep(ns, cfg, dev, prefix, members)
        return

    ceilings = None
    if not ns.no_ceilings:
        ceilings = measured_ceilings()
        log(f"[bench] measured ceilings {ceilings}")

    if ns.warmup > 0:
        t = time.perf_counter()
        run_steps(prefix, members, cfg, ns.warmup)
        torch.cuda.synchronize()
        log(f"[bench] warmup {ns.warmup} step(s) {time.perf_counter() - t:.1f} s")

    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    api.profile_begin()
    t0 = time.perf_counter()
    ev0.record()
    cycles = [] if ns.workload == "reuse" else None
    grp, results = run_steps(prefix, members, cfg, ns.steps, cycle_log=cycles)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kstats = api.profile_end()
    ms = ev0.elapsed_time(ev1)
    log(f"[bench] timed {ns.steps} step(s): {ms / 1e3:.2f} s (wall {wall:.2f} s)")

    flops_step = cfg.G * configs.member_flops(cfg)
    tflops = flops_step * ns.steps / (ms / 1e3) / 1e12

    # roofline of the dominant kernel: algorithmic flops per launch / its mean launch time
    pairs = block_pairs(cfg)
    blocks_timed = ns.steps * cfg.G * cfg.n_blocks
    kern = {k: {"launches": v[0], "total_ms": round(v[1], 3), "mean_ms": round(v[1] / max(1, v[0]), 4)}
            for k, v in kstats.items()}
    dom = max((k for k in kern if k in KERNEL_UNITS), key=lambda k: kern[k]["total_ms"])
    alg_flops_total = ns.steps * cfg.G * sum(2 * KERNEL_UNITS[dom] * cfg.hq * cfg.d * p for p in pairs)
    n_launch = kern[dom]["launches"]
    # one launch per block, or one per chunk when a block's dS is stored a chunk at a time
    achieved = alg_flops_total / (kern[dom]["total_ms"] / 1e3) / 1e12
    for k in kern:
        if k in KERNEL_UNITS:
            f = ns.steps * cfg.G * sum(2 * KERNEL_UNITS[k] * cfg.hq * cfg.d * p for p in pairs)
            kern[k]["tflops"] = round(f / (kern[k]["total_ms"] / 1e3) / 1e12, 1)

    peaks = [r.peak_bytes for r in results]
    plan = grp.plan
    out = {
        "metric": replay_metric(cfg),
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": ns.steps,
        "warmup": ns.warmup,
        "ms_per_step": round(ms / ns.steps, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: one attention layer, P={cfg.P} prompt tokens in 64-token pages with "
                               f"a seeded permuted page table, S={cfg.S} shards, G={cfg.G} members x R={cfg.R} "
                               f"response rows in reverse blocks of {cfg.B}, Hq={cfg.hq}, Hkv={cfg.hkv}, d={cfg.d}, "
                               f"N(0,1) inputs",
                   "P": cfg.P, "R": cfg.R, "B": cfg.B, "G": cfg.G, "S": cfg.S, "hq": cfg.hq, "hkv": cfg.hkv,
                   "d": cfg.d},
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "counted_tflop_per_step": round(flops_step / 1e12, 3),
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(cfg.name, dom),
                     "flops_per_unit": f"{2 * KERNEL_UNITS[dom]}*d per visible (row, key) pair and query head",
                     "mean_launch_ms": kern[dom]["mean_ms"], "launches_per_block": round(n_launch / blocks_timed, 3)},
        "kernels": kern,
        "backward": {"form": plan.describe(prefix), "ds_heads": plan.heads, "ds_parts": plan.parts,
                     "workspace_gb": round(results[0].ws_bytes / 1e9, 3),
                     "ds_budget_gb": ns.ds_budget_gb},
        "peak_mem_gb_per_member": [round(p / 1e9, 3) for p in peaks],
        "peak_mem_gb": round(max(peaks) / 1e9, 3),
    }
    if ceilings is not None:
        out["measured_ceilings"] = ceilings
        out["pct_measured_mfma_peak"] = round(100 * tflops / ceilings["mfma_bf16_tflops"], 2)
        out["roofline"]["measured_peak"] = ceilings["mfma_bf16_tflops"]
        out["roofline"]["frac_measured_peak"] = round(achieved / ceilings["mfma_bf16_tflops"], 4)
        # the same chains on random operands: the ceiling the chip holds on N(0, 1)-like data
        rnd = ceilings["mfma_bf16_random_operands_tflops"]
        out["pct_random_operand_mfma_ceiling"] = round(100 * tflops / rnd, 2)
        out["roofline"]["random_operand_peak"] = rnd
        out["roofline"]["frac_random_operand_peak"] = round(achieved / rnd, 4)
    if FUSED:
        out["metric"] = FUSED_METRIC.format(P=cfg.P, G=cfg.G, B=cfg.B, S=cfg.S)
        out["backward"]["form"] = "fused forward + dQ pass, then the recomputing dK/dV pass without dQ"
    if cycles is not None:
        out["metric"] = REUSE_METRIC
        out["config"]["workload"] = (f"{cfg.name}: {ns.steps} consecutive optimizer cycles over one capture; "
                                     + out["config"]["workload"].split(": ", 1)[1])
        out["cycle_ms"] = [round(c[0], 1) for c in cycles]
        out["cycle_peak_gb"] = [round(c[1] / 1e9, 3) for c in cycles]
    timed_peak, timed_form = grp.peak_bytes, plan.describe(prefix)
    del grp, results  # release the timed group's gradient pages before anything else runs
    if not ns.no_power and cycles is None and not FUSED:
        t = time.perf_counter()
        try:
            out["power"] = power_phases(prefix, members, cfg, ns.power_dump)
        except Exception as exc:  # amdsmi missing or refused: the figures are context, not the metric
            out["power"] = {"error": f"{type(exc).__name__}: {exc}"}
        torch.cuda.synchronize()
        log(f"[bench] power phases {time.perf_counter() - t:.1f} s")
    if not ns.no_memory_sweep and cycles is None and not FUSED:
        t = time.perf_counter()
        out["peak_mem_gb_vs_G"] = memory_vs_g(prefix, members, cfg, timed_peak, timed_form)
        torch.cuda.synchronize()
        log(f"[bench] memory sweep {time.perf_counter() - t:.1f} s: {out['peak_mem_gb_vs_G']}")
    if not ns.no_cpu_baseline:
        t = time.perf_counter()
        out["cpu_baseline"] = cpu_baseline(cfg, kp, vp, members[0])
        log(f"[bench] cpu baseline {time.perf_counter() - t:.1f} s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
