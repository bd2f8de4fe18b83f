#!/usr/bin/env python3
"""Benchmark of the fused Q4_K SwiGLU MLP on one MI355X.

Headline: one 4096 -> 11008 -> 4096 Q4_K SwiGLU MLP layer on a 256-token
prefill tile (seed 1), timed over K repeats after W warmup calls, inputs
already resident in HBM.  A step is one call of zinc_mlp_q4k_prefill: the
fused kernel (per-chunk fp16 partial outputs at y's scale) and the reduce
kernel that sums them in fp32 into fp16 y.

Printed as ONE JSON line: tokens/s, the fused kernel's MFMA roofline fraction
(its duration measured with HIP events recorded on its own stream by the
library's timing hook), the HBM traffic from the committed rocprofv3 counter
summary when it matches the current kernel source, and the CPU oracle timed
on the host.  Secondary lines (decode M=1/M=4 over 32 independent layers,
the 64-expert MoE over two rotated expert sets, the router, the MLP block
with its RMS norm and residual, the 2048-token prefill over 32 layers) ride in
"secondary".  ``--only staged`` instead times the fused prefill against its
staged baseline (the intermediate in device memory) at M=256 and M=2048.

Also in the line: the measured peaks of this chip (an MFMA-only loop, HBM
stream read and copy; libzinc_peaks.so), the graphics clock and socket power
sampled through amdsmi right after the headline's timed calls, and the headline
fraction against the spec peak, the measured peak and the spec peak at the
observed clock.

usage: python bench.py [--gpus 1] [--steps 200] [--warmup 300] [--no-secondary] [--no-cpu-baseline] [--no-peaks]
                      [--no-extras]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Q4_K SwiGLU-MLP tokens/s at 4096/11008 M=256; % of MFMA/HBM roofline"
PEAK_F16_TFLOPS = 2500.0      # MI355X dense fp16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_fused_m256_traffic.json")
KERNEL_SOURCES = ("q4_swiglu_mlp_amd/csrc/fused16.hpp", "q4_swiglu_mlp_amd/csrc/fused_core.hpp",
                  "q4_swiglu_mlp_amd/csrc/q4k_device.hpp", "q4_swiglu_mlp_amd/csrc/k_prefill.hip")


_CODE_TOKENS = re.compile(r'("(?:\\.|[^"\\])*")|//[^\n]*|/\*.*?\*/', re.S)


def kernel_source_hash() -> str:
    """Hash of the prefill kernel's sources with comments removed and
    whitespace collapsed: the stored traffic counters stay valid across
    comment edits and become stale on any change to the code."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = _CODE_TOKENS.sub(lambda m: m.group(1) or " ", f.read())
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def q4k_bytes(rows: int, cols: int) -> int:
    return rows * (cols // 256) * 144


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def time_calls(fn, steps: int, warmup: int, torch, warm_s: float = 0.0):
    """Warmup (`warmup` calls, and for the secondary workloads at least `warm_s`
    seconds of calls, so the clock has settled after the host work that sets
    each workload up), then time exactly `steps` calls bracketed by
    synchronize; returns (wall seconds, per-call main-kernel durations in ms
    from the timing hook)."""
    import q4_swiglu_mlp_amd as Z
    t0, i = time.perf_counter(), 0
    while i < warmup or time.perf_counter() - t0 < warm_s:
        fn(i)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    Z.timing_enable(4 * steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = Z.timing_collect(4 * steps)
    Z.timing_disable()
    return t1 - t0, ms


PEAKS_LIB = os.path.join(ROOT, "q4_swiglu_mlp_amd", "_lib", "libzinc_peaks.so")
SPEC_GFX_MHZ = 2400.0         # the clock the 2.5 PFLOP/s dense fp16 figure is quoted at


def measure_peaks(torch):
    """What the chip delivers in practice: an MFMA-only loop (16x16x32 and
    32x32x16 fp16, fp32 accumulate) and streaming HBM reads and copies of
    buffers far larger than the 256 MB last-level cache, timed with HIP events
    on the stream the kernels run on (libzinc_peaks.so)."""
    import ctypes
    lib = ctypes.CDLL(PEAKS_LIB)
    lib.zinc_peak_mfma_f16.restype = ctypes.c_double
    lib.zinc_peak_mfma_f16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.zinc_peak_hbm_read.restype = ctypes.c_int
    lib.zinc_peak_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p]
    lib.zinc_peak_hbm_copy.restype = ctypes.c_int
    lib.zinc_peak_hbm_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                       ctypes.c_void_p]
    dev = torch.device("cuda:0")
    cur = torch.cuda.current_stream()
    sh = cur.cuda_stream
    ncu = torch.cuda.get_device_properties(0).multi_processor_count

    def timed(fn, reps, warm_s=0.3):
        # run the kernel back to back for warm_s first: the clocks ramp up
        # under load and a cold first launch would read low
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < warm_s:
            fn()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        best = float("inf")
        for _ in range(reps):
            e0.record(cur)
            fn()
            e1.record(cur)
            e1.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e-3)
        return best

    out = {}
    # one 12-wave workgroup per CU (three waves per SIMD), each wave with eight
    # independent accumulators
    blocks = ncu
    res = torch.empty(blocks * 768, dtype=torch.float32, device=dev)
    for shape in (16, 32):
        flops = [0.0]

        def run(iters, shape=shape):
            flops[0] = lib.zinc_peak_mfma_f16(shape, blocks, iters, res.data_ptr(), sh)
        # burst: launches of about 1 ms, as the MLP kernels run (warm-up of a
        # few launches only); sustained: after 0.3 s of back-to-back launches,
        # when the clock has settled under the load
        t = timed(lambda: run(2048), 5, warm_s=0.005)
        out[f"mfma_f16_{shape}x{shape}_tflops_burst"] = round(flops[0] / t / 1e12, 1)
        t = timed(lambda: run(2048), 5, warm_s=0.3)
        out[f"mfma_f16_{shape}x{shape}_tflops_sustained"] = round(flops[0] / t / 1e12, 1)
        if shape == 16:
            out["clock_during_mfma_loop"] = sample_clock(torch, lambda _i: run(2048),
                                                         "the 16x16x32 MFMA-only loop for 2 s, the last 0.8 s")
            # the clock the sustained rate implies: one 16x16x32 MFMA (16384
            # flops) per 16 cycles on each of the four SIMDs of every CU
            out["clock_implied_by_mfma_rate_mhz"] = round(
                out["mfma_f16_16x16_tflops_sustained"] * 1e12 / (ncu * 4 * 1024) / 1e6, 1)
    nbytes = 4 << 30
    src = torch.empty(nbytes // 4, dtype=torch.int32, device=dev).fill_(7)
    dst = torch.empty(nbytes // 8, dtype=torch.int32, device=dev)
    rres = torch.empty(ncu * 16 * 256, dtype=torch.int32, device=dev)
    t = timed(lambda: lib.zinc_peak_hbm_read(src.data_ptr(), nbytes, ncu * 16, rres.data_ptr(), sh), 5)
    out["hbm_read_GBs"] = round(nbytes / t / 1e9, 1)
    half = nbytes // 2
    t = timed(lambda: lib.zinc_peak_hbm_copy(src.data_ptr(), dst.data_ptr(), half, ncu * 16, sh), 5)
    out["hbm_copy_GBs_read_plus_write"] = round(2 * half / t / 1e9, 1)
    del src, dst, rres, res
    torch.cuda.empty_cache()
    out["method"] = ("best of 5 launches each, HIP events on the launch stream; MFMA: 12 waves per CU, 8 "
                     "independent accumulators per wave, launches of about 1 ms, timed after a few launches (burst) "
                     "and after 0.3 s of back-to-back launches (sustained); HBM: 4 GiB read and 2 GiB copied with "
                     "16-byte loads, after 0.3 s of the same launches")
    return out


def measure_issue_probes(torch):
    """Two probes of what a SIMD can issue (libzinc_peaks.so), timed like the
    peaks: (1) 16x16x32 MFMAs with kv independent packed-fp16 FMAs per MFMA,
    issued by the same wave or by a second wave on the SIMD; (2) the fused
    prefill unit's phase-1 loop (Q4_K decode in registers, B operands from
    LDS, gate and up MFMAs) on L2-resident weights, whole and with parts
    removed.  Times are per MFMA and SIMD, and as a fraction of the MFMA-only
    rate of probe (1) at kv = 0."""
    import ctypes
    lib = ctypes.CDLL(PEAKS_LIB)
    lib.zinc_peak_mfma_valu.restype = ctypes.c_double
    lib.zinc_peak_mfma_valu.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p, ctypes.c_void_p]
    lib.zinc_peak_mfma32_valu.restype = ctypes.c_double
    lib.zinc_peak_mfma32_valu.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p, ctypes.c_void_p]
    lib.zinc_peak_decode_loop.restype = ctypes.c_double
    lib.zinc_peak_decode_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    import numpy as np
    import q4k_synth as S
    dev = torch.device("cuda:0")
    cur = torch.cuda.current_stream()
    sh = cur.cuda_stream
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(ncu * 768, dtype=torch.float32, device=dev)

    def per_mfma_ns(fn, reps=5):
        n = [0.0]

        def run():
            n[0] = fn()
            if n[0] <= 0:
                raise RuntimeError("probe launch failed")
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.2:
            run()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        best = float("inf")
        for _ in range(reps):
            e0.record(cur)
            run()
            e1.record(cur)
            e1.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e6)
        return best / n[0]

    res = {"mfma_with_valu": {}, "phase1_loop": {}}
    base = None
    for same in (1, 0):
        for kv in range(5):
            ns = per_mfma_ns(lambda same=same, kv=kv: lib.zinc_peak_mfma_valu(same, kv, ncu, 4096, out.data_ptr(), sh))
            base = ns if (same, kv) == (1, 0) else base
            res["mfma_with_valu"][f"{'same_wave' if same else 'second_wave'}_kv{kv}"] = {
                "ns_per_mfma": round(ns, 3), "mfma_rate_frac": round(base / ns, 3)}
    lib.zinc_peak_mfma_valu_agpr.restype = ctypes.c_double
    lib.zinc_peak_mfma_valu_agpr.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p, ctypes.c_void_p]
    res["mfma_with_valu_agpr_acc"] = {}
    for kv in range(5):
        ns = per_mfma_ns(lambda kv=kv: lib.zinc_peak_mfma_valu_agpr(kv, ncu, 4096, out.data_ptr(), sh))
        res["mfma_with_valu_agpr_acc"][f"same_wave_kv{kv}"] = {"ns_per_mfma": round(ns, 3),
                                                             "mfma_rate_frac": round(base / ns, 3)}
    res["mfma32_with_valu"] = {}
    base32 = None
    for kv in (0, 1, 2, 3, 4, 6, 8, 12):
        ns = per_mfma_ns(lambda kv=kv: lib.zinc_peak_mfma32_valu(kv, ncu, 4096, out.data_ptr(), sh))
        base32 = ns if kv == 0 else base32
        res["mfma32_with_valu"][f"same_wave_kv{kv}"] = {"ns_per_mfma": round(ns, 3),
                                                        "time_vs_mfma_only": round(ns / base32, 3)}
    rng = np.random.default_rng(11)
    nblk = 16
    wg = torch.from_numpy(S.gen_q4k_blob(rng, 192, nblk * 256)).to(dev)
    wu = torch.from_numpy(S.gen_q4k_blob(rng, 192, nblk * 256)).to(dev)
    names = {0: "whole", 2: "no_decode", 4: "no_weight_loads", 5: "no_loads_b_in_registers"}
    for ng in (4, 8):
        for var in (0, 2, 4, 5):
            ns = per_mfma_ns(lambda ng=ng, var=var: lib.zinc_peak_decode_loop(
                ng, var, wg.data_ptr(), wu.data_ptr(), nblk, 64, ncu, out.data_ptr(), sh))
            res["phase1_loop"][f"{16 * ng}_tokens_{names[var]}"] = {"ns_per_mfma": round(ns, 3),
                                                                   "mfma_rate_frac": round(base / ns, 3)}
    lib.zinc_peak_decode_loop32.restype = ctypes.c_double
    lib.zinc_peak_decode_loop32.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    res["phase1_loop_32x32x16"] = {}
    for var in (0, 2, 4, 5):
        ns = per_mfma_ns(lambda var=var: lib.zinc_peak_decode_loop32(
            var, wg.data_ptr(), wu.data_ptr(), nblk, 64, ncu, out.data_ptr(), sh))
        res["phase1_loop_32x32x16"][f"64_tokens_{names[var]}"] = {"ns_per_16x16x32_equivalent": round(ns, 3),
                                                                  "mfma_rate_frac": round(base / ns, 3)}
    res["method"] = ("one workgroup per CU (8 waves for probe 1 and its 32x32x16 form; 12 waves for 64 tokens and 8 "
                     "for 128 in probe 2); "
                     "best of 5 launches after 0.2 s of back-to-back launches; ns per MFMA issued on one SIMD; "
                     "mfma_rate_frac = the MFMA-only loop's ns per MFMA / this one's")
    del out, wg, wu
    return res


def measure_partial_sinks(torch):
    """Where the fused prefill unit's split-K partials could go, at the M = 256
    unit's shape (232 workgroups of 12 waves, each a 64-token x 4096-row partial
    written in 32-row tiles, libzinc_peaks.so): fp16 stores to a region per
    workgroup (what the unit does, 121.6 MB), fp32 stores (243 MB), or fp32
    atomic adds into one accumulator per (XCD, token tile), chosen by the
    hardware XCC id so that each accumulator is updated from one XCD (32 MB).
    Best of five launches; the atomic form is checked element by element."""
    import ctypes
    lib = ctypes.CDLL(PEAKS_LIB)
    lib.zinc_peak_partial_sink.restype = ctypes.c_int
    lib.zinc_peak_partial_sink.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    cur = torch.cuda.current_stream()
    n_wg, tok, H = 232, 64, 4096
    acc = torch.zeros(8 * 4 * tok * H, dtype=torch.float32, device=dev)
    part = torch.empty(n_wg * tok * H, dtype=torch.float32, device=dev)
    xcc = torch.zeros(n_wg, dtype=torch.int32, device=dev)
    res = {}
    for mode, name, mb in ((0, "fp16_stores_per_unit", n_wg * tok * H * 2 / 1e6),
                           (1, "fp32_stores_per_unit", n_wg * tok * H * 4 / 1e6),
                           (2, "fp32_atomics_per_xcd_accumulator", 8 * 4 * tok * H * 4 / 1e6)):
        best = float("inf")
        for r in range(6):
            acc.zero_()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(cur)
            if lib.zinc_peak_partial_sink(mode, n_wg, acc.data_ptr(), part.data_ptr(), xcc.data_ptr(),
                                          cur.cuda_stream) != 0:
                raise RuntimeError("partial-sink probe launch failed")
            e1.record(cur)
            e1.synchronize()
            if r:
                best = min(best, e0.elapsed_time(e1) * 1e3)
        res[name] = {"us": round(best, 2), "MB_written": round(mb, 1)}
        if mode == 2:
            x = xcc.cpu().numpy() & 7
            counts = torch.zeros(8, 4, dtype=torch.float32)
            for b in range(n_wg):
                counts[x[b], b % 4] += 1
            want = counts.to(dev).reshape(8, 4, 1).expand(8, 4, tok * H).reshape(-1)
            res[name]["wrong_elements"] = int((acc != want).sum().item())
            res[name]["workgroups_off_block_id_mod_8"] = int(sum(int(x[b]) != b % 8 for b in range(n_wg)))
    del acc, part, xcc
    return res


def measure_stream_layouts(torch):
    """Bandwidth of three ways to read a 4096 x 11008 gate/up pair of Q4_K
    matrices (50.7 MB), over 32 rotating pairs so that every launch reads from
    HBM (libzinc_peaks.so): a row per wave with the lanes along the row (the
    decode row kernels); 16-row tiles per wave in the MFMA lane layout, walked
    one block column at a time (the fused units and the MFMA decode); the same
    tiles two block columns long, so that a tile is 4.6 KB of contiguous
    memory."""
    import ctypes
    lib = ctypes.CDLL(PEAKS_LIB)
    lib.zinc_peak_q4k_stream.restype = ctypes.c_int
    lib.zinc_peak_q4k_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    cur = torch.cuda.current_stream()
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    rows, nb = 11008, 16
    nbytes = rows * nb * 144
    pairs = [(torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=dev),
              torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=dev)) for _ in range(32)]
    out = torch.empty(ncu * 2 * 256, dtype=torch.int32, device=dev)
    res = {}
    for name, layout, lnb, lrows in (("row_per_wave", 0, nb, rows), ("mfma_tiles_16_blocks", 1, nb, rows),
                                     ("mfma_tiles_2_blocks", 1, 2, rows * nb // 2)):
        def run(i):
            g, u = pairs[i % 32]
            if lib.zinc_peak_q4k_stream(layout, g.data_ptr(), u.data_ptr(), lnb, lrows, 2 * ncu, out.data_ptr(),
                                        cur.cuda_stream) != 0:
                raise RuntimeError("stream probe launch failed")
        for i in range(64):
            run(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        best = float("inf")
        for _ in range(3):
            e0.record(cur)
            for i in range(32):
                run(i)
            e1.record(cur)
            e1.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e-3 / 32)
        res[name] = {"us": round(best * 1e6, 2), "GBs": round(2 * nbytes / best / 1e9, 1)}
    res["method"] = ("loads only (folded into a sink), two 4-wave workgroups per CU, best of three sweeps of 32 "
                     "launches over 32 rotating pairs")
    del pairs, out
    torch.cuda.empty_cache()
    return res


class ClockSampler:
    """Samples the GPU's graphics clock and socket power through amdsmi in a
    background thread while a timed region runs (every ~10 ms).  Any failure
    leaves the record empty with the reason, and never stops the benchmark.
    The driver's figures lag the load by up to about a second (a sampler
    started with the load has read the idle clock throughout), so record()
    keeps only the samples taken after `settle_s`."""

    def __init__(self, torch):
        import threading
        self.samples, self.error, self._stop = [], None, threading.Event()
        self._thread, self._h, self._smi = None, None, None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            want = None
            try:
                p = torch.cuda.get_device_properties(0)
                want = (int(getattr(p, "pci_domain_id", 0)), int(p.pci_bus_id), int(p.pci_device_id))
            except Exception:
                pass
            pick = handles[0] if len(handles) == 1 else None
            for h in handles:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)        # "dddd:bb:dd.f"
                dom, bus, rest = bdf.split(":")
                if want and (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                    pick = h
            if pick is None:
                raise RuntimeError(f"no amdsmi device matches the HIP device ({len(handles)} seen)")
            self._h, self._smi = pick, amdsmi
        except Exception as e:   # noqa: BLE001 - reported in the record
            self.error = f"{type(e).__name__}: {e}"

    def _read(self):
        smi = self._smi
        clk = smi.amdsmi_get_clock_info(self._h, smi.AmdSmiClkType.GFX)
        pw = smi.amdsmi_get_power_info(self._h)
        watts = pw.get("socket_power", pw.get("current_socket_power", pw.get("average_socket_power")))
        return float(clk.get("clk", clk.get("cur_clk"))), (float(watts) if watts not in (None, "N/A") else None)

    def __enter__(self):
        import threading
        import time as _t
        if self._h is None:
            return self

        def loop():
            while not self._stop.is_set():
                try:
                    self.samples.append((_t.perf_counter(), *self._read()))
                except Exception as e:   # noqa: BLE001
                    self.error = f"{type(e).__name__}: {e}"
                    return
                _t.sleep(0.01)
        self._thread = threading.Thread(target=loop, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread:
            self._thread.join(timeout=2)

    def record(self, where: str, settle_s: float = 0.0):
        if not self.samples:
            return {"samples": 0, "where": where, "error": self.error or "no sample taken"}
        t0 = self.samples[0][0]
        kept = [(c, w) for t, c, w in self.samples if t - t0 >= settle_s] or [s[1:] for s in self.samples[-1:]]
        clk = sorted(c for c, _ in kept)
        pw = [w for _, w in kept if w is not None]
        return {"samples": len(clk), "where": where, "after_s": settle_s, "gfx_mhz_median": clk[len(clk) // 2],
                "gfx_mhz_min": clk[0], "gfx_mhz_max": clk[-1],
                "power_w_median": (sorted(pw)[len(pw) // 2] if pw else None), "error": self.error}


def sample_clock(torch, fn, where, seconds=2.0, settle_s=1.2):
    """The graphics clock and socket power while `fn` runs back to back, from
    the samples taken after the first `settle_s` seconds."""
    sampler = ClockSampler(torch)
    with sampler:
        t0, i = time.perf_counter(), 0
        while time.perf_counter() - t0 < seconds:
            fn(i)
            i += 1
            if i % 64 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
    return sampler.record(where, settle_s)


def call_percentiles(torch, fn, calls=50):
    """Whole-call durations, one HIP event pair per call on the current stream:
    median, p10 and p90 in microseconds."""
    cur = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for i, (a, b) in enumerate(ev):
        a.record(cur)
        fn(i)
        b.record(cur)
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    q = lambda f: round(us[min(len(us) - 1, int(f * len(us)))], 2)
    return {"median": q(0.5), "p10": q(0.1), "p90": q(0.9), "calls": calls}


def headline(args, torch, peaks=None):
    import numpy as np

    import q4_swiglu_mlp_amd as Z
    import q4k_synth as S
    w = S.WORKLOADS["prefill_m256"]
    dev = torch.device("cuda:0")
    wg, wu, wd = S.layer_weights(w.seed, 0, w.hidden, w.inter)
    x = S.workload_x(w)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    gwg, gwu, gwd, gx = t(wg), t(wu), t(wd), t(x)
    y = torch.empty((w.M, w.hidden), dtype=torch.float16, device=dev)
    ws = torch.empty(Z.prefill_workspace_size(w.M, w.hidden, w.inter), dtype=torch.uint8, device=dev)

    def call(_i):
        Z.zinc_mlp_q4k_prefill(gwg, gwu, gwd, w.hidden, w.inter, gx, w.inter_shift, w.out_shift, y=y, workspace=ws)

    wall, ms = time_calls(call, args.steps, args.warmup, torch)
    extras = not getattr(args, "no_extras", False)
    clock = (sample_clock(torch, call, "back-to-back headline calls for 2 s after the timed region, the last 0.8 s")
             if extras else {"samples": 0, "error": "not sampled (--no-extras)"})
    kern_ms = sum(ms) / len(ms)
    pct = call_percentiles(torch, call) if extras else None
    graph_us = prefill_graph_us(torch, call, y) if extras else None
    flops = 6.0 * w.M * w.hidden * w.inter
    achieved = flops / (kern_ms * 1e-3) / 1e12
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE))
        if rec.get("source_sha256") == kernel_source_hash():
            traffic = rec.get("hbm_bytes_per_launch")
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_F16_TFLOPS, 4), "traffic": traffic,
                "kernel": "k_prefill_fused16", "kernel_ms": round(kern_ms, 5),
                "flops_per_launch": flops}
    if peaks and peaks.get("mfma_f16_16x16_tflops_burst"):
        mp = max(peaks["mfma_f16_16x16_tflops_burst"], peaks.get("mfma_f16_32x32_tflops_burst", 0.0))
        roofline["frac_of_measured_peak"] = round(achieved / mp, 4)
        roofline["measured_peak"] = mp
    if clock.get("gfx_mhz_median"):
        # the spec peak scaled to the clock observed during the timed calls
        roofline["frac_at_observed_clock"] = round(
            achieved / (PEAK_F16_TFLOPS * clock["gfx_mhz_median"] / SPEC_GFX_MHZ), 4)
    res = {
        "value": w.M * args.steps / wall,
        "ms_per_step": wall / args.steps * 1e3,
        "roofline": roofline,
        "whole_call_tflops": round(flops / (wall / args.steps) / 1e12, 2),
        "graph_replay": ({"us_per_call": round(graph_us, 3), "tokens_per_s": round(w.M / (graph_us * 1e-6), 1)}
                         if graph_us else None),
        "call_us": pct,
        "clock": clock,
    }
    inputs = (wg, wu, wd, x)
    return res, inputs


def prefill_graph_us(torch, call, y, replays=200, warm_s=0.1):
    """Per-call time of the whole prefill call (staging, fused kernel,
    reduce) captured once in a HIP graph and replayed: the device-side rate
    without the host's launch cost.  Every replay must reproduce the eager
    output bit for bit.  The timed replays follow at least warm_s seconds of
    back-to-back replays, as the clock climbs for the first ~200 calls after
    the device idles."""
    call(0)
    torch.cuda.synchronize()
    want = y.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(0)
    for _ in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(y, want):
            raise RuntimeError("graph replay of the prefill call differs from the eager call")
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        for _ in range(20):
            g.replay()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(replays):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / replays * 1e6


def host_cpu():
    """The host's CPU model, sockets and the cores this process may use."""
    model, sockets = None, set()
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name") and model is None:
                model = line.split(":", 1)[1].strip()
            elif line.startswith("physical id"):
                sockets.add(line.split(":", 1)[1].strip())
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count()
    return {"cpu_model": model, "sockets": len(sockets) or None, "nproc": nproc}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:   # noqa: BLE001
        return None


def _time_until(fn, min_s, max_reps):
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_s or reps >= max_reps:
            return reps, dt


def cpu_baseline(inputs, full: bool = False):
    """The oracle as it stands (numpy float64: decode + three matmuls), on the
    host cores: the headline workload's full layer (256 tokens) repeated for
    at least 10 s, then one call each of the other workloads' shapes (tiny,
    decode M=1 and M=4, the 64-expert MoE) and the tiny layer on one thread.
    ``full`` adds the headline layer on one thread (tens of seconds)."""
    import numpy as np

    import oracle as O
    import q4k_synth as S
    w = S.WORKLOADS["prefill_m256"]
    wg, wu, wd, x = inputs
    cores = blas_threads() or os.cpu_count()
    reps, dt = _time_until(lambda: O.mlp(x, wg, wu, wd, w.hidden, w.inter), 10.0, 50)
    res = {"value": round(reps * w.M / dt, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": f"the full 4096/11008 layer, {w.M} tokens, {reps} times (numpy float64 oracle: decode + 3 "
                     f"matmuls), {dt:.2f} s; cores = the BLAS threads numpy ran with"}
    res.update(host_cpu())
    other = {}
    t = S.WORKLOADS["tiny"]
    tw = S.layer_weights(t.seed, 0, t.hidden, t.inter)
    tx = S.workload_x(t)
    r, d = _time_until(lambda: O.mlp(tx, *tw, t.hidden, t.inter), 1.0, 1000)
    other["tiny_256_768_M8_tokens_per_s"] = round(r * t.M / d, 1)
    dw = S.WORKLOADS["decode_m4"]
    lw = S.layer_weights(dw.seed, 0, dw.hidden, dw.inter)
    dx = S.workload_x(dw)
    for M in (1, 4):
        r, d = _time_until(lambda: O.mlp(dx[:M], *lw, dw.hidden, dw.inter), 2.0, 20)
        other[f"decode_M{M}_s_per_layer"] = round(d / r, 3)
        other[f"decode_M{M}_32_layers_s_extrapolated"] = round(32 * d / r, 2)
    mw = S.WORKLOADS["moe_e64"]
    eg, eu, ed = S.expert_weights(mw.seed, mw.n_experts, mw.hidden, mw.inter)
    mx = S.workload_x(mw)
    ids, p = S.workload_routing(mw)
    t0 = time.perf_counter()
    O.moe(mx, eg, eu, ed, ids, p, mw.hidden, mw.inter)
    d = time.perf_counter() - t0
    other["moe_e64_top8_M512_s_per_call"] = round(d, 3)
    other["moe_e64_top8_M512_tokens_per_s"] = round(mw.M / d, 1)
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            r, d = _time_until(lambda: O.mlp(tx, *tw, t.hidden, t.inter), 1.0, 1000)
            other["tiny_tokens_per_s_one_thread"] = round(r * t.M / d, 1)
            if full:
                r, d = _time_until(lambda: O.mlp(x, wg, wu, wd, w.hidden, w.inter), 1.0, 3)
                other["headline_layer_tokens_per_s_one_thread"] = round(r * w.M / d, 3)
    except Exception as e:   # noqa: BLE001
        other["one_thread_error"] = f"{type(e).__name__}: {e}"
    res["other_workloads"] = other
    return res


def secondary(args, torch):
    import numpy as np

    import q4_swiglu_mlp_amd as Z
    import q4k_synth as S
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    out = []
    if args.only in (None, "decode"):
        out += decode_lines(args, torch, np, Z, S, dev, t)
    if args.only in (None, "moe"):
        out += moe_lines(args, torch, np, Z, S, dev, t)
    if args.only in (None, "block"):
        out += block_lines(args, torch, np, Z, S, dev, t)
    if args.only in (None, "m2048"):
        out += m2048_lines(args, torch, np, Z, S, dev, t)
    if args.only == "staged":   # its own run: its fused calls at M=2048 would mix into the headline kernel's trace
        out += staged_lines(args, torch, np, Z, S, dev, t)
    if args.only == "m384":     # its own run, for the counters of the 257-511-token unit
        out += m384_lines(args, torch, np, Z, S, dev, t)
    return out


def m384_lines(args, torch, np, Z, S, dev, t):
    """A mid-size prefill that the plan gives to the 64-token unit with
    384-row chunks (257-511 tokens): 384 tokens through layer 0 of the M=256
    workload's weights (seed 1, its shifts), x ~ N(0, 1) of its own seed;
    whole-call time and the fused kernel by HIP events."""
    w = S.WORKLOADS["prefill_m256"]
    M = 384
    wg, wu, wd = (t(a) for a in S.layer_weights(w.seed, 0, w.hidden, w.inter))
    gx = t(S.gen_x(np.random.default_rng([w.seed, 384]), M, w.hidden))
    y = torch.empty((M, w.hidden), dtype=torch.float16, device=dev)
    ws = torch.empty(Z.prefill_workspace_size(M, w.hidden, w.inter), dtype=torch.uint8, device=dev)

    def call(_i):
        Z.zinc_mlp_q4k_prefill(wg, wu, wd, w.hidden, w.inter, gx, w.inter_shift, w.out_shift, y=y, workspace=ws)

    steps = 50
    wall, ms = time_calls(call, steps, 10, torch, warm_s=0.1)
    per = wall / steps
    kern = sum(ms) / len(ms)
    flops = 6.0 * M * w.hidden * w.inter
    out = [{
        "workload": "prefill 4096/11008 M=384 (layer 0 of seed 1), the 257-511-token unit",
        "tokens_per_s": round(M / per, 1),
        "us_per_call": round(per * 1e6, 2),
        "fused_kernel_us": round(kern * 1e3, 2),
        "fused_kernel_mfma_frac": round(flops / (kern * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
    }]
    log(f"[bench] {out[-1]}")
    return out


def m2048_lines(args, torch, np, Z, S, dev, t):
    """The large prefill: 2048 tokens through 32 independent 4096/11008 layers
    (seed 2, x sd 0.5), each layer one call; whole-call time per layer."""
    w = S.WORKLOADS["prefill_m2048"]
    n_layers = min(args.layers, w.layers)
    layers = [tuple(t(a) for a in S.layer_weights(w.seed, l, w.hidden, w.inter)) for l in range(n_layers)]
    gx = t(S.workload_x(w))
    y = torch.empty((w.M, w.hidden), dtype=torch.float16, device=dev)
    ws = torch.empty(Z.prefill_workspace_size(w.M, w.hidden, w.inter), dtype=torch.uint8, device=dev)

    def call(i):
        lg, lu, ld = layers[i % n_layers]
        Z.zinc_mlp_q4k_prefill(lg, lu, ld, w.hidden, w.inter, gx, w.inter_shift, w.out_shift, y=y, workspace=ws)

    steps = 3 * n_layers
    wall, ms = time_calls(call, steps, n_layers, torch, warm_s=0.05)
    per = wall / steps
    kern = sum(ms) / len(ms)   # the fused kernel of each call (HIP events on its stream)
    flops = 6.0 * w.M * w.hidden * w.inter
    out = [{
        "workload": f"prefill 4096/11008 M=2048, {n_layers}-layer sweep (seed 2)",
        "tokens_per_s": round(w.M / per, 1),
        "us_per_layer": round(per * 1e6, 2),
        "whole_call_tflops": round(flops / per / 1e12, 2),
        "whole_call_mfma_frac": round(flops / per / 1e12 / PEAK_F16_TFLOPS, 4),
        "fused_kernel_us": round(kern * 1e3, 2),
        "fused_kernel_mfma_frac": round(flops / (kern * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
    }]
    log(f"[bench] {out[-1]}")
    del layers
    return out


def block_lines(args, torch, np, Z, S, dev, t):
    """The MLP block entry points (pre-MLP RMS norm + MLP + residual) against
    the plain MLP call: prefill M=256 and decode M=1, whole calls."""
    out = []
    for name, fblock, fplain, steps in (("prefill_m256", Z.zinc_mlp_q4k_prefill_block, Z.zinc_mlp_q4k_prefill, 100),
                                        ("decode_m1", Z.zinc_mlp_q4k_decode_block, Z.zinc_mlp_q4k_decode, 200)):
        w = S.WORKLOADS[name]
        wg, wu, wd = (t(a) for a in S.layer_weights(w.seed, 0, w.hidden, w.inter))
        gx = t(S.workload_x(w))
        gamma = t(np.random.default_rng(w.seed).uniform(0.5, 1.5, w.hidden).astype(np.float16))
        y = torch.empty((w.M, w.hidden), dtype=torch.float16, device=dev)
        wsb = torch.empty(4 << 20 if w.M == 1 else 160 << 20, dtype=torch.uint8, device=dev)

        def blk(_i):
            fblock(wg, wu, wd, w.hidden, w.inter, gx, gamma, 1e-5, 1.0, w.inter_shift, w.out_shift, y=y, workspace=wsb)

        def plain(_i):
            fplain(wg, wu, wd, w.hidden, w.inter, gx, w.inter_shift, w.out_shift, y=y, workspace=wsb)

        tb = min(time_calls(blk, steps, 5, torch, warm_s=0.05)[0] for _ in range(2)) / steps
        tp = min(time_calls(plain, steps, 5, torch, warm_s=0.05)[0] for _ in range(2)) / steps
        out.append({
            "workload": f"MLP block (RMS norm + MLP + residual) vs plain MLP call, {name} (4096/11008, M={w.M})",
            "block_us": round(tb * 1e6, 2),
            "plain_us": round(tp * 1e6, 2),
            "block_tokens_per_s": round(w.M / tb, 1),
        })
        log(f"[bench] {out[-1]}")
    return out


def staged_lines(args, torch, np, Z, S, dev, t):
    """The fused prefill against its staged comparison baseline (unit D's
    units with G, U and the intermediate in device memory), whole calls.  At
    M=256 both calls run unit D, so they differ only in where the intermediate
    lives; at M=2048 the fused call runs its default unit (the 128-token unit
    E) and the staged call unit D."""
    out = []
    for name, steps in (("prefill_m256", 50), ("prefill_m2048", 10)):
        w = S.WORKLOADS[name]
        wg, wu, wd = (t(a) for a in S.layer_weights(w.seed, 0, w.hidden, w.inter))
        gx = t(S.workload_x(w))
        y = torch.empty((w.M, w.hidden), dtype=torch.float16, device=dev)
        wsf = torch.empty(Z.prefill_workspace_size(w.M, w.hidden, w.inter), dtype=torch.uint8, device=dev)
        wss = torch.empty(Z.prefill_staged_workspace_size(w.M, w.hidden, w.inter), dtype=torch.uint8, device=dev)

        def fused(_i):
            Z.zinc_mlp_q4k_prefill(wg, wu, wd, w.hidden, w.inter, gx, w.inter_shift, w.out_shift, y=y, workspace=wsf)

        def staged(_i):
            Z.zinc_mlp_q4k_prefill_staged(wg, wu, wd, w.hidden, w.inter, gx, w.inter_shift, w.out_shift, y=y,
                                          workspace=wss)

        # alternate the two a few times (same thermal state), keep each one's best round
        best_f, best_s = float("inf"), float("inf")
        for _ in range(3):
            best_f = min(best_f, time_calls(fused, steps, 3, torch, warm_s=0.05)[0] / steps)
            best_s = min(best_s, time_calls(staged, steps, 3, torch, warm_s=0.05)[0] / steps)
        crossing = 6 * w.M * w.inter * 2
        out.append({
            "workload": f"fused vs staged prefill 4096/11008 M={w.M} (seed {w.seed}, layer 0)",
            "units": "fused D, staged D" if w.M <= 256 else "fused E, staged D",
            "fused_us": round(best_f * 1e6, 2),
            "staged_us": round(best_s * 1e6, 2),
            "staged_over_fused": round(best_s / best_f, 3),
            "fused_tokens_per_s": round(w.M / best_f, 1),
            "staged_tokens_per_s": round(w.M / best_s, 1),
            "intermediate_crossings_MB": round(crossing / 1e6, 2),
        })
        log(f"[bench] {out[-1]}")
        del wsf, wss
    return out


def decode_graph_us(torch, Z, layers, w, gx, y, ws, replays=30, warm_s=0.1):
    """Per-layer time of the 32-layer sweep captured once in a HIP graph and
    replayed: the device-side rate without the host's per-call launch cost,
    timed after at least warm_s seconds of back-to-back replays."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for lg, lu, ld in layers:   # warm the path on the capture stream
            Z.zinc_mlp_q4k_decode(lg, lu, ld, w.hidden, w.inter, gx, w.inter_shift, w.out_shift, y=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for lg, lu, ld in layers:
            Z.zinc_mlp_q4k_decode(lg, lu, ld, w.hidden, w.inter, gx, w.inter_shift, w.out_shift, y=y, workspace=ws)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        g.replay()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(replays):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / (replays * len(layers)) * 1e6


def decode_lines(args, torch, np, Z, S, dev, t):
    out = []
    # decode: 32 independent layers so the 2.4 GB of weights stream from HBM
    w1 = S.WORKLOADS["decode_m1"]
    layers = [tuple(t(a) for a in S.layer_weights(w1.seed, l, w1.hidden, w1.inter))
              for l in range(min(args.layers, w1.layers))]
    layer_bytes = 2 * q4k_bytes(w1.inter, w1.hidden) + q4k_bytes(w1.hidden, w1.inter)
    for name in ("decode_m1", "decode_m4"):
        w = S.WORKLOADS[name]
        gx = t(S.workload_x(w))
        y = torch.empty((w.M, w.hidden), dtype=torch.float16, device=dev)
        ws = torch.empty(Z.decode_workspace_size(w.M, w.hidden, w.inter), dtype=torch.uint8, device=dev)

        def call(i, w=w, gx=gx, y=y, ws=ws):
            lg, lu, ld = layers[i % len(layers)]
            Z.zinc_mlp_q4k_decode(lg, lu, ld, w.hidden, w.inter, gx, w.inter_shift, w.out_shift, y=y, workspace=ws)

        steps = len(layers) * 10
        wall, ms = time_calls(call, steps, len(layers), torch, warm_s=0.05)
        per_layer = wall / steps
        kern_ms = sum(ms) / steps   # the timed kernels of one call (gate+up and down)
        graph_us = decode_graph_us(torch, Z, layers, w, gx, y, ws)
        out.append({
            "workload": f"decode 4096/11008 M={w.M}, {len(layers)}-layer sweep",
            "tokens_per_s_per_layer": round(w.M / per_layer, 1),
            "us_per_layer": round(per_layer * 1e6, 3),
            "hbm_GBs_whole_call": round(layer_bytes / per_layer / 1e9, 1),
            "hbm_frac_whole_call": round(layer_bytes / per_layer / 1e9 / PEAK_HBM_GBS, 4),
            "us_per_layer_graph": round(graph_us, 3),
            "hbm_frac_graph": round(layer_bytes / (graph_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "kernel_us": round(kern_ms * 1e3, 3),
            "kernel_GBs": round(layer_bytes / (kern_ms * 1e-3) / 1e9, 1),
            "kernel_hbm_frac": round(layer_bytes / (kern_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        })
        log(f"[bench] {out[-1]}")
    del layers
    return out


def moe_lines(args, torch, np, Z, S, dev, t):
    out = []
    # MoE: two rotated expert sets (340 MB > the 256 MB last-level cache)
    w = S.WORKLOADS["moe_e64"]
    sets = [tuple(t(a) for a in S.expert_weights(w.seed, w.n_experts, w.hidden, w.inter, layer=l)) for l in range(2)]
    gx = t(S.workload_x(w))
    ids, p = S.workload_routing(w)
    gids, gp = t(ids), t(p)
    y = torch.empty((w.M, w.hidden), dtype=torch.float16, device=dev)
    ws = torch.empty(Z.moe_workspace_size(w.M, w.top_k, w.n_experts, w.hidden, w.inter), dtype=torch.uint8,
                     device=dev)

    def mcall(i):
        eg, eu, ed = sets[i % 2]
        Z.zinc_moe_q4k_experts(eg, eu, ed, w.n_experts, w.hidden, w.inter, gx, gids, gp, w.inter_shift, w.out_shift,
                               y=y, workspace=ws)

    steps = 100
    wall, ms = time_calls(mcall, steps, 10, torch, warm_s=0.05)
    per = wall / steps
    kern = sum(ms) / len(ms)
    wbytes = w.n_experts * (2 * q4k_bytes(w.inter, w.hidden) + q4k_bytes(w.hidden, w.inter))
    flops = 6.0 * w.M * w.top_k * w.hidden * w.inter
    out.append({
        "workload": "MoE E=64 top-8, 2048->768, M=512, two rotated expert sets",
        "tokens_per_s": round(w.M / per, 1),
        "us_per_call": round(per * 1e6, 3),
        "k_moe_fused_us": round(kern * 1e3, 3),
        "hbm_frac_fused_kernel": round(wbytes / (kern * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "mfma_frac_fused_kernel": round(flops / (kern * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
    })
    log(f"[bench] {out[-1]}")

    # the same call on one expert set (170 MB, within the 256 MB last-level
    # cache): the warm case, beside the cold one above
    def mcall_warm(_i):
        eg, eu, ed = sets[0]
        Z.zinc_moe_q4k_experts(eg, eu, ed, w.n_experts, w.hidden, w.inter, gx, gids, gp, w.inter_shift, w.out_shift,
                               y=y, workspace=ws)

    wall, ms = time_calls(mcall_warm, steps, 10, torch, warm_s=0.05)
    per = wall / steps
    kern = sum(ms) / len(ms)
    out.append({
        "workload": "MoE E=64 top-8, 2048->768, M=512, one expert set (cache-warm)",
        "tokens_per_s": round(w.M / per, 1),
        "us_per_call": round(per * 1e6, 3),
        "k_moe_fused_us": round(kern * 1e3, 3),
        "weight_GBs_fused_kernel": round(wbytes / (kern * 1e-3) / 1e9, 1),
        "mfma_frac_fused_kernel": round(flops / (kern * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
    })
    log(f"[bench] {out[-1]}")

    # the router on the GPU (top-8 of 64 logits per token), alone and feeding
    # the expert call: the MoE block with no host read-back between the two
    glog = t(S.workload_router_logits(w))
    rids = torch.empty((w.M, w.top_k), dtype=torch.int32, device=dev)
    rp = torch.empty((w.M, w.top_k), dtype=torch.float32, device=dev)

    def rcall(_i):
        Z.zinc_moe_route_topk(glog, w.top_k, expert_ids=rids, expert_weights=rp)

    def lcall(i):
        rcall(i)
        eg, eu, ed = sets[i % 2]
        Z.zinc_moe_q4k_experts(eg, eu, ed, w.n_experts, w.hidden, w.inter, gx, rids, rp, w.inter_shift, w.out_shift,
                               y=y, workspace=ws)

    # the same experts with their down projections in Q5_K and Q5_1 (one
    # expert set each, the weights rotated with the Q4_K set's up projections)
    rng = np.random.default_rng([w.seed, 50])
    for fmt in ("q5_k", "q5_1"):
        wd5 = t(np.stack([S.gen_down_blob(rng, fmt, w.hidden, w.inter) for _ in range(w.n_experts)]))

        def fcall(i):
            eg, eu, _ = sets[i % 2]
            Z.zinc_moe_experts_fmt(eg, eu, wd5, fmt, w.n_experts, w.hidden, w.inter, gx, gids, gp, w.inter_shift,
                                   w.out_shift, y=y, workspace=ws)

        fwall, fms = time_calls(fcall, steps, 10, torch, warm_s=0.05)
        out.append({
            "workload": f"MoE E=64 top-8, 2048->768, M=512, down projections in {fmt.upper()}",
            "tokens_per_s": round(w.M / (fwall / steps), 1),
            "us_per_call": round(fwall / steps * 1e6, 3),
            "k_moe_fused_us": round(sum(fms) / len(fms) * 1e3, 3),
        })
        log(f"[bench] {out[-1]}")
        del wd5

    rwall, rms = time_calls(rcall, steps, 10, torch, warm_s=0.05)
    lwall, _ = time_calls(lcall, steps, 10, torch, warm_s=0.05)
    out.append({
        "workload": "MoE router, top-8 of 64 fp32 logits, M=512; then router + experts as one block",
        "router_us_per_call": round(rwall / steps * 1e6, 3),
        "router_kernel_us": round(sum(rms) / len(rms) * 1e3, 3),
        "router_plus_experts_us": round(lwall / steps * 1e6, 3),
        "router_plus_experts_tokens_per_s": round(w.M / (lwall / steps), 1),
    })
    log(f"[bench] {out[-1]}")
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # the graphics clock climbs for the first ~200 calls (~25 ms) of back-to-back
    # work after idle: the timed calls start once it has settled
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["decode", "moe", "block", "m2048", "staged", "m384", "peaks", "cpu"],
                    default=None,
                    help="development and profiling runs: skip the headline and run one part (a secondary line, "
                         "the measured peaks, or the full CPU oracle table including one-thread figures)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak microbenchmarks")
    ap.add_argument("--no-extras", action="store_true",
                    help="headline: only the warmup and timed calls (no clock sampling, percentile calls or graph "
                         "replay), for counter collection")
    ap.add_argument("--layers", type=int, default=32,
                    help="layers of the 32-layer sweeps (decode, 2048-token prefill); fewer for profiling runs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (3x), the reference kernel that "
                         "scales the FETCH_SIZE/WRITE_SIZE counters to bytes")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": src.numel() * 4, "copies": 3}))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the path has no multi-GPU mode (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}). Token-parallel sharding of this layer needs no collective.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.only == "peaks":
        print(json.dumps({"measured_peaks": measure_peaks(torch), "issue_probes": measure_issue_probes(torch),
                          "q4k_stream_layouts": measure_stream_layouts(torch),
                          "partial_sinks": measure_partial_sinks(torch)}), flush=True)
        return
    if args.only == "cpu":
        import q4k_synth as S
        w = S.WORKLOADS["prefill_m256"]
        inputs = (*S.layer_weights(w.seed, 0, w.hidden, w.inter), S.workload_x(w))
        print(json.dumps({"cpu_baseline": cpu_baseline(inputs, full=True)}), flush=True)
        return
    if args.only:
        print(json.dumps({"secondary": secondary(args, torch)}), flush=True)
        return
    peaks = None
    if not args.no_peaks:
        try:
            peaks = measure_peaks(torch)
            log(f"[bench] measured peaks {peaks}")
        except Exception as e:   # noqa: BLE001 - the peaks are context, never the headline
            peaks = {"error": f"{type(e).__name__}: {e}"}
    log("[bench] headline: prefill 4096/11008 M=256")
    res, inputs = headline(args, torch, peaks)
    log(f"[bench] headline {res['value']:.1f} tok/s, kernel {res['roofline']['kernel_ms'] * 1e3:.1f} us, "
        f"{res['roofline']['achieved']} TFLOP/s")
    sec = None if args.no_secondary else secondary(args, torch)
    cpu = None if args.no_cpu_baseline else cpu_baseline(inputs)
    if cpu:
        log(f"[bench] cpu baseline {cpu}")
    line = {
        "metric": METRIC,
        "value": round(res["value"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "one Q4_K SwiGLU MLP layer, hidden 4096, intermediate 11008, 256-token prefill tile, "
                               "seed 1", "hidden": 4096, "inter": 11008, "M": 256, "weights": "Q4_K",
                   "compute": "fp16 MFMA, fp32 accumulate"},
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
        "whole_call_tflops": res["whole_call_tflops"],
        "graph_replay": res["graph_replay"],
        "call_us": res["call_us"],
        "clock": res["clock"],
        "measured_peaks": peaks,
        "secondary": sec,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
