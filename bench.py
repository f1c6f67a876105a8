"""Benchmark of the routed-expert MoE layer on one MI355X.

One step = one pass of the whole layer (router, exact top-6, expert FFNs with
the shared expert, combine) over one batch of synthetic input with every
input already resident in HBM.

  value          single-token decode: 384 experts, top-6, d=4096, f=2048, a
                 Q8 shared expert, IQ2 gate/up, Q2K down, fp32 x -- tokens/s
                 of one layer (steps/s at T=1)
  prefill_1024   the same layer on 1024-token bf16 chunks
  small_batch_16 16 fp32 tokens of 4 interleaved sessions with expert reuse
                 (caller routes), on the decode path (two calls of 8) and on
                 the prefill path (one call)
  crossover      T = 1 .. 128 on both paths (decode in calls of at most 8)
  long_prefill   8 layers of the same shape, 4096 bf16 tokens each, Zipf(1.1)
                 routes (caller supplied): per-GEMM MFMA and HBM fractions
  probes         achievable HBM read bandwidth and fp16 MFMA rate on this GPU

Cold-HBM protocol: the 256 MB Infinity Cache would otherwise hold a decode
step's ~75 MB.  Steps cycle over 16 layer descriptors, each with its own
router and shared expert, over two physical copies of the routed experts, and
16 distinct tokens (so routes differ step to step): the working set is far
beyond the cache.  Decode steps are captured in a graph of 16 steps and
replayed; any remainder runs eagerly, so exactly --steps steps are timed.

Per-kernel durations come from HIP events the library records on the launch
stream (eager pass); the roofline object is for the dominant decode kernel.
The CPU baseline is the test oracle (never tuned) on a bounded sample.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
F16_PEAK_TFLOPS = 2500.0    # MI355X dense fp16/bf16 MFMA, published
N_DESC = 16  # layer descriptors (router + shared expert sets) cycled by the steps
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
PROBE_LIB = os.path.join(ROOT, "quantized_moe_amd", "libqmoe_probe.so")
METRIC = "MoE layer tokens/s (decode B=1, prefill 1024) + achieved HBM GB/s / MFMA % of peak"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_moe_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from committed PMC counter runs, if they were taken
    on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


COPY_BYTES = 512 << 20  # calibration copy: reads and writes exactly this many bytes per dispatch

# library kernel (as named by the per-launch timing hooks) -> substring of the
# device kernel name in a rocprofv3 record
KERNEL_SYMBOLS = {
    "decode_router": "k1_kernel",
    "decode_gateup": "k2_kernel",
    "decode_down_combine": "k3_kernel",
    "prefill_gateup": "gemm_kernel<1, true",
    "prefill_down": "gemm_kernel<2, false",
}
# the shared expert's kernels (Q8: fp16 weight copies, the two library GEMMs
# -- hipBLASLt's kernel names start with Cijk_ -- and the SwiGLU), for the
# instruction-counter tables only
PMC_EXTRA_SYMBOLS = {"prefill_shared_dequant": "dequant_q8_kernel", "prefill_shared_gemms (hipBLASLt)": "Cijk_",
                     "prefill_shared_swiglu": "swiglu_kernel"}


def pmc_table(dirs) -> int:
    """Per-launch means of every SQ/GRBM counter in rocprofv3 --pmc runs of
    bench.py --pmc-mode, per library kernel, and the ratios derived from
    them.  Kernel cycles C = GRBM_GUI_ACTIVE / 8 (the counter is summed over
    the 8 XCDs); 256 CUs, 1024 SIMDs."""
    import csv
    import glob

    vals = {}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    vals.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    syms = {**KERNEL_SYMBOLS, **PMC_EXTRA_SYMBOLS}
    rows = {}
    for (kname, counter), vs in vals.items():
        for lib_name, sym in syms.items():
            if sym in kname:
                rows.setdefault(lib_name, {}).setdefault(counter, []).extend(vs)
    def m(r, c):
        v = r.get(c)
        return float(np.mean(v)) if v else None
    for lib_name in syms:
        r = rows.get(lib_name)
        if not r:
            continue
        print(f"{lib_name}:")
        for c in sorted(r):
            print(f"  {c:32s} {m(r, c):16.0f}")
        C = m(r, "GRBM_GUI_ACTIVE")
        C = C / 8.0 if C else None
        def ratio(num, den, scale=1.0):
            a, b = m(r, num), (m(r, den) if isinstance(den, str) else den)
            return None if a is None or not b else a * scale / b
        derived = {
            "kernel cycles C (GRBM_GUI_ACTIVE / 8)": C,
            "VALU instructions per wave": ratio("SQ_INSTS_VALU", "SQ_WAVES"),
            "LDS instructions per wave": ratio("SQ_INSTS_LDS", "SQ_WAVES"),
            "VALU busy per SIMD (4 ACTIVE_INST_VALU / 1024 C)": ratio("SQ_ACTIVE_INST_VALU", 1024 * C, 4) if C else None,
            "MFMA busy per SIMD (MFMA_BUSY_CYCLES / 1024 C)": ratio("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * C) if C else None,
            "LDS busy per CU (LDS_IDX_ACTIVE / 256 C)": ratio("SQ_LDS_IDX_ACTIVE", 256 * C) if C else None,
            "LDS bank-conflict share (BANK_CONFLICT / IDX_ACTIVE)": ratio("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"),
            "wave time waiting on anything (WAIT_ANY / WAVE_CYCLES)": ratio("SQ_WAIT_ANY", "SQ_WAVE_CYCLES"),
            "wave time waiting to issue (WAIT_INST_ANY / WAVE_CYCLES)": ratio("SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"),
        }
        for k, v in derived.items():
            if v is not None:
                print(f"  = {k:58s} {v:12.3f}" if v < 100 else f"  = {k:58s} {v:12.0f}")
    return 0


def pmc_summarize(fetch_dir: str, write_dir: str) -> int:
    """HBM bytes per launch of each kernel from two rocprofv3 --pmc runs of
    bench.py --pmc-mode (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch),
    each scaled by what the same counter reads for the calibration copy."""
    import csv
    import glob

    def per_kernel(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        vals = {}
        for path in files:
            with open(path) as f:
                for r in csv.DictReader(f):
                    if r["Counter_Name"] == counter:
                        vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    out = {"kernel_source_hash": kernel_source_hash(), "copy_bytes": COPY_BYTES, "kernels": {}}
    for counter, d, key in (("FETCH_SIZE", fetch_dir, "fetch"), ("WRITE_SIZE", write_dir, "write")):
        vals = per_kernel(d, counter)
        copy = [v for name, vs in vals.items() if "copy" in name.lower() for v in vs]
        if not copy:
            raise SystemExit(f"no calibration copy kernel in the {counter} run")
        cal = COPY_BYTES / (float(np.median(copy)) * 1024.0)  # bytes per counted byte
        out[f"{key}_calibration"] = round(cal, 4)
        for kname, sym in KERNEL_SYMBOLS.items():
            vs = [v for name, vv in vals.items() if sym in name for v in vv]
            if vs:
                rec = out["kernels"].setdefault(kname, {"dispatches": len(vs)})
                rec[f"{key}_bytes_per_launch"] = round(float(np.mean(vs)) * 1024.0 * cal)
    for rec in out["kernels"].values():
        if "fetch_bytes_per_launch" in rec and "write_bytes_per_launch" in rec:
            rec["hbm_bytes_per_launch"] = rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))
    return 0


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def pct(a) -> dict:
    a = np.asarray(a, np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 6), "p50": round(float(np.median(a)), 6),
            "p90": round(float(np.percentile(a, 90)), 6)}


class Timer:
    """HIP events on torch's current stream (the one every launch goes to)."""

    def __init__(self, torch):
        self.torch = torch

    def __call__(self, fn, reps):
        t = self.torch
        evs = [(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i in range(reps):
            evs[i][0].record()
            fn(i)
            evs[i][1].record()
        t.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs]  # ms per rep


# ------------------------------------------------------------------ probes --
def run_probes(torch, dev, timer):
    """Achievable HBM read bandwidth (at a decode launch's size, rotating
    over buffers so the set exceeds the Infinity Cache, and at the size of a
    prefill chunk's weights) and fp16 MFMA throughput."""
    L = ctypes.CDLL(PROBE_LIB)
    L.qmoe_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.qmoe_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream
    blocks = 256 * 8
    sink = torch.empty(blocks, dtype=torch.int32, device=dev)
    out = {}
    small = 44 << 20  # the decode gate/up launch streams ~43.8 MB
    bufs = [torch.empty(small, dtype=torch.uint8, device=dev) for _ in range(8)]
    big = torch.empty(2750 << 20, dtype=torch.uint8, device=dev)  # a prefill chunk's weights
    for b in bufs + [big]:
        b.fill_(1)
    torch.cuda.synchronize()
    for name, blist, nbytes, reps in (("read_44MB", bufs, small, 64), ("read_2750MB", [big], big.numel(), 6)):
        def go(i, blist=blist, nbytes=nbytes):
            rc = L.qmoe_probe_read(blist[i % len(blist)].data_ptr(), nbytes, blocks, sink.data_ptr(), stream)
            assert rc == 0, rc
        go(0)
        ms = timer(go, reps)
        out[name] = {"GBs": round(nbytes / (float(np.median(ms)) * 1e-3) / 1e9, 1), "bytes": nbytes,
                     "launches": reps, "blocks": blocks}
    del bufs, big
    iters = 4096
    mblocks = 256 * 8
    fsink = torch.empty(mblocks, dtype=torch.float32, device=dev)

    def mf(i):
        rc = L.qmoe_probe_mfma(iters, mblocks, fsink.data_ptr(), stream)
        assert rc == 0, rc
    mf(0)
    ms = timer(mf, 5)
    flops = mblocks * 4 * iters * 8 * 16384.0
    out["mfma_f16_16x16x32"] = {"TFLOPs": round(flops / (float(np.median(ms)) * 1e-3) / 1e12, 1)}
    L.qmoe_probe_mfma32.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]

    def mf32(i):
        rc = L.qmoe_probe_mfma32(iters, mblocks, fsink.data_ptr(), stream)
        assert rc == 0, rc
    mf32(0)
    ms = timer(mf32, 5)
    flops = mblocks * 4 * iters * 4 * 32768.0
    out["mfma_f16_32x32x16"] = {"TFLOPs": round(flops / (float(np.median(ms)) * 1e-3) / 1e12, 1)}
    torch.cuda.empty_cache()
    log(f"probes: {out}")
    return out


def frac_pair(achieved, spec, probe):
    return {"frac": round(achieved / spec, 4), "frac_of_probe": round(achieved / probe, 4) if probe else None}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=4000, help="timed decode steps")
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--prefill-steps", type=int, default=40)
    ap.add_argument("--profile-steps", type=int, default=256, help="eager steps with per-kernel events")
    ap.add_argument("--long-prefill-steps", type=int, default=3, help="timed passes over the 8 long-prefill layers")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bias-gain", action="store_true",
                    help="give every layer a router selection bias and per-channel down gains (not the headline)")
    ap.add_argument("--routed-fmt", choices=["iq2-q2k", "q4k", "mxfp4", "vq12", "vq13"], default="iq2-q2k",
                    help="routed experts: IQ2_XXS-like gate/up + Q2_K-like down (the headline), Q4_K-like, "
                         "MXFP4 or 12/13-bit VQ gate/up/down (variants; not the headline)")
    ap.add_argument("--only", default="all",
                    help="comma list of: decode, prefill, small-batch, crossover, long-prefill, probes (default all)")
    ap.add_argument("--pmc-mode", action="store_true",
                    help="no timing: a few decode and prefill steps and a plain copy of known size, for "
                         "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs")
    ap.add_argument("--pmc-summarize", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn the two counter runs into profiles/traffic_counters.json (no GPU)")
    ap.add_argument("--pmc-table", nargs="+", metavar="DIR",
                    help="print per-kernel instruction/LDS/MFMA counters of --pmc-mode runs (no GPU)")
    args = ap.parse_args()

    if args.pmc_summarize:
        return pmc_summarize(*args.pmc_summarize)
    if args.pmc_table:
        return pmc_table(args.pmc_table)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (expert-parallel sharding is "
              "designed, not built). Run with --gpus 1.", file=sys.stderr)
        return 2
    sections = {"decode", "prefill", "small-batch", "crossover", "long-prefill", "probes"}
    want = sections if args.only == "all" else set(args.only.split(","))
    if not want <= sections:
        print(f"--only: unknown sections {sorted(want - sections)}", file=sys.stderr)
        return 2

    import torch

    from quantized_moe_amd import lib, synth

    lib.lib()  # fails loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    timer = Timer(torch)
    spec = synth.DECODE_SPEC
    if args.routed_fmt != "iq2-q2k":
        fr = {"q4k": synth.FMT_Q4K, "mxfp4": synth.FMT_MX4, "vq12": synth.FMT_VQ12,
              "vq13": synth.FMT_VQ13}[args.routed_fmt]
        spec = synth.scaled_spec(E=spec.E, k=spec.k, d=spec.d, f=spec.f, fmt_gate_up=fr, fmt_down=fr)
    E, k, d, f = spec.E, spec.k, spec.d, spec.f
    FGU, FDN = spec.fmt_gate_up, spec.fmt_down
    headline = args.routed_fmt == "iq2-q2k" and not args.bias_gain

    def traffic(kernel):  # counters were taken on the headline configuration
        return measured_traffic(kernel) if headline else None

    result = {}
    if "probes" in want and not args.pmc_mode:
        result["probes"] = run_probes(torch, dev, timer)
    probes = result.get("probes", {})
    probe_small = probes.get("read_44MB", {}).get("GBs")
    probe_big = probes.get("read_2750MB", {}).get("GBs")
    probe_mfma = probes.get("mfma_f16_16x16x32", {}).get("TFLOPs")

    # ------------------------------------------------------------ layers ----
    t0 = time.time()
    L = synth.random_layer(spec, seed=0, workload="decode")
    base = lib.DeviceLayer.from_synth(L, dev)
    routed_copies = [base.tensors]
    second = {n: base.tensors[n].clone() for n in ("w_gate", "w_up", "w_down")}
    routed_copies.append(second)
    descs, keep = [], []
    for i in range(N_DESC):
        wr = torch.from_numpy(synth.router_weights(0, ("bench", i, "router"), E, d)).to(dev)
        sh = {}
        for name, rows, K in (("s_gate", f, d), ("s_up", f, d), ("s_down", d, f)):
            canon = torch.from_numpy(synth.random_matrix(0, ("bench", i, name), synth.FMT_Q8, rows, K)).to(dev)
            sh[name] = torch.empty_like(canon)
            lib.repack(synth.FMT_Q8, 1, rows, K, canon, sh[name])
        rc = routed_copies[i % 2]
        desc = lib.MoeLayer.from_buffer_copy(base.desc)
        desc.w_gate, desc.w_up, desc.w_down = rc["w_gate"].data_ptr(), rc["w_up"].data_ptr(), rc["w_down"].data_ptr()
        desc.w_router = wr.data_ptr()
        desc.s_gate, desc.s_up, desc.s_down = (sh[n].data_ptr() for n in ("s_gate", "s_up", "s_down"))
        extra = ()
        if args.bias_gain:
            rng = np.random.default_rng(1000 + i)
            bias = torch.from_numpy(rng.normal(0, 0.05, E).astype(np.float32)).to(dev)
            gain = torch.from_numpy(rng.uniform(0.5, 1.5, (E, d)).astype(np.float32)).to(dev)
            desc.router_bias, desc.down_gain = bias.data_ptr(), gain.data_ptr()
            extra = (bias, gain)
        descs.append(desc)
        keep.append((wr, sh) + extra)
    torch.cuda.synchronize()
    log(f"layers ready in {time.time() - t0:.1f}s (routed copies: 2 x {sum(t.numel() for t in second.values())/1e9:.2f} GB)")

    gu_mat = lib.matrix_bytes(FGU, 1, f, d)
    dn_mat = lib.matrix_bytes(FDN, 1, d, f)
    q8_gu = lib.matrix_bytes(synth.FMT_Q8, 1, f, d)
    q8_dn = lib.matrix_bytes(synth.FMT_Q8, 1, d, f)
    expert_b = 2 * gu_mat + dn_mat
    shared_b = 2 * q8_gu + q8_dn

    def to_bf16(x):
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    def profile(fn, n):
        lib.profile_reset()
        lib.profile_enable(True)
        for i in range(n):
            fn(i)
        torch.cuda.synchronize()
        prof = lib.profile_collect()
        lib.profile_enable(False)
        lib.profile_reset()
        return {name: {"avg_us": round(ms / cnt * 1000, 3), "launches": cnt} for name, (cnt, ms) in prof.items()}

    if args.pmc_mode:
        # decode steps, prefill steps, then the calibration copy (each kernel
        # is one dispatch record in the counter runs)
        xs = torch.from_numpy(synth.activations(0, ("bench", "decode-x"), N_DESC, d, synth.F32)).to(dev)
        ys = torch.empty(N_DESC, d, dtype=torch.float32, device=dev)
        ws = base.workspace(1)
        for i in range(8):
            lib.layer_forward(descs[i], xs[i:i + 1], ys[i:i + 1], ws)
        T = 1024
        xp = to_bf16(synth.activations(0, ("bench", "prefill-x", 0), T, d, synth.BF16))
        yp = torch.empty(T, d, dtype=torch.float32, device=dev)
        wsp = base.workspace(T)
        for i in range(2):
            lib.layer_forward(descs[i], xp, yp, wsp)
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"pmc mode done ({COPY_BYTES} B calibration copy x4)")
        return 0

    # ------------------------------------------------------------ decode ----
    # one token: router + x in the first launch, the routed and the shared
    # gate/up in the second, all down projections in the third
    bytes_k1 = E * d * 4 + d * 4
    bytes_k2 = k * 2 * gu_mat + 2 * q8_gu
    bytes_k3 = k * dn_mat + q8_dn + d * 4
    decode_bytes = bytes_k1 + bytes_k2 + bytes_k3
    decode_kernels = {"decode_router": bytes_k1, "decode_gateup": bytes_k2, "decode_down_combine": bytes_k3}
    if "decode" in want:
        xs = torch.from_numpy(synth.activations(0, ("bench", "decode-x"), N_DESC, d, synth.F32)).to(dev)
        ys = torch.empty(N_DESC, d, dtype=torch.float32, device=dev)
        ws = base.workspace(1)

        def step(i):
            j = i % N_DESC
            lib.layer_forward(descs[j], xs[j:j + 1], ys[j:j + 1], ws)

        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        # graph of one cycle of descriptors
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        with torch.cuda.graph(g, stream=cap):
            for i in range(N_DESC):
                step(i)
        g.replay()
        torch.cuda.synchronize()
        K = args.steps
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        ev0.record()
        for _ in range(K // N_DESC):
            g.replay()
        for i in range(K % N_DESC):
            step(i)
        ev1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        ms_step = ev0.elapsed_time(ev1) / K
        log(f"decode: {K} steps, {ms_step * 1000:.2f} us/step (wall {wall * 1e3 / K * 1000:.2f} us/step)")
        # spread: each graph replay (16 steps) timed on its own
        per_replay = timer(lambda i: g.replay(), max(16, K // (4 * N_DESC)))
        spread_us = pct(np.asarray(per_replay) * 1000.0 / N_DESC)
        del g

        prof = profile(step, args.profile_steps)
        kern = {}
        for name, nbytes in decode_kernels.items():
            if name not in prof:  # (a library build without that launch)
                continue
            avg_us = prof[name]["avg_us"]
            kern[name] = {"avg_us": avg_us, "launches": prof[name]["launches"], "algorithmic_bytes": nbytes,
                          "achieved_GBs": round(nbytes / (avg_us * 1e-6) / 1e9, 1)}
        dominant = max(kern, key=lambda n: kern[n]["avg_us"])
        dk = kern[dominant]
        result["decode"] = {
            "ms_per_step": ms_step,
            "us_per_step_spread": spread_us,
            "tokens_per_s": 1000.0 / ms_step,
            "algorithmic_bytes_per_step": decode_bytes,
            "achieved_GBs_whole_step": decode_bytes / (ms_step * 1e-3) / 1e9,
            "kernels": kern,
            "roofline": {"kernel": dominant, "bound": "hbm", "achieved": dk["achieved_GBs"], "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", **frac_pair(dk["achieved_GBs"], HBM_PEAK_GBS, probe_small),
                         "probe_peak": probe_small, "traffic": traffic(dominant)},
        }

    # ----------------------------------------------------------- prefill ----
    if "prefill" in want:
        T = 1024
        xp = [to_bf16(synth.activations(0, ("bench", "prefill-x", i), T, d, synth.BF16)) for i in range(2)]
        yp = torch.empty(T, d, dtype=torch.float32, device=dev)
        idx = torch.empty(T, k, dtype=torch.int32, device=dev)
        wsp = base.workspace(T)

        def pstep(i):
            lib.layer_forward(descs[i % N_DESC], xp[i % 2], yp, wsp, idx_out=idx)

        for i in range(3):
            pstep(i)
        torch.cuda.synchronize()
        P = args.prefill_steps
        ms_list = timer(pstep, P)
        ms_p = float(np.mean(ms_list))
        uniq = int(torch.unique(idx).numel())
        p_bytes = uniq * expert_b + shared_b + E * d * 4 + T * d * 2 + T * d * 4
        flops = 2.0 * T * (k + 1) * 3 * f * d
        log(f"prefill: {P} steps, {ms_p:.3f} ms/step, {uniq} experts touched")
        pk = profile(pstep, 8)
        gu_b = uniq * 2 * gu_mat + T * d * 2
        dn_b = uniq * dn_mat
        for name, nb, fl in (("prefill_gateup", gu_b, 2.0 * T * k * 2 * f * d),
                             ("prefill_down", dn_b, 2.0 * T * k * f * d),
                             ("prefill_shared_gateup", 2 * q8_gu, 2.0 * T * 2 * f * d),
                             ("prefill_shared_down", q8_dn, 2.0 * T * f * d)):
            us = pk[name]["avg_us"]
            pk[name]["algorithmic_bytes"] = nb
            pk[name]["achieved_GBs"] = round(nb / (us * 1e-6) / 1e9, 1)
            pk[name]["mfma_TFLOPs"] = round(fl / (us * 1e-6) / 1e12, 1)
            pk[name]["mfma_frac"] = round(fl / (us * 1e-6) / 1e12 / F16_PEAK_TFLOPS, 4)
        pdom = max(("prefill_gateup", "prefill_down"), key=lambda n: pk[n]["avg_us"])
        result["prefill"] = {
            "ms_per_step": ms_p,
            "ms_per_step_spread": pct(ms_list),
            "tokens_per_s": T / (ms_p * 1e-3),
            "experts_touched": uniq,
            "algorithmic_bytes_per_step": p_bytes,
            "achieved_GBs_whole_step": p_bytes / (ms_p * 1e-3) / 1e9,
            "mfma_TFLOPs_whole_step": flops / (ms_p * 1e-3) / 1e12,
            "mfma_frac_of_f16_peak": flops / (ms_p * 1e-3) / 1e12 / F16_PEAK_TFLOPS,
            "kernels": pk,
            "roofline": {"kernel": pdom, "bound": "hbm", "achieved": pk[pdom]["achieved_GBs"], "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", **frac_pair(pk[pdom]["achieved_GBs"], HBM_PEAK_GBS, probe_big),
                         "probe_peak": probe_big, "traffic": traffic(pdom)},
        }

    # --------------------------------- small batch and the T crossover ----
    def both_paths(T, x_host, idx_h, wt_h, reps):
        """Caller routes on both paths: decode in calls of at most 8 tokens,
        prefill in one call; cycling over the descriptors (cold HBM)."""
        x = torch.from_numpy(x_host).to(dev)
        it = torch.from_numpy(idx_h).to(dev)
        wt = torch.from_numpy(wt_h).to(dev)
        y = torch.empty(T, d, dtype=torch.float32, device=dev)
        wsd = base.workspace(min(T, lib.MOE_DECODE_MAX_T), lib.MOE_OP_DECODE)
        wsp = base.workspace(T, lib.MOE_OP_PREFILL)
        chunks = [(a, min(T, a + lib.MOE_DECODE_MAX_T)) for a in range(0, T, lib.MOE_DECODE_MAX_T)]

        def dec(i):
            for a, b in chunks:
                lib.expert_ffn_decode(descs[i % N_DESC], x[a:b], it[a:b], wt[a:b], y[a:b], wsd)

        def pre(i):
            lib.expert_ffn_prefill(descs[i % N_DESC], x, it, wt, y, wsp)
        dec(0)
        pre(0)
        torch.cuda.synchronize()
        return float(np.median(timer(dec, reps))) * 1000.0, float(np.median(timer(pre, reps))) * 1000.0

    if "small-batch" in want:
        T = 16
        idx_h, wt_h = synth.session_routes(0)
        x_h = synth.activations(0, ("bench", "small_batch"), T, d, synth.F32)
        dec_us, pre_us = both_paths(T, x_h, idx_h, wt_h, 64)
        U = int(np.unique(idx_h).size)
        sb_bytes = U * expert_b + shared_b + T * d * 8
        result["small_batch_16"] = {
            "tokens": T, "sessions": 4, "unique_experts": U, "algorithmic_bytes": sb_bytes,
            "decode_path": {"us": round(dec_us, 2), "tokens_per_s": round(T / (dec_us * 1e-6), 1),
                            "achieved_GBs": round(sb_bytes / (dec_us * 1e-6) / 1e9, 1), "calls": 2},
            "prefill_path": {"us": round(pre_us, 2), "tokens_per_s": round(T / (pre_us * 1e-6), 1),
                             "achieved_GBs": round(sb_bytes / (pre_us * 1e-6) / 1e9, 1), "calls": 1},
        }
        log(f"small batch 16: decode {dec_us:.1f} us, prefill {pre_us:.1f} us, {U} unique experts")

    if "crossover" in want:
        rows = {}
        for T in (1, 2, 4, 8, 16, 24, 32, 64, 128):
            idx_h, wt_h = synth.session_routes(0, sessions=max(1, T // 4) if T >= 4 else T, steps=min(4, T) if T >= 4
                                               else 1, tag=f"sweep{T}")
            x_h = synth.activations(0, ("bench", "sweep", T), T, d, synth.F32)
            dec_us, pre_us = both_paths(T, x_h, idx_h, wt_h, 32)
            rows[str(T)] = {"decode_us": round(dec_us, 2), "prefill_us": round(pre_us, 2),
                            "unique_experts": int(np.unique(idx_h).size)}
        faster = [int(t) for t, r in rows.items() if r["decode_us"] <= r["prefill_us"]]
        result["crossover"] = {"by_T": rows, "decode_faster_up_to_T": max(faster) if faster else 0,
                               "routes": "session generator (4 consecutive tokens per session)",
                               "library_auto_decode_max_T": lib.MOE_AUTO_DECODE_MAX_T}
        log(f"crossover: {rows}")

    # ------------------------------------------------------ long prefill ----
    if "long-prefill" in want:
        T, NL = 4096, synth.LONG_PREFILL_LAYERS
        xs_l, idx_l, wt_l, uniq_l = [], [], [], []
        for layer in range(NL):
            idx_h, wt_h = synth.zipf_routes(0, T, layer=layer)
            xs_l.append(to_bf16(synth.activations(0, ("bench", "long_prefill", layer), T, d, synth.BF16)))
            idx_l.append(torch.from_numpy(idx_h).to(dev))
            wt_l.append(torch.from_numpy(wt_h).to(dev))
            uniq_l.append(int(np.unique(idx_h).size))
        y = torch.empty(T, d, dtype=torch.float32, device=dev)
        wsp = base.workspace(T, lib.MOE_OP_PREFILL)

        def lstep(i):  # one pass through the 8 layers
            for layer in range(NL):
                lib.expert_ffn_prefill(descs[layer], xs_l[layer], idx_l[layer], wt_l[layer], y, wsp)
        lstep(0)
        torch.cuda.synchronize()
        ms_list = timer(lstep, args.long_prefill_steps)
        ms_pass = float(np.median(ms_list))
        lk = profile(lambda i: lstep(i), 1)
        flops_gu = 2.0 * T * k * 2 * f * d
        flops_dn = 2.0 * T * k * f * d
        per_layer_ms = ms_pass / NL
        gu_bytes = float(np.mean(uniq_l)) * 2 * gu_mat + T * d * 2
        dn_bytes = float(np.mean(uniq_l)) * dn_mat
        for name, fl, nb in (("prefill_gateup", flops_gu, gu_bytes), ("prefill_down", flops_dn, dn_bytes),
                             ("prefill_shared_gateup", 2.0 * T * 2 * f * d, 2 * q8_gu),
                             ("prefill_shared_down", 2.0 * T * f * d, q8_dn)):
            us = lk[name]["avg_us"]
            tf = fl / (us * 1e-6) / 1e12
            gbs = nb / (us * 1e-6) / 1e9
            lk[name].update({"mfma_TFLOPs": round(tf, 1), "algorithmic_bytes": round(nb),
                             "mfma": frac_pair(tf, F16_PEAK_TFLOPS, probe_mfma),
                             "hbm": frac_pair(gbs, HBM_PEAK_GBS, probe_big)})
        routed_us = lk["prefill_gateup"]["avg_us"] + lk["prefill_down"]["avg_us"]
        routed_tf = (flops_gu + flops_dn) / (routed_us * 1e-6) / 1e12
        all_flops = 2.0 * T * (k + 1) * 3 * f * d
        result["long_prefill"] = {
            "layers": NL, "tokens": T, "routes": "Zipf(1.1), caller supplied",
            "ms_per_pass": round(ms_pass, 4), "ms_per_pass_spread": pct(ms_list),
            "ms_per_layer": round(per_layer_ms, 4),
            "tokens_per_s_per_layer": round(T / (per_layer_ms * 1e-3), 1),
            "tokens_per_s_through_all_layers": round(T / (ms_pass * 1e-3), 1),
            "unique_experts_mean": float(np.mean(uniq_l)),
            "mfma_TFLOPs_whole_layer": round(all_flops / (per_layer_ms * 1e-3) / 1e12, 1),
            "routed_gemms": {"TFLOPs": round(routed_tf, 1), **frac_pair(routed_tf, F16_PEAK_TFLOPS, probe_mfma)},
            "kernels": lk,
        }
        log(f"long prefill: {ms_pass:.2f} ms per 8-layer pass, routed GEMMs {routed_tf:.0f} TFLOP/s")

    # ------------------------------------------------------ CPU baseline ----
    cpu = None
    if not args.no_cpu_baseline and "decode" in want:
        import oracle

        oracle.set_threads(len(os.sched_getaffinity(0)))
        threads = oracle.threads()
        xs_h = synth.activations(0, ("bench", "cpu-x"), 1024, d, synth.F32)
        t0 = time.perf_counter()
        n = 0
        while n < xs_h.shape[0]:
            oracle.layer_forward(L, xs_h[n:n + 1], synth.F32)
            n += 1
            if time.perf_counter() - t0 > 10.0:
                break
        el = time.perf_counter() - t0
        oracle.set_threads(1)
        t1 = time.perf_counter()
        n1 = 0
        while n1 < 4:
            oracle.layer_forward(L, xs_h[n1:n1 + 1], synth.F32)
            n1 += 1
            if time.perf_counter() - t1 > 4.0:
                break
        el1 = time.perf_counter() - t1
        oracle.set_threads(threads)
        # prefill: the oracle's expert-grouped evaluation on 48 tokens of a 1024-token chunk
        xp_h = synth.activations(0, ("bench", "prefill-x", 0), 1024, d, synth.BF16)
        tok = np.arange(0, 1024, 1024 // 48)[:48]
        t2 = time.perf_counter()
        _, pidx, pwt = oracle.route(xp_h[tok], oracle.BF16, L.w_router, k)
        oracle.ffn(L, xp_h[tok], oracle.BF16, pidx, pwt, grouped=True)
        el2 = time.perf_counter() - t2
        cpu = {"value": round(n / el, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"{n} single-token decode steps of the same layer (router + top-6 + 6 experts + shared "
                         f"expert, fp64 FFN) on {threads} threads, {el:.1f} s",
               "cpu": cpu_model(),
               "single_thread": {"value": round(n1 / el1, 4), "unit": "tokens/s",
                                 "sample": f"{n1} decode steps on 1 thread, {el1:.1f} s"},
               "prefill": {"value": round(len(tok) / el2, 3), "unit": "tokens/s",
                           "sample": f"{len(tok)} tokens of the 1024-token chunk, expert-grouped oracle, "
                                     f"{threads} threads, {el2:.1f} s"}}
        log(f"cpu oracle: {n} tokens in {el:.1f}s on {threads} threads; 1 thread {n1 / el1:.2f} tok/s; "
            f"prefill {len(tok) / el2:.2f} tok/s")

    # -------------------------------------------------------------- line ----
    dec = result.get("decode")
    line = {
        "metric": METRIC,
        "value": round(dec["tokens_per_s"], 1) if dec else None,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 6) if dec else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp32 activations x E4M3 codewords (routed), i16-fixed-point x i8 (shared)"
                  if args.routed_fmt in ("vq12", "vq13")
                  else "i16-fixed-point x i2/i8 integer dot products, fp32 scales"),
        "data": "synthetic",
        "config": {"workload": "decode: one MoE layer, 384 experts, top-6, d=4096, f=2048, shared Q8_0-like "
                               "expert, " + {"iq2-q2k": "IQ2_XXS-like gate/up, Q2_K-like down",
                                             "q4k": "Q4_K-like gate/up and down",
                                             "mxfp4": "MXFP4 gate/up and down",
                                             "vq12": "VQ 12-bit codeword indices gate/up and down",
                                             "vq13": "VQ 13-bit codeword indices gate/up and down"}[args.routed_fmt]
                               + ", T=1 fp32 token",
                   "routed_formats": args.routed_fmt,
                   "layer_descriptors": N_DESC, "routed_copies": 2, "graph_steps": N_DESC,
                   "router_bias_and_down_gains": bool(args.bias_gain)},
        "roofline": dec["roofline"] if dec else None,
        "cpu_baseline": cpu,
        "decode": dec,
        "prefill_1024": result.get("prefill"),
        "small_batch_16": result.get("small_batch_16"),
        "crossover": result.get("crossover"),
        "long_prefill": result.get("long_prefill"),
        "probes": result.get("probes"),
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
