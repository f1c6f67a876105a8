"""Benchmark of the routed-expert MoE layer on one MI355X.

One step = one pass of the whole layer (router, exact top-6, expert FFNs with
the shared expert, combine) over one batch of synthetic input with every
input already resident in HBM.

  value          single-token decode: 384 experts, top-6, d=4096, f=2048, a
                 Q8 shared expert, IQ2 gate/up, Q2K down, fp32 x -- tokens/s
                 of one layer (steps/s at T=1)
  prefill_1024   the same layer on 1024-token bf16 chunks (second figure)

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
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
N_DESC = 16  # layer descriptors (router + shared expert sets) cycled by the steps
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


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


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=4000, help="timed decode steps")
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--prefill-steps", type=int, default=40)
    ap.add_argument("--profile-steps", type=int, default=256, help="eager steps with per-kernel events")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bias-gain", action="store_true",
                    help="give every layer a router selection bias and per-channel down gains (not the headline)")
    ap.add_argument("--routed-fmt", choices=["iq2-q2k", "q4k"], default="iq2-q2k",
                    help="routed experts: IQ2_XXS-like gate/up + Q2_K-like down (the headline), or Q4_K-like "
                         "gate/up/down (the 4-bit variant; not the headline)")
    ap.add_argument("--only", choices=["all", "decode", "prefill"], default="all")
    ap.add_argument("--pmc-mode", action="store_true",
                    help="no timing: a few decode and prefill steps and a plain copy of known size, for "
                         "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs")
    ap.add_argument("--pmc-summarize", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn the two counter runs into profiles/traffic_counters.json (no GPU)")
    args = ap.parse_args()

    if args.pmc_summarize:
        return pmc_summarize(*args.pmc_summarize)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (expert-parallel sharding is "
              "designed, not built). Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch

    from quantized_moe_amd import lib, synth

    lib.lib()  # fails loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    spec = synth.DECODE_SPEC
    if args.routed_fmt == "q4k":
        spec = synth.scaled_spec(E=spec.E, k=spec.k, d=spec.d, f=spec.f, fmt_gate_up=synth.FMT_Q4K,
                                 fmt_down=synth.FMT_Q4K)
    E, k, d, f = spec.E, spec.k, spec.d, spec.f
    FGU, FDN = spec.fmt_gate_up, spec.fmt_down
    headline = args.routed_fmt == "iq2-q2k" and not args.bias_gain

    def traffic(kernel):  # counters were taken on the headline configuration
        return measured_traffic(kernel) if headline else None

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

    result = {}

    if args.pmc_mode:
        # decode steps, prefill steps, then the calibration copy (each kernel
        # is one dispatch record in the counter runs)
        xs = torch.from_numpy(synth.activations(0, ("bench", "decode-x"), N_DESC, d, synth.F32)).to(dev)
        ys = torch.empty(N_DESC, d, dtype=torch.float32, device=dev)
        ws = base.workspace(1)
        for i in range(8):
            lib.layer_forward(descs[i], xs[i:i + 1], ys[i:i + 1], ws)
        T = 1024
        xp = torch.from_numpy(synth.activations(0, ("bench", "prefill-x", 0), T, d, synth.BF16).view(np.int16)) \
            .to(dev).view(torch.bfloat16)
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
    bytes_k2 = k * 2 * lib.matrix_bytes(FGU, 1, f, d) + 2 * lib.matrix_bytes(synth.FMT_Q8, 1, f, d)
    bytes_k3 = k * lib.matrix_bytes(FDN, 1, d, f) + lib.matrix_bytes(synth.FMT_Q8, 1, d, f) + d * 4
    decode_bytes = bytes_k1 + bytes_k2 + bytes_k3
    decode_kernels = {"decode_router": bytes_k1, "decode_gateup": bytes_k2, "decode_down_combine": bytes_k3}
    if args.only in ("all", "decode"):
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

        # per-kernel durations (eager, events on the launch stream)
        lib.profile_reset()
        lib.profile_enable(True)
        for i in range(args.profile_steps):
            step(i)
        torch.cuda.synchronize()
        prof = lib.profile_collect()
        lib.profile_enable(False)
        lib.profile_reset()
        kern = {}
        for name, nbytes in decode_kernels.items():
            n, ms = prof[name]
            avg_us = ms / n * 1000
            kern[name] = {"avg_us": round(avg_us, 3), "launches": n, "algorithmic_bytes": nbytes,
                          "achieved_GBs": round(nbytes / (avg_us * 1e-6) / 1e9, 1)}
        dominant = max(kern, key=lambda n: kern[n]["avg_us"])
        dk = kern[dominant]
        dom_traffic = traffic(dominant)
        result["decode"] = {
            "ms_per_step": ms_step,
            "tokens_per_s": 1000.0 / ms_step,
            "algorithmic_bytes_per_step": decode_bytes,
            "achieved_GBs_whole_step": decode_bytes / (ms_step * 1e-3) / 1e9,
            "kernels": kern,
            "roofline": {"kernel": dominant, "bound": "hbm", "achieved": dk["achieved_GBs"], "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(dk["achieved_GBs"] / HBM_PEAK_GBS, 4),
                         "traffic": dom_traffic},
        }
        # cross-check that the graph-replayed steps compute the eager result
        del g

    # ----------------------------------------------------------- prefill ----
    if args.only in ("all", "prefill"):
        T = 1024
        xp = [torch.from_numpy(synth.activations(0, ("bench", "prefill-x", i), T, d, synth.BF16).view(np.int16))
              .to(dev).view(torch.bfloat16) for i in range(2)]
        yp = torch.empty(T, d, dtype=torch.float32, device=dev)
        idx = torch.empty(T, k, dtype=torch.int32, device=dev)
        wsp = base.workspace(T)

        def pstep(i):
            lib.layer_forward(descs[i % N_DESC], xp[i % 2], yp, wsp, idx_out=idx)

        for i in range(3):
            pstep(i)
        torch.cuda.synchronize()
        P = args.prefill_steps
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for i in range(P):
            pstep(i)
        ev1.record()
        torch.cuda.synchronize()
        ms_p = ev0.elapsed_time(ev1) / P
        uniq = int(torch.unique(idx).numel())
        routed_b = uniq * (2 * lib.matrix_bytes(FGU, 1, f, d) + lib.matrix_bytes(FDN, 1, d, f))
        shared_b = 2 * lib.matrix_bytes(synth.FMT_Q8, 1, f, d) + lib.matrix_bytes(synth.FMT_Q8, 1, d, f)
        p_bytes = routed_b + shared_b + E * d * 4 + T * d * 2 + T * d * 4
        flops_routed = 2.0 * T * k * 3 * f * d
        flops_shared = 2.0 * T * 3 * f * d
        log(f"prefill: {P} steps, {ms_p:.3f} ms/step, {uniq} experts touched")
        lib.profile_reset()
        lib.profile_enable(True)
        for i in range(8):
            pstep(i)
        torch.cuda.synchronize()
        prof = lib.profile_collect()
        lib.profile_enable(False)
        lib.profile_reset()
        gu_b = uniq * 2 * lib.matrix_bytes(FGU, 1, f, d) + T * d * 2
        dn_b = uniq * lib.matrix_bytes(FDN, 1, d, f)
        pk = {}
        for name, (n, ms) in prof.items():
            pk[name] = {"avg_us": round(ms / n * 1000, 2), "launches": n}
        pk["prefill_gateup"]["algorithmic_bytes"] = gu_b
        pk["prefill_gateup"]["achieved_GBs"] = round(gu_b / (pk["prefill_gateup"]["avg_us"] * 1e-6) / 1e9, 1)
        pk["prefill_gateup"]["mfma_TFLOPs"] = round(2.0 * T * k * 2 * f * d / (pk["prefill_gateup"]["avg_us"] * 1e-6) / 1e12, 1)
        pk["prefill_down"]["algorithmic_bytes"] = dn_b
        pk["prefill_down"]["achieved_GBs"] = round(dn_b / (pk["prefill_down"]["avg_us"] * 1e-6) / 1e9, 1)
        pk["prefill_down"]["mfma_TFLOPs"] = round(2.0 * T * k * f * d / (pk["prefill_down"]["avg_us"] * 1e-6) / 1e12, 1)
        pdom = max(("prefill_gateup", "prefill_down"), key=lambda n: pk[n]["avg_us"])
        result["prefill"] = {
            "ms_per_step": ms_p,
            "tokens_per_s": T / (ms_p * 1e-3),
            "experts_touched": uniq,
            "algorithmic_bytes_per_step": p_bytes,
            "achieved_GBs_whole_step": p_bytes / (ms_p * 1e-3) / 1e9,
            "mfma_TFLOPs_whole_step": (flops_routed + flops_shared) / (ms_p * 1e-3) / 1e12,
            "mfma_frac_of_bf16_peak": (flops_routed + flops_shared) / (ms_p * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "kernels": pk,
            "roofline": {"kernel": pdom, "bound": "hbm", "achieved": pk[pdom]["achieved_GBs"], "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(pk[pdom]["achieved_GBs"] / HBM_PEAK_GBS, 4),
                         "traffic": traffic(pdom)},
        }

    # ------------------------------------------------------ CPU baseline ----
    cpu = None
    if not args.no_cpu_baseline and args.only in ("all", "decode"):
        import oracle

        threads = oracle.threads()
        xs_h = synth.activations(0, ("bench", "cpu-x"), 1024, d, synth.F32)
        t0 = time.perf_counter()
        n = 0
        while n < xs_h.shape[0]:
            oracle.layer_forward(L, xs_h[n:n + 1], synth.F32)
            n += 1
            if time.perf_counter() - t0 > 12.0:
                break
        el = time.perf_counter() - t0
        cpu = {"value": round(n / el, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"{n} single-token decode steps of the same layer (router + top-6 + 6 experts + shared "
                         f"expert, fp64 FFN) on {threads} threads, {el:.1f} s",
               "cpu": platform.processor() or platform.machine()}
        log(f"cpu oracle: {n} tokens in {el:.1f}s on {threads} threads")

    # -------------------------------------------------------------- line ----
    dec = result.get("decode")
    line = {
        "metric": "MoE layer tokens/s (decode B=1, prefill 1024) + achieved HBM GB/s / MFMA % of peak",
        "value": round(dec["tokens_per_s"], 1) if dec else None,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 6) if dec else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i16-fixed-point x i2/i8 integer dot products, fp32 scales",
        "data": "synthetic",
        "config": {"workload": "decode: one MoE layer, 384 experts, top-6, d=4096, f=2048, shared Q8_0-like "
                               "expert, " + ("IQ2_XXS-like gate/up, Q2_K-like down" if args.routed_fmt == "iq2-q2k"
                                             else "Q4_K-like gate/up and down") + ", T=1 fp32 token",
                   "routed_formats": args.routed_fmt,
                   "layer_descriptors": N_DESC, "routed_copies": 2, "graph_steps": N_DESC,
                   "router_bias_and_down_gains": bool(args.bias_gain)},
        "roofline": dec["roofline"] if dec else None,
        "cpu_baseline": cpu,
        "decode": dec,
        "prefill_1024": result.get("prefill"),
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
