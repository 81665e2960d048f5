#!/usr/bin/env python3
"""Throughput of the timestep-adaptive-bit linear stack on one MI355X.

One bench step is one pass of a whole denoising schedule through the hot
path: for every denoising step t and every linear l of the stack, the
per-token activation quantizer (block FWHT + absmax INT8, or MXFP4) and the
GEMM at that (t, l)'s precision (TASQ LSB mask k, or MXFP4), driven by the
library's native schedule runner.  Inputs are seeded synthetic tensors of the
workload's shapes, resident in HBM before timing starts.

Default workload: the PixArt-Sigma-shaped stack (28 blocks, hidden 1152,
4096 tokens, 20 steps, QKV / out / MLP-up / MLP-down), masked INT8 path.

Prints one JSON line.  `value` is masked-GEMM work (2*M*N*K per layer-step,
summed over the schedule) divided by the wall time of the schedule, quantizer
and launch gaps included.  `roofline` is the GEMM kernel alone, timed with HIP
events recorded on the launch stream around every GEMM of the timed region.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0     # MI355X dense INT8 MFMA (5.0 POPS)
MXFP4_PEAK_TOPS = 10100.0   # MI355X dense MXFP4 (10.1 PFLOP/s)
HBM_PEAK_GBS = 8000.0


class Hip:
    """Minimal HIP runtime access for events (measurement plumbing only)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n: int):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if self.lib.hipEventCreateWithFlags(ctypes.byref(h), 0) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            arr[i] = h
        return arr

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, arr):
        for h in arr:
            self.lib.hipEventDestroy(h)


def cpu_baseline(wl, rows: int):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    from oracle import tabit_oracle as O
    import tabit_synth as S
    seen = {}
    for li, layer in enumerate(wl.layers):
        key = (layer.M, layer.N, layer.K, int(wl.fmt[0, li]))
        seen.setdefault(key, (li, layer))
    total_ops, total_s = 0, 0.0
    parts = []
    for (M, N, K, fmt), (li, layer) in seen.items():
        r = min(rows, M)
        x = S.gen_activation(M, K, seed=S.activation_seed(0, K))[:r]
        w = S.gen_weight(N, K, seed=li)
        xb, wb = S.bf16_bits(x), S.bf16_bits(w)
        if fmt == 0:
            wq, sw = O.quantize_weights_int8(wb, wl.had_block)        # offline prep, untimed
            t0 = time.perf_counter()
            xq, sa = O.quantize_act_int8(xb, wl.had_block)
            acc = O.masked_gemm_i32(xq, wq, int(wl.k_bits[0, li]))
            O.dequant(acc, sa, sw)
            dt = time.perf_counter() - t0
        else:
            wf, we = O.mx_quantize_rows(O.bf16_to_f32(wb), wl.had_block)
            t0 = time.perf_counter()
            xf, xe = O.mx_quantize_rows(O.bf16_to_f32(xb), wl.had_block)
            O.mxfp4_gemm(xf, xe, wf, we, 1.0 / max(wl.had_block, 1))
            dt = time.perf_counter() - t0
        total_ops += 2 * r * N * K
        total_s += dt
        parts.append(f"{r}x{N}x{K}")
    return {
        "value": total_ops / total_s / 1e12,
        "unit": "TOPS",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{rows} token rows of step 0 of each distinct linear shape "
                   f"({', '.join(parts)}): oracle quantizer + GEMM + dequant, "
                   f"{total_ops / 1e9:.1f} GOP in {total_s:.1f} s; numpy, single thread"),
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5, help="timed schedule passes")
    ap.add_argument("--warmup", type=int, default=2, help="untimed schedule passes")
    ap.add_argument("--workload", default="c2", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--path", default="masked", choices=["masked", "bitserial"])
    ap.add_argument("--had-block", type=int, default=None, help="override the workload's block")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=512)
    ap.add_argument("--no-events", action="store_true", help="skip per-GEMM event timing")
    ap.add_argument("--no-tune", action="store_true", help="skip the warm-up tile autotuning")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: the linear shards by tokens with no communication, "
              "so this build runs and reports the single-GPU share only (--gpus 1).",
              file=sys.stderr)
        return 2

    import torch
    import tabit_synth as S
    import timestep_adaptive_bit_amd as T

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = S.WORKLOADS[args.workload]() if args.had_block is None else \
        S.WORKLOADS[args.workload](had_block=args.had_block)
    b = wl.had_block
    L, Tn = wl.num_layers, wl.steps
    ctx = T.Context()
    ctx.set_step_schedule(wl.k_bits, wl.fmt)
    path = T.PATH_BITSERIAL if args.path == "bitserial" else T.PATH_MASKED

    # ---- weights: one shared INT8 buffer per layer (+ MX copy where scheduled)
    weights = []
    for li, layer in enumerate(wl.layers):
        w = S.gen_weight(layer.N, layer.K, seed=li).to(dev)
        needs_mx = bool(wl.fmt[:, li].any())
        needs_i8 = bool((wl.fmt[:, li] == 0).any())
        weights.append(ctx.quantize_weights(w, b, int8=needs_i8, mx=needs_mx))
        del w
    # ---- activations: one per distinct (M, K) per step; outputs: one per layer
    xs = {}
    for t in range(Tn):
        for layer in wl.layers:
            key = (t, layer.M, layer.K)
            if key not in xs:
                xs[key] = S.gen_activation(layer.M, layer.K, seed=S.activation_seed(t, layer.K)).to(dev)
    ys = [torch.empty((l.M, l.N), dtype=torch.bfloat16, device=dev) for l in wl.layers]
    ws_bytes = max(T.act_workspace_bytes(l.M, l.K) for l in wl.layers)
    act_ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    layers = (T.Layer * L)()
    for li, (layer, wt) in enumerate(zip(wl.layers, weights)):
        layers[li].M, layers[li].N, layers[li].K = layer.M, layer.N, layer.K
        layers[li].w_q = wt["w_q"].data_ptr() if "w_q" in wt else None
        layers[li].w_scale = wt["w_scale"].data_ptr() if "w_scale" in wt else None
        layers[li].w_fp4 = wt["w_fp4"].data_ptr() if "w_fp4" in wt else None
        layers[li].w_e8m0 = wt["w_e8m0"].data_ptr() if "w_e8m0" in wt else None
        layers[li].y_bf16 = ys[li].data_ptr()
    x_ptrs = (ctypes.c_void_p * (Tn * L))()
    for t in range(Tn):
        for li, layer in enumerate(wl.layers):
            x_ptrs[t * L + li] = xs[(t, layer.M, layer.K)].data_ptr()

    # ---- warm-up tuning: time every tile configuration once per distinct GEMM shape
    tuned = {}
    if not args.no_tune:
        for li, layer in enumerate(wl.layers):
            for fmt in sorted(set(int(f) for f in wl.fmt[:, li])):
                key = (fmt, layer.M, layer.N, layer.K)
                if key in tuned:
                    continue
                x = xs[(0, layer.M, layer.K)]
                if fmt == 0:
                    xq, xs_ = ctx.hadamard_quant_act(x, b, T.FMT_INT8)
                    tuned[key] = ctx.autotune_gemm(path, xq, xs_, weights[li]["w_q"],
                                                   weights[li]["w_scale"], layer.M, layer.N,
                                                   layer.K, 2, ys[li], reps=3)
                else:
                    xf, xe = ctx.hadamard_quant_act(x, b, T.FMT_MXFP4)
                    tuned[key] = ctx.autotune_gemm(T.PATH_MXFP4_GEMM, xf, xe, weights[li]["w_fp4"],
                                                   weights[li]["w_e8m0"], layer.M, layer.N,
                                                   layer.K, 0, ys[li], reps=3)
                del x
        torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev).cuda_stream
    hip = Hip()

    def one_pass(events=None):
        ctx.run_schedule(0, Tn, layers, x_ptrs, b, act_ws, path=path, gemm_events=events,
                         stream=stream)

    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()

    ev_sets = [] if args.no_events else [hip.events(2 * Tn * L) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        one_pass(None if args.no_events else ev_sets[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # ---- work accounting
    int8_ops = mx_ops = 0
    gemm_bytes = 0
    for t in range(Tn):
        for li, layer in enumerate(wl.layers):
            ops = 2 * layer.M * layer.N * layer.K
            if wl.fmt[t, li] == 0:
                int8_ops += ops
            else:
                mx_ops += ops
    total_ops = int8_ops + mx_ops
    value = total_ops / (ms_per_step / 1e3) / 1e12

    roofline = None
    detail = {}
    if not args.no_events:
        gemm_ms_i8 = gemm_ms_mx = 0.0
        n_i8 = n_mx = 0
        for s in range(args.steps):
            ev = ev_sets[s]
            for t in range(Tn):
                for li in range(L):
                    i = t * L + li
                    ms = hip.elapsed_ms(ev[2 * i], ev[2 * i + 1])
                    if wl.fmt[t, li] == 0:
                        gemm_ms_i8 += ms
                        n_i8 += 1
                    else:
                        gemm_ms_mx += ms
                        n_mx += 1
        for e in ev_sets:
            hip.destroy(e)
        if n_i8:
            achieved = (int8_ops * args.steps) / (gemm_ms_i8 / 1e3) / 1e12
            roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": INT8_PEAK_TOPS,
                        "unit": "TOPS", "frac": round(achieved / INT8_PEAK_TOPS, 4), "traffic": None,
                        "kernel": "gemm_i8_kernel (masked)" if path == T.PATH_MASKED
                        else "gemm_i8_kernel (bitserial)",
                        "avg_launch_us": round(gemm_ms_i8 * 1e3 / n_i8, 3)}
            detail["gemm_int8_ms_per_step"] = round(gemm_ms_i8 / args.steps, 3)
        if n_mx:
            mx_tops = (mx_ops * args.steps) / (gemm_ms_mx / 1e3) / 1e12
            detail["gemm_mxfp4_tops"] = round(mx_tops, 2)
            detail["gemm_mxfp4_frac_of_peak"] = round(mx_tops / MXFP4_PEAK_TOPS, 4)
            detail["gemm_mxfp4_ms_per_step"] = round(gemm_ms_mx / args.steps, 3)
            if roofline is None:
                roofline = {"bound": "mfma", "achieved": round(mx_tops, 2), "peak": MXFP4_PEAK_TOPS,
                            "unit": "TFLOP/s", "frac": round(mx_tops / MXFP4_PEAK_TOPS, 4),
                            "traffic": None, "kernel": "gemm_mxfp4_kernel",
                            "avg_launch_us": round(gemm_ms_mx * 1e3 / n_mx, 3)}

    out = {
        "metric": "masked W8A8 GEMM TOPS and % of INT8 MFMA peak per denoising schedule",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8" if mx_ops == 0 else "i8+mxfp4",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": L, "denoise_steps": Tn,
                   "tokens": sorted({l.M for l in wl.layers}), "had_block": b,
                   "path": args.path, "step": "one full denoising schedule (quantizer + GEMM per layer-step)",
                   "int8_layer_steps": int((wl.fmt == 0).sum()), "mxfp4_layer_steps": int((wl.fmt == 1).sum())},
        "frac_of_int8_peak": round(value / INT8_PEAK_TOPS, 4),
        "roofline": roofline,
        "detail": detail,
        "tuned_tiles": {f"{'mxfp4' if k[0] else 'int8'} {k[1]}x{k[2]}x{k[3]}": T.gemm_config_info(v)[:2]
                        if k[0] == 0 else v for k, v in tuned.items()},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_rows)
    print(json.dumps(out), flush=True)
    ctx.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
