#!/usr/bin/env python3
"""Throughput of one GPU's share of a tensor-parallel layer on MI355X.

Timed step: the Llama-3-70B (h=8192, F=28672) TP=8 SwiGLU MLP shard, forward
(tp_mlp_shard_fwd: [gate|up] GEMM with the SiLU*up epilogue, then the
row-parallel GEMM to the f32 partial) and backward (tp_mlp_shard_bwd: dY W_down^T
with the SwiGLU backward epilogue, dX partial, dW_gate|up, dW_down), N = 4096
tokens, bf16 inputs already resident in HBM. value = GEMM FLOPs of the step
(2164.66 GFLOP) / time, in TFLOP/s.

Also measured in the same run (reported under "rows"): every single-kernel
GEMM of the step (HIP events on the stream the kernels run on), the fused-QKV
regroup (GB/s, buffers rotated past the 256 MB Infinity Cache), the attention
projections (QKV + W_O) forward and backward at N = 4096 and decode at N = 16,
the GPT-style GeLU MLP shard (N = 8192, h = 4096, F = 16384, t = 4), and, as
context, the ROCm BLAS library (torch.matmul) on the step's GEMM shapes. The
fp64 oracle is timed on the same MLP workload (and, as legs, the GeLU shard
and the attention projections) on the host cores (cpu_baseline).

roofline: the step's dominant kernel (largest single launch), its FLOPs per
launch over its average launch time (HIP events over back-to-back launches),
against the bf16 dense peak; traffic: its HBM bytes per launch from the
committed counter summary (profiles/), if taken on the current kernel sources.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

PEAK_BF16_TFLOPS = 2516.6     # 256 CUs x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0         # HBM3E
METRIC = "TFLOP/s + % bf16 MFMA peak, Llama-3-70B TP=8 MLP shard fwd+bwd, 1 GPU"


# What each timed product launches (one gemm_kernel instantiation each).
KERNEL_DESC = {
    "gemm1_gate_up_swiglu": "gemm_kernel NN ping-pong, 256x256 tile (128 gate + 128 up columns), 8 waves, "
                            "SwiGLU epilogue",
    "gemm2_down_partial": "gemm_kernel NN ping-pong, 256x256 tile, 8 waves, fp32 store",
    "bwd_dz_swiglu": "gemm_kernel NT, 256x224 tile, 8 waves, SwiGLU backward epilogue reading H",
    "bwd_dx_partial": "gemm_kernel NT, 256x256 tile, fp32 store",
    "bwd_dw_gate_up": "gemm_kernel TN, 256x224 tile, 8 waves, fp32 store",
    "bwd_dw_down": "gemm_kernel TN, 224x256 tile, 8 waves, fp32 store",
}
TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "traffic_dominant_kernel.json")


def kernel_sources_sha() -> str:
    """Hash of the library's kernel sources (not the stand-alone probes beside
    them), to tell whether recorded counters are current."""
    import hashlib
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tensor_sharded_matmul_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".h", ".hip")) and f not in ("mfma_rate.hip", "store_rate.hip"):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def committed_traffic(product: str):
    """HBM bytes per launch of `product` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by a copy of known size), or None if
    there is none for this product or the kernel sources changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sources_sha") != kernel_sources_sha():
        return None
    return t.get("products", {}).get(product, {}).get("hbm_bytes_per_launch")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # 3000 steps: the timed region lasts about 5 s, long enough for an
    # outside sampler of GPU activity to see it (20, 2000 and 20000 steps
    # gave the same time per step, within 0.2 %)
    ap.add_argument("--steps", type=int, default=3000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--reps", type=int, default=10, help="repetitions per single-kernel timing")
    ap.add_argument("--cpu-tokens", type=int, default=4096,
                    help="tokens of the workload the oracle CPU baseline runs (0 = skip)")
    ap.add_argument("--no-rows", action="store_true", help="skip the per-row measurements")
    ap.add_argument("--data", choices=("normal", "zeros", "ints"), default="normal",
                    help="values of the step's inputs: the seeded synthetic workload (normal, the default), "
                         "all zeros, or small integers in [-2, 2]; same shapes and kernels (for the power "
                         "study: the chip's clock under the step depends on the data's switching activity)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only copy BYTES device-to-device 5 times (scale for HBM byte counters), then exit")
    ap.add_argument("--regroup-only", type=int, default=0, metavar="CALLS",
                    help="only run the fused-QKV regroup CALLS times (4 rotated sources, ranks 0..7; "
                         "for profiling), then exit")
    ap.add_argument("--attn-prefill-only", type=int, default=0, metavar="CALLS",
                    help="only run the six attention-projection products of one Llama-3-70B rank at 4096 "
                         "tokens (and the vendor BLAS on the same products and output dtypes) CALLS times (for "
                         "profiling), then exit")
    ap.add_argument("--store-rate", action="store_true",
                    help="only run the store-throughput probe (one CU's fp32 / bf16 stores) and print its records")
    ap.add_argument("--mfma-rate", action="store_true",
                    help="only run the MFMA rate probe (bf16 16x16x32 MFMAs on register operands, no memory "
                         "traffic; random and all-zero data) and print its JSON lines, then exit")
    ap.add_argument("--chunked-only", type=int, default=0, metavar="CALLS",
                    help="only run the chunked schedule on the Llama-3-70B MLP shard CALLS times: GEMM2 in 1, 2, "
                         "4 and 8 token-row chunks, dX_part in 1, 2, 4 and 8 chunks, then dX_part in 8 chunks "
                         "followed by dW_gate|up (for profiling), then exit")
    ap.add_argument("--embed-only", type=int, default=0, metavar="CALLS",
                    help="only run the vocab-parallel embedding of one Llama-3-70B rank (16128 rows, 4096 tokens) "
                         "forward and backward CALLS times, then eager torch's lookup and zeroed table + "
                         "index_add_ CALLS times (for profiling), then exit")
    ap.add_argument("--decode-only", type=int, default=0, metavar="CALLS",
                    help="only run the decode-sized (16 tokens) QKV and W_O products of the Llama-3-70B "
                         "attention shard CALLS times (16 rotated weight copies; for profiling), then exit")
    return ap.parse_args()


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the TP layer; --gpus {args.gpus} is not "
              "supported (the library computes one GPU's share of the layer and has no collectives).", file=sys.stderr)
        return 2
    import numpy as np
    import torch

    import synth
    import tensor_sharded_matmul_amd as T

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.mfma_rate:
        for r in mfma_rate():
            print(json.dumps(r), flush=True)
        return 0
    if args.store_rate:
        for r in run_probe("store_rate"):
            print(json.dumps(r), flush=True)
        return 0
    T.load()
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.empty(args.copy_calibration, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {args.copy_calibration} bytes 5 times")
        return 0
    if args.regroup_only:
        q = synth.WORKLOADS["llama70b_qkv_t8"]
        width = (q.n_h + 2 * q.n_kv) * q.d_h
        gen = torch.Generator(device=dev)
        gen.manual_seed(q.seed)
        srcs = [torch.randn((q.h, width), device=dev, generator=gen).to(torch.bfloat16) for _ in range(4)]
        dsts = [torch.empty((q.h, width // q.t), device=dev, dtype=torch.bfloat16) for _ in range(4)]
        for i in range(args.regroup_only):
            T.tp_qkv_regroup(srcs[i % 4], q.n_h, q.n_kv, q.d_h, q.t, (i // 4) % q.t, W_r=dsts[i % 4])
        torch.cuda.synchronize()
        log(f"[bench] regrouped {args.regroup_only} times")
        return 0
    if args.attn_prefill_only:
        q = synth.WORKLOADS["llama70b_qkv_t8"]
        wq, wo, Np = (q.n_h + 2 * q.n_kv) * q.d_h // q.t, q.n_h * q.d_h // q.t, 4096
        gen = torch.Generator(device=dev)
        gen.manual_seed(q.seed)
        rnd = lambda *shape: torch.randn(shape, device=dev, generator=gen).to(torch.bfloat16)  # noqa: E731
        X, Wr, O, WO, dQ, dY = rnd(Np, q.h), rnd(q.h, wq), rnd(Np, wo), rnd(wo, q.h), rnd(Np, wq), rnd(Np, q.h)
        f32 = torch.float32
        Y = torch.empty((Np, wq), device=dev, dtype=torch.bfloat16)
        P, dX = torch.empty((Np, q.h), device=dev, dtype=f32), torch.empty((Np, q.h), device=dev, dtype=f32)
        dW, dWO = torch.empty((q.h, wq), device=dev, dtype=f32), torch.empty((wo, q.h), device=dev, dtype=f32)
        dO = torch.empty((Np, wo), device=dev, dtype=torch.bfloat16)
        # the vendor BLAS on the same products and output dtypes (fp32 where
        # ours are fp32), as plain NN products of contiguous operands (the
        # transposes made beforehand)
        Wrt, Xt, WOt, Ot = Wr.t().contiguous(), X.t().contiguous(), WO.t().contiguous(), O.t().contiguous()
        mm32, _ = mm_fp32_out(torch)
        vend = ((torch.mm, X, Wr), (mm32, O, WO), (mm32, dQ, Wrt), (mm32, Xt, dQ), (torch.mm, dY, WOt),
                (mm32, Ot, dY))
        for _ in range(args.attn_prefill_only):
            T.tp_col_linear(X, Wr, "none", Y=Y)
            T.tp_row_linear_partial(O, WO, P=P)
            T.tp_col_linear_bwd(X, Wr, dQ, dX_part=dX, dW=dW)
            T.tp_row_linear_bwd(O, WO, dY, dZ=dO, dW=dWO)
            for mm_, a_, b_ in vend:
                mm_(a_, b_)
        torch.cuda.synchronize()
        log(f"[bench] attention prefill products run {args.attn_prefill_only} times")
        return 0
    if args.chunked_only:
        w = synth.WORKLOADS["llama70b_swiglu_t8"]
        gen = torch.Generator(device=dev)
        gen.manual_seed(w.seed)
        rnd = lambda *shape: torch.randn(shape, device=dev, generator=gen).to(torch.bfloat16)  # noqa: E731
        Xc, Wg, Zc, Wd, dHc = rnd(w.N, w.h), rnd(w.h, 2 * w.f), rnd(w.N, w.f), rnd(w.f, w.h), rnd(w.N, 2 * w.f)
        Pc = torch.empty((w.N, w.h), device=dev, dtype=torch.float32)
        dXc = torch.empty((w.N, w.h), device=dev, dtype=torch.float32)
        dWc = torch.empty((w.h, 2 * w.f), device=dev, dtype=torch.float32)
        evs = {nc: [torch.cuda.Event() for _ in range(nc)] for nc in (1, 2, 4, 8)}
        for _ in range(args.chunked_only):
            for nc in (1, 2, 4, 8):
                T.tp_row_linear_partial_chunked(Zc, Wd, nc, P=Pc, events=evs[nc])
            for nc in (1, 2, 4, 8):
                T.tp_col_linear_bwd_chunked(Xc, Wg, dHc, nc, dX_part=dXc, want_dw=False, events=evs[nc])
            T.tp_col_linear_bwd_chunked(Xc, Wg, dHc, 8, dX_part=dXc, dW=dWc, events=evs[8])
        torch.cuda.synchronize()
        log(f"[bench] chunked schedule run {args.chunked_only} times")
        return 0
    if args.embed_only:
        lw = synth.WORKLOADS["llama70b_lm_head_t8"]
        v_loc = lw.extra["V_pad"] // lw.t
        gen = torch.Generator(device=dev)
        gen.manual_seed(lw.seed + 1)
        E = torch.randn((v_loc, lw.h), device=dev, generator=gen).to(torch.bfloat16)
        ids = torch.randint(0, lw.extra["V"], (lw.N,), device=dev, generator=gen, dtype=torch.int32)
        dYe = torch.randn((lw.N, lw.h), device=dev, generator=gen)
        out = torch.empty((lw.N, lw.h), dtype=torch.bfloat16, device=dev)
        dE = torch.empty((v_loc, lw.h), dtype=torch.float32, device=dev)
        inr = (ids >= 0) & (ids < v_loc)
        idc = ids.clamp(0, v_loc - 1).long()
        id_in, dY_in = idc[inr], dYe[inr].contiguous()
        for _ in range(args.embed_only):
            T.tp_vocab_embed_fwd(ids, E, 0, out=out)
            T.tp_vocab_embed_bwd(ids, dYe, 0, v_loc, dE_i=dE)
        for _ in range(args.embed_only):
            torch.where(inr[:, None], torch.nn.functional.embedding(idc, E), 0.0)
            torch.zeros((v_loc, lw.h), dtype=torch.float32, device=dev).index_add_(0, id_in, dY_in)
        torch.cuda.synchronize()
        log(f"[bench] embedding run {args.embed_only} times")
        return 0
    if args.decode_only:
        q = synth.WORKLOADS["llama70b_qkv_t8"]
        wq, wo = (q.n_h + 2 * q.n_kv) * q.d_h // q.t, q.n_h * q.d_h // q.t
        gen = torch.Generator(device=dev)
        gen.manual_seed(q.seed)
        rnd = lambda *shape: torch.randn(shape, device=dev, generator=gen).to(torch.bfloat16)  # noqa: E731
        Xd, Od = rnd(16, q.h), rnd(16, wo)
        Wrs = [rnd(q.h, wq) for _ in range(16)]
        WOs = [rnd(wo, q.h) for _ in range(16)]
        Yd = torch.empty((16, wq), device=dev, dtype=torch.bfloat16)
        Pd = torch.empty((16, q.h), device=dev, dtype=torch.float32)
        for i in range(args.decode_only):
            T.tp_col_linear(Xd, Wrs[i % 16], "none", Y=Yd)
            T.tp_row_linear_partial(Od, WOs[i % 16], P=Pd)
        torch.cuda.synchronize()
        log(f"[bench] decode products run {args.decode_only} times")
        return 0
    props = torch.cuda.get_device_properties(0)
    log(f"[bench] device {props.name} {props.gcnArchName} CUs={props.multi_processor_count}")

    def to_dev(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---------------- workload: Llama-3-70B SwiGLU MLP shard, t = 8 ----------------
    w = synth.WORKLOADS["llama70b_swiglu_t8"]
    wb = synth.WORKLOADS["llama70b_swiglu_t8_bwd"]
    N, h, f = w.N, w.h, w.f
    t0 = time.perf_counter()
    d = synth.mlp_inputs(w.seed, N, h, w.F, w.t, "swiglu")
    dY_bits = synth.mlp_bwd_inputs(wb.seed, N, h)["dY"]
    log(f"[bench] inputs generated in {time.perf_counter() - t0:.1f}s")
    if args.data != "normal":
        # same shapes, other values: all zeros, or integers in [-2, 2]
        if args.data == "zeros":
            def alt(shape, seed):
                return np.zeros(shape, np.uint16)
        else:
            def alt(shape, seed):
                return synth.int_inputs(seed, shape)
        d = {k: alt(v.shape, 100 + i) for i, (k, v) in enumerate(d.items())}
        dY_bits = alt(dY_bits.shape, 99)
    input_digests = {k: synth.digest(d[k]) for k in ("X", "W_in", "W_out")}
    input_digests["dY"] = synth.digest(dY_bits)
    X, W_in, W_out, dY = to_dev(d["X"]), to_dev(d["W_in"]), to_dev(d["W_out"]), to_dev(dY_bits)
    bf, f32 = torch.bfloat16, torch.float32
    Z = torch.empty((N, f), dtype=bf, device=dev)
    H = torch.empty((N, 2 * f), dtype=bf, device=dev)
    P = torch.empty((N, h), dtype=f32, device=dev)
    dH = torch.empty((N, 2 * f), dtype=bf, device=dev)
    dX = torch.empty((N, h), dtype=f32, device=dev)
    dWi = torch.empty((h, 2 * f), dtype=f32, device=dev)
    dWo = torch.empty((f, h), dtype=f32, device=dev)

    fl = {
        "gemm1_gate_up_swiglu": 2 * N * (2 * f) * h,
        "gemm2_down_partial": 2 * N * h * f,
        "bwd_dz_swiglu": 2 * N * f * h,
        "bwd_dx_partial": 2 * N * h * (2 * f),
        "bwd_dw_gate_up": 2 * h * (2 * f) * N,
        "bwd_dw_down": 2 * f * h * N,
    }
    fwd_flops = fl["gemm1_gate_up_swiglu"] + fl["gemm2_down_partial"]
    bwd_flops = sum(v for k, v in fl.items() if k.startswith("bwd"))
    step_flops = fwd_flops + bwd_flops

    def fwd():
        T.tp_mlp_shard_fwd(X, W_in, W_out, "swiglu", Z=Z, H_save=H, P=P)

    def bwd():
        T.tp_mlp_shard_bwd(X, W_in, W_out, H, Z, dY, "swiglu", dH=dH, dX_part=dX, dW_in=dWi,
                           dW_out=dWo)

    def step():
        fwd()
        bwd()

    stream = torch.cuda.current_stream()

    def time_fn(fn, reps, warm=2, inner=4):
        """ms per call: `reps` HIP event pairs on the launch stream, each around
        `inner` back-to-back calls, so that the GPU queue stays full and the
        binding's host time per call (about 10 us) is not counted for kernels
        longer than that; mean, median and min over the pairs."""
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for a, b in evs:
            a.record(stream)
            for _ in range(inner):
                fn()
            b.record(stream)
        torch.cuda.synchronize()
        ts = [a.elapsed_time(b) / inner for a, b in evs]
        return float(np.mean(ts)), float(np.median(ts)), float(np.min(ts))

    def time_graph(fn, calls, replays=8):
        """Average ms per call of `fn` replayed from a HIP graph: `calls` calls
        are captured once on a side stream (after two eager warm-up rounds on
        it) and the graph is replayed `replays` times between two events. For
        launch-bound calls (decode, regroup) this is the GPU time without the
        Python binding's per-call host cost."""
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for _ in range(2 * calls):
                fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for _ in range(calls):
                fn()
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(side):  # replay() launches on the current stream
            e0.record(side)
            for _ in range(replays):
                graph.replay()
            e1.record(side)
        torch.cuda.synchronize()
        del graph
        return e0.elapsed_time(e1) / (calls * replays)

    # ---------------- timed region: K steps ----------------
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    value = step_flops / (ms_step * 1e-3) / 1e12
    log(f"[bench] step {ms_step:.4f} ms  {value:.1f} TFLOP/s  "
        f"{100 * value / PEAK_BF16_TFLOPS:.1f}% of peak  (wall {wall:.3f}s)")

    # The context rows are measured after the step: a Python-level failure in
    # one of them (an error a call returns, a probe that cannot run) is
    # recorded under rows["errors"] and the line is still printed.
    errors = {}

    def guarded(name, fn):
        try:
            return fn()
        except Exception as e:  # noqa: BLE001
            import traceback
            traceback.print_exc(file=sys.stderr)
            errors[name] = f"{type(e).__name__}: {e}"[:400]
            return None

    # ---------------- per-kernel timings (single-kernel entry points) ----------------
    # Each entry point below launches exactly the kernel (same template
    # instantiation and launch shape) that the step launches for that product.
    kern = {
        "gemm1_gate_up_swiglu": lambda: T.tp_col_linear(X, W_in, "swiglu", Y=Z, H_save=H),
        "gemm2_down_partial": lambda: T.tp_row_linear_partial(Z, W_out, P=P),
        # the backward call with no gradient requested: dZ = dY W_down^T with
        # the SwiGLU backward epilogue (reads H, writes dH) alone
        "bwd_dz_swiglu": lambda: T.tp_mlp_shard_bwd(X, W_in, W_out, H, Z, dY, "swiglu", dH=dH, want=()),
        "bwd_dx_partial": lambda: T.tp_col_linear_bwd(X, W_in, dH, dX_part=dX, want_dw=False),
        "bwd_dw_gate_up": lambda: T.tp_col_linear_bwd(X, W_in, dH, dW=dWi, want_dx=False),
        "bwd_dw_down": lambda: T.tp_row_linear_bwd(Z, W_out, dY, dW=dWo, want_dz=False),
    }
    kt = {}
    for name, fn in kern.items():
        mean, med, mn = time_fn(fn, args.reps)
        kt[name] = {"ms": round(mean, 4), "ms_median": round(med, 4),
                    "tflops": round(fl[name] / (mean * 1e-3) / 1e12, 1)}
        log(f"[bench] {name:24s} {mean:.4f} ms  {kt[name]['tflops']} TFLOP/s")
    bwd_mean = time_fn(bwd, args.reps)[0]

    # dominant kernel: the single launch with the largest share of the step,
    # timed over `reps` back-to-back launches on the launch stream
    dom = max((n for n in kern), key=lambda n: kt[n]["ms"])
    fn = kern[dom]
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    per_launch_ms = e0.elapsed_time(e1) / args.reps
    achieved = fl[dom] / (per_launch_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": committed_traffic(dom), "kernel": KERNEL_DESC[dom],
                "flop_per_launch": fl[dom], "avg_launch_ms": round(per_launch_ms, 4)}
    log(f"[bench] dominant {dom}: {per_launch_ms:.4f} ms per launch, {achieved:.1f} TFLOP/s")

    # GEMM2 computed in token-row chunks with an event per chunk (the schedule
    # that lets the exchange of chunk c overlap chunk c + 1): its overhead
    chunked = {}
    for nc in (() if args.no_rows else (2, 4, 8)):
        evs = [torch.cuda.Event() for _ in range(nc)]

        def g2c():
            T.tp_row_linear_partial_chunked(Z, W_out, nc, P=P, events=evs)

        ms_c = time_fn(g2c, args.reps)[0]
        chunked[str(nc)] = {"ms": round(ms_c, 4), "tflops": round(fl["gemm2_down_partial"] / (ms_c * 1e-3) / 1e12, 1),
                            "overhead": round(ms_c / kt["gemm2_down_partial"]["ms"] - 1, 3)}
    if chunked:
        kt["gemm2_down_partial_chunked"] = chunked
    # dX_part of the backward in token-row chunks (its exchange could start
    # chunk by chunk), then the same followed by dW_gate|up over all tokens
    # against the unchunked column-parallel backward of both
    chunked = {}
    for nc in (() if args.no_rows else (2, 4, 8)):
        evs = [torch.cuda.Event() for _ in range(nc)]

        def dxc():
            T.tp_col_linear_bwd_chunked(X, W_in, dH, nc, dX_part=dX, want_dw=False, events=evs)

        ms_c = time_fn(dxc, args.reps)[0]
        chunked[str(nc)] = {"ms": round(ms_c, 4), "tflops": round(fl["bwd_dx_partial"] / (ms_c * 1e-3) / 1e12, 1),
                            "overhead": round(ms_c / kt["bwd_dx_partial"]["ms"] - 1, 3)}
    if chunked:
        kt["bwd_dx_partial_chunked"] = chunked
        evs = [torch.cuda.Event() for _ in range(8)]
        ms_both = time_fn(lambda: T.tp_col_linear_bwd(X, W_in, dH, dX_part=dX, dW=dWi), args.reps)[0]
        ms_c8 = time_fn(lambda: T.tp_col_linear_bwd_chunked(X, W_in, dH, 8, dX_part=dX, dW=dWi, events=evs),
                        args.reps)[0]
        kt["col_bwd_dx_8_chunks_then_dw"] = {"ms": round(ms_c8, 4), "unchunked_ms": round(ms_both, 4),
                                             "overhead": round(ms_c8 / ms_both - 1, 3)}
    # The step's fp32 products against the vendor BLAS writing the same fp32
    # outputs (torch.mm with fp32 output, transposed operands made contiguous
    # outside the timing), side by side, three rounds in turn, medians
    if not args.no_rows:
        def fp32_side_by_side():
            mm32, vout = mm_fp32_out(torch)
            if not vout.startswith("fp32"):
                return {"skipped": vout}
            W_inT, XT, ZT = W_in.t().contiguous(), X.t().contiguous(), Z.t().contiguous()
            pairs = {"gemm2_down_partial": (kern["gemm2_down_partial"], lambda: mm32(Z, W_out)),
                     "bwd_dx_partial": (kern["bwd_dx_partial"], lambda: mm32(dH, W_inT)),
                     "bwd_dw_gate_up": (kern["bwd_dw_gate_up"], lambda: mm32(XT, dH)),
                     "bwd_dw_down": (kern["bwd_dw_down"], lambda: mm32(ZT, dY))}
            rr = {k: ([], []) for k in pairs}
            for _ in range(3):
                for k, (ours, vend) in pairs.items():
                    rr[k][0].append(time_fn(ours, args.reps)[1])
                    rr[k][1].append(time_fn(vend, args.reps)[1])
            del W_inT, XT, ZT
            res = {}
            for k, (o, v) in rr.items():
                mo, mv = float(np.median(o)), float(np.median(v))
                res[k] = {"ms": round(mo, 4), "vendor_fp32_out_ms": round(mv, 4),
                          "ours_faster_by": round(mv / mo - 1, 3)}
            log(f"[bench] fp32 products vs vendor BLAS with fp32 outputs: " +
                ", ".join(f"{k} {v['ms']} vs {v['vendor_fp32_out_ms']}" for k, v in res.items()))
            return res
        sbs = guarded("vendor_fp32_side_by_side", fp32_side_by_side)
        if sbs is not None:
            kt["vendor_fp32_side_by_side"] = sbs

    # The fp32 epilogue's cost: GEMM2's output shape (512 tiles of 256 x 256,
    # two waves on 256 CUs) contracted over K = 64, two k32 sub-steps, so a
    # launch is almost only its prologue and the 128 MiB of fp32 stores; the
    # per-CU store rate is the output bytes / time / CUs.
    if not args.no_rows:
        Zk64, Wk64 = Z[:, :64].contiguous(), W_out[:64].contiguous()
        ms_st = time_fn(lambda: T.tp_row_linear_partial(Zk64, Wk64, P=P), args.reps)[0]
        del Zk64, Wk64
        out_bytes = 4 * N * h
        kt["gemm2_shape_k64_store_bound"] = {
            "ms": round(ms_st, 4), "output_bytes": out_bytes,
            "gbs": round(out_bytes / (ms_st * 1e-3) / 1e9, 1),
            "per_cu_gbs": round(out_bytes / (ms_st * 1e-3) / 1e9 / props.multi_processor_count, 1)}
        log(f"[bench] GEMM2 shape at K = 64 (stores): {kt['gemm2_shape_k64_store_bound']}")

    # Epilogue fusion, for context: the same products with a plain bf16 store,
    # then the activation (or its derivative) as a separate elementwise pass
    # in eager torch (several kernels). A single ideal pass would move 84 MiB
    # forward (read G, U; write Z) and 140 MiB backward (read dZ, G, U; write
    # dG, dU); its rate is reported against those bytes.
    if not args.no_rows:
        Hp = torch.empty((N, 2 * f), dtype=bf, device=dev)
        Zp = torch.empty((N, f), dtype=bf, device=dev)
        dZp = torch.empty((N, f), dtype=bf, device=dev)
        dHp = torch.empty((N, 2 * f), dtype=bf, device=dev)

        def act_fwd():
            torch.mul(torch.nn.functional.silu(Hp[:, :f]), Hp[:, f:], out=Zp)

        def act_bwd():
            g, u, dz = H[:, :f].float(), H[:, f:].float(), dZp.float()
            sg = torch.sigmoid(g)
            dHp[:, :f] = dz * u * sg * (1 + g * (1 - sg))
            dHp[:, f:] = dz * g * sg

        g1p = time_fn(lambda: T.tp_col_linear(X, W_in, "none", Y=Hp), args.reps)[0]
        afp = time_fn(act_fwd, args.reps)[0]
        dzp = time_fn(lambda: T.tp_row_linear_bwd(Z, W_out, dY, dZ=dZp, want_dw=False), args.reps)[0]
        abp = time_fn(act_bwd, args.reps)[0]
        mib = 1 << 20
        kt["epilogue_fusion"] = {
            "fwd": {"fused_ms": kt["gemm1_gate_up_swiglu"]["ms"], "plain_gemm_ms": round(g1p, 4),
                    "separate_pass_ms": round(afp, 4), "pass_ideal_bytes": 84 * mib,
                    "pass_gbs_vs_ideal_bytes": round(84 * mib / (afp * 1e-3) / 1e9, 1)},
            "bwd": {"fused_ms": kt["bwd_dz_swiglu"]["ms"], "plain_gemm_ms": round(dzp, 4),
                    "separate_pass_ms": round(abp, 4), "pass_ideal_bytes": 140 * mib,
                    "pass_gbs_vs_ideal_bytes": round(140 * mib / (abp * 1e-3) / 1e9, 1)},
        }
        log(f"[bench] epilogue fusion: {kt['epilogue_fusion']}")
        del Hp, Zp, dZp, dHp

    rows = {"mlp_kernels": kt,
            "fwd_ms": round(time_fn(fwd, args.reps)[0], 4), "bwd_ms": round(bwd_mean, 4)}
    rows["fwd_tflops"] = round(fwd_flops / (rows["fwd_ms"] * 1e-3) / 1e12, 1)
    rows["bwd_tflops"] = round(bwd_flops / (rows["bwd_ms"] * 1e-3) / 1e12, 1)

    del Z, H, P, dH, dX, dWi, dWo
    if not args.no_rows:
        rows.update(guarded("rows", lambda: measure_rows(T, synth, np, torch, dev, to_dev, time_fn, time_graph,
                                                          args.reps)) or {})
        vr = guarded("vendor_gemm_reference", lambda: vendor_reference(torch, dev, time_fn, args.reps, N, h, f))
        if vr is not None:
            rows["vendor_gemm_reference"] = vr
    torch.cuda.synchronize()
    if not args.no_rows:
        guarded("probes", lambda: probe_rows(rows, value, np))
    if errors:
        rows["errors"] = errors

    # ---------------- CPU baseline: the oracle on a token sample ----------------
    cpu = None
    if args.cpu_tokens > 0:
        cpu = guarded("cpu_baseline", lambda: cpu_baseline(d, dY_bits, args.cpu_tokens, synth, np))
        if errors:
            rows["errors"] = errors

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": {"normal": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) weights)",
                 "zeros": "all-zero inputs (power study, not the workload)",
                 "ints": "integers in [-2, 2] (power study, not the workload)"}[args.data],
        "config": {"workload": "llama3-70b-tp8-swiglu-mlp-shard-fwd-bwd", "tokens": N, "h": h,
                   "F": w.F, "t": w.t, "f": f, "step_gflop": round(step_flops / 1e9, 2),
                   # SHA-256 (first 16 hex digits) of the bf16 inputs, to identify the data
                   "input_digests": input_digests},
        "pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "rows": rows,
        "device": {"name": props.name, "arch": props.gcnArchName, "cus": props.multi_processor_count},
    }
    print(json.dumps(out), flush=True)
    return 0


def measure_rows(T, synth, np, torch, dev, to_dev, time_fn, time_graph, reps):
    """The other rows of the hot path, each timed on its own."""
    res = {}
    bf, f32 = torch.bfloat16, torch.float32
    # --- fused-QKV regroup, Llama-3-70B t=8, 4 rotated source copies (> Infinity Cache) ---
    q = synth.WORKLOADS["llama70b_qkv_t8"]
    n_h, n_kv, d_h, t, h = q.n_h, q.n_kv, q.d_h, q.t, q.h
    width = (n_h + 2 * n_kv) * d_h
    gen = torch.Generator(device=dev)
    gen.manual_seed(q.seed)
    srcs = [torch.randn((h, width), device=dev, dtype=f32, generator=gen).to(bf) for _ in range(4)]
    dsts = [torch.empty((h, width // t), device=dev, dtype=bf) for _ in range(4)]
    it = [0]

    def regroup():
        i = it[0]
        it[0] += 1
        T.tp_qkv_regroup(srcs[i % 4], n_h, n_kv, d_h, t, (i // 4) % t, W_r=dsts[i % 4])

    ms_eager = time_fn(regroup, max(reps, 32), warm=4)[0]
    ms = time_graph(regroup, 32)
    moved = 2 * h * (width // t) * 2
    # context: a plain device copy of the same bytes (contiguous), same graph
    # timing, reading a different slice of the sources as the ranks rotate
    # (8 slices x 4 sources = 671 MB), so that, like the regroup's, its reads
    # come from HBM and not from the 256 MB Infinity Cache
    it[0] = 0
    n_slice = h * (width // t)

    def plain_copy():
        i = it[0]
        it[0] += 1
        k = (i // 4) % t
        dsts[i % 4].view(-1).copy_(srcs[i % 4].view(-1)[k * n_slice:(k + 1) * n_slice])

    ms_copy = time_graph(plain_copy, 32)
    res["qkv_regroup"] = {"ms": round(ms, 5), "ms_eager": round(ms_eager, 5), "bytes": moved,
                          "gbs": round(moved / (ms * 1e-3) / 1e9, 1),
                          "frac_hbm": round(moved / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3),
                          "plain_copy_ms": round(ms_copy, 5)}
    # the same at t = 16 > n_kv = 8: each KV head replicated on two ranks
    t16 = 16
    w16 = T.regroup_width(n_h, n_kv, d_h, t16)
    dsts = [torch.empty((h, w16), device=dev, dtype=bf) for _ in range(4)]
    it[0] = 0

    def regroup16():
        i = it[0]
        it[0] += 1
        T.tp_qkv_regroup(srcs[i % 4], n_h, n_kv, d_h, t16, (i // 4) % t16, W_r=dsts[i % 4])

    ms = time_graph(regroup16, 32)
    moved = 2 * h * w16 * 2
    res["qkv_regroup_t16_replicated_kv"] = {"ms": round(ms, 5), "bytes": moved,
                                            "gbs": round(moved / (ms * 1e-3) / 1e9, 1),
                                            "frac_hbm": round(moved / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)}
    # replica K|V weight-gradient sum at t = 16 (f32 [h, (n_h/t + 2) d_h] shards)
    gw = [torch.randn((h, w16), device=dev, generator=gen) for _ in range(8)]
    it[0] = 0

    def kv_sum():
        i = it[0]
        it[0] += 1
        T.tp_kv_grad_accumulate(gw[(2 * i) % 8], gw[(2 * i + 1) % 8], n_h, n_kv, d_h, t16)

    ms = time_graph(kv_sum, 32)
    moved = 3 * h * 2 * d_h * 4
    res["kv_grad_accumulate_t16"] = {"ms": round(ms, 5), "bytes": moved,
                                     "gbs": round(moved / (ms * 1e-3) / 1e9, 1),
                                     "frac_hbm": round(moved / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)}
    del srcs, dsts, gw

    # --- attention projections: QKV column GEMM + W_O row partial, fwd and bwd ---
    dq = synth.qkv_inputs(q.seed, q.N, h, n_h, n_kv, d_h, t)
    Wr_bits = dq["W_qkv"][:, :width // t]   # rank-0 shape; values do not change timing
    W_r, W_O = to_dev(np.ascontiguousarray(Wr_bits)), to_dev(dq["W_O"])
    X, O, dQKV, dY = to_dev(dq["X"]), to_dev(dq["O"]), to_dev(dq["dQKV"]), to_dev(dq["dY"])
    Nq = q.N
    Y = torch.empty((Nq, width // t), dtype=bf, device=dev)
    P = torch.empty((Nq, h), dtype=f32, device=dev)
    fl_fwd = 2 * Nq * h * (width // t) + 2 * Nq * (n_h * d_h // t) * h

    def attn_fwd():
        T.tp_col_linear(X, W_r, "none", Y=Y)
        T.tp_row_linear_partial(O, W_O, P=P)

    dXq = torch.empty((Nq, h), dtype=f32, device=dev)
    dWq = torch.empty((h, width // t), dtype=f32, device=dev)
    dO = torch.empty((Nq, n_h * d_h // t), dtype=bf, device=dev)
    dWO = torch.empty((n_h * d_h // t, h), dtype=f32, device=dev)

    def attn_bwd():
        T.tp_col_linear_bwd(X, W_r, dQKV, dX_part=dXq, dW=dWq)
        T.tp_row_linear_bwd(O, W_O, dY, dZ=dO, dW=dWO)

    # The vendor BLAS (torch.mm) on the same operands, as plain NN products
    # of contiguous operands (the transposes made here, out of the timing),
    # writing the same output dtypes as ours (fp32 for W_O, dX, dW, dW_O;
    # bf16 for QKV and dO) where torch offers fp32 outputs of bf16 products.
    # Both are timed side by side, three rounds in turn (medians): the chip's
    # power state carries over from one measurement to the next, so only
    # measurements taken together compare.
    W_rT, W_OT, XT, OT = W_r.t().contiguous(), W_O.t().contiguous(), X.t().contiguous(), O.t().contiguous()
    mm32, vendor_out = mm_fp32_out(torch)

    def vendor_fwd():
        torch.mm(X, W_r)
        mm32(O, W_O)

    def vendor_bwd():
        mm32(dQKV, W_rT)
        mm32(XT, dQKV)
        torch.mm(dY, W_OT)
        mm32(OT, dY)

    rounds = {k: [] for k in ("fwd", "vendor_fwd", "bwd", "vendor_bwd")}
    for _ in range(3):
        for k, fn in (("fwd", attn_fwd), ("vendor_fwd", vendor_fwd), ("bwd", attn_bwd), ("vendor_bwd", vendor_bwd)):
            rounds[k].append(time_fn(fn, reps, warm=8)[0])
    for k, fl in (("fwd", fl_fwd), ("bwd", 2 * fl_fwd)):
        ms, mv = float(np.median(rounds[k])), float(np.median(rounds["vendor_" + k]))
        res[f"attn_proj_{k}_prefill"] = {
            "ms": round(ms, 4), "gflop": round(fl / 1e9, 2), "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
            "vendor_blas_ms": round(mv, 4), "vendor_blas_tflops": round(fl / (mv * 1e-3) / 1e12, 1),
            "rounds_ms": [round(x, 4) for x in rounds[k]],
            "vendor_rounds_ms": [round(x, 4) for x in rounds["vendor_" + k]], "vendor_outputs": vendor_out}
    log(f"[bench] attention prefill, ours vs vendor BLAS side by side: fwd "
        f"{res['attn_proj_fwd_prefill']['ms']} vs {res['attn_proj_fwd_prefill']['vendor_blas_ms']} ms, bwd "
        f"{res['attn_proj_bwd_prefill']['ms']} vs {res['attn_proj_bwd_prefill']['vendor_blas_ms']} ms")
    del W_rT, W_OT, XT, OT
    del dXq, dWq, dO, dWO, Y, P
    # decode, N = 16: weights rotated over 16 copies (> Infinity Cache)
    Wrs = [W_r.clone() for _ in range(16)]
    WOs = [W_O.clone() for _ in range(16)]
    Xd, Od = X[:16].contiguous(), O[:16].contiguous()
    Yd = torch.empty((16, width // t), dtype=bf, device=dev)
    Pd = torch.empty((16, h), dtype=f32, device=dev)
    it[0] = 0

    def decode():
        i = it[0] % 16
        it[0] += 1
        T.tp_col_linear(Xd, Wrs[i], "none", Y=Yd)
        T.tp_row_linear_partial(Od, WOs[i], P=Pd)

    ms_eager = time_fn(decode, max(reps, 32), warm=4)[0]
    ms = time_graph(decode, 16)
    wbytes = 2 * h * (width // t) + 2 * (n_h * d_h // t) * h
    # context: the vendor BLAS on the same two products (bf16 outputs), same graph timing
    it[0] = 0

    def decode_blas():
        i = it[0] % 16
        it[0] += 1
        torch.matmul(Xd, Wrs[i], out=Yd)
        torch.matmul(Od, WOs[i])

    ms_blas = time_graph(decode_blas, 16)
    res["attn_proj_decode_n16"] = {"ms": round(ms, 4), "ms_eager": round(ms_eager, 4), "weight_bytes": wbytes,
                                   "gbs": round(wbytes / (ms * 1e-3) / 1e9, 1),
                                   "frac_hbm": round(wbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3),
                                   "blas_ms": round(ms_blas, 4)}
    # context for the launch-bound rows: a kernel that does almost nothing
    # (a 16-element add), replayed from the same kind of graph
    tiny = torch.zeros(16, device=dev)
    res["graph_launch_floor"] = {"us_per_kernel": round(1000 * time_graph(lambda: tiny.add_(1.0), 16), 2)}
    del tiny
    del Wrs, WOs, X, O, dQKV, dY, W_r, W_O

    # --- Llama-3-70B vocab-parallel LM head + fused cross-entropy, one shard of 8 ---
    lw = synth.WORKLOADS["llama70b_lm_head_t8"]
    v_loc = lw.extra["V_pad"] // lw.t
    dl = synth.vocab_ce_inputs(lw.seed, lw.N, lw.h, v_loc, lw.extra["V"])
    Xl, Wl = to_dev(dl["X"]), to_dev(dl["W_i"])
    yl = torch.from_numpy(dl["targets"]).to(dev)
    dlo = torch.from_numpy(dl["dloss"]).to(dev)
    fl_ce = 2 * lw.N * lw.h * v_loc
    stats = {}

    def ce_fwd():
        stats["s"] = T.tp_vocab_ce_fwd(Xl, Wl, yl, 0)

    ms_f = time_fn(ce_fwd, reps)[0]
    loss, m_ce, S_ce = T.tp_vocab_ce_combine(*(st[None] for st in stats["s"]))
    dZl = torch.empty((lw.N, v_loc), dtype=bf, device=dev)
    dXl = torch.empty((lw.N, lw.h), dtype=f32, device=dev)
    dWl = torch.empty((lw.h, v_loc), dtype=f32, device=dev)

    def ce_bwd():
        T.tp_vocab_ce_bwd(Xl, Wl, yl, 0, m_ce, S_ce, dlo, dZ=dZl, dX_part=dXl, dW_i=dWl)

    ms_b = time_fn(ce_bwd, reps)[0]
    res["lm_head_ce_fwd"] = {"ms": round(ms_f, 4), "gflop": round(fl_ce / 1e9, 2),
                             "tflops": round(fl_ce / (ms_f * 1e-3) / 1e12, 1),
                             "logit_bytes_not_written": 4 * lw.N * v_loc}
    res["lm_head_ce_bwd"] = {"ms": round(ms_b, 4), "gflop": round(3 * fl_ce / 1e9, 2),
                             "tflops": round(3 * fl_ce / (ms_b * 1e-3) / 1e12, 1)}
    # The unfused alternative, timed side by side (three rounds in turn,
    # medians): the vendor BLAS writes the fp32 logits, then eager torch
    # takes each row's max, sum of exp(z - max) and target logit (forward);
    # the backward recomputes the logits, forms (softmax - one-hot) * dloss in
    # bf16 and runs dX and dW as vendor products with fp32 outputs.
    try:
        mm32, vout = mm_fp32_out(torch)
        inr = (yl >= 0) & (yl < v_loc)
        yc = yl.clamp(0, v_loc - 1).long()
        rows_in = torch.arange(lw.N, device=dev)[inr]
        cols_in = yc[inr]
        minus1 = torch.tensor(-1.0, device=dev)
        WlT, XlT = Wl.t().contiguous(), Xl.t().contiguous()

        def vendor_ce_fwd():
            z = mm32(Xl, Wl)
            m = z.amax(dim=1)
            torch.exp(z - m[:, None]).sum(dim=1)
            torch.where(inr, z.gather(1, yc[:, None]).squeeze(1), 0.0)

        def vendor_ce_bwd():
            z = mm32(Xl, Wl)
            pz = torch.exp(z - m_ce.reshape(-1, 1)) / S_ce.reshape(-1, 1)
            pz.index_put_((rows_in, cols_in), minus1, accumulate=True)
            dz = (pz * dlo.reshape(-1, 1)).to(bf)
            mm32(dz, WlT)
            mm32(XlT, dz)

        rr = {k: [] for k in ("fwd", "vfwd", "bwd", "vbwd")}
        for _ in range(3):
            for k, fn in (("fwd", ce_fwd), ("vfwd", vendor_ce_fwd), ("bwd", ce_bwd), ("vbwd", vendor_ce_bwd)):
                rr[k].append(time_fn(fn, reps)[1])
        res["lm_head_ce_fwd"].update({"side_by_side_ms": round(float(np.median(rr["fwd"])), 4),
                                      "vendor_unfused_ms": round(float(np.median(rr["vfwd"])), 4),
                                      "vendor_outputs": vout})
        res["lm_head_ce_bwd"].update({"side_by_side_ms": round(float(np.median(rr["bwd"])), 4),
                                      "vendor_unfused_ms": round(float(np.median(rr["vbwd"])), 4),
                                      "vendor_outputs": vout})
        log(f"[bench] LM head + CE, fused vs vendor unfused side by side: fwd "
            f"{res['lm_head_ce_fwd']['side_by_side_ms']} vs {res['lm_head_ce_fwd']['vendor_unfused_ms']} ms, bwd "
            f"{res['lm_head_ce_bwd']['side_by_side_ms']} vs {res['lm_head_ce_bwd']['vendor_unfused_ms']} ms")
        del WlT, XlT
    except Exception as e:  # noqa: BLE001  (context only: the fused rows above stand)
        res["lm_head_ce_fwd"]["vendor_unfused_error"] = f"{type(e).__name__}: {e}"[:300]
    del Xl, Wl, dZl, dXl, dWl, stats

    # --- Llama-3-70B vocab-parallel input embedding, one shard of 8 (rank 0) ---
    gen.manual_seed(lw.seed + 1)
    El = torch.randn((v_loc, lw.h), device=dev, generator=gen).to(bf)
    idl = torch.from_numpy(dl["targets"]).to(dev)           # token ids, uniform over the vocabulary
    in_range = int(((idl >= 0) & (idl < v_loc)).sum())
    outl = torch.empty((lw.N, lw.h), dtype=bf, device=dev)
    ms = time_graph(lambda: T.tp_vocab_embed_fwd(idl, El, 0, out=outl), 16)
    eb = 2 * lw.h * (in_range + lw.N)   # rows read + every output row written
    res["embed_fwd"] = {"ms": round(ms, 5), "bytes": eb, "gbs": round(eb / (ms * 1e-3) / 1e9, 1),
                        "frac_hbm": round(eb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)}
    dYe = torch.randn((lw.N, lw.h), device=dev, generator=gen)
    dEl = torch.empty((v_loc, lw.h), dtype=f32, device=dev)
    ms = time_fn(lambda: T.tp_vocab_embed_bwd(idl, dYe, 0, v_loc, dE_i=dEl), reps)[0]
    eb = 4 * lw.h * (in_range + v_loc)  # gradient rows read + every table row written
    res["embed_bwd"] = {"ms": round(ms, 5), "bytes": eb, "gbs": round(eb / (ms * 1e-3) / 1e9, 1),
                        "frac_hbm": round(eb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)}
    # The same two steps in eager torch, timed side by side (three rounds in
    # turn, medians): a masked F.embedding for the lookup, a zeroed fp32 table
    # with index_add_ of the in-range tokens' gradient rows for the gradient.
    try:
        inr_e = (idl >= 0) & (idl < v_loc)
        idc = idl.clamp(0, v_loc - 1).long()
        tok_in = torch.arange(lw.N, device=dev)[inr_e]
        id_in = idc[inr_e]
        dY_in = dYe[tok_in].contiguous()

        def torch_embed_fwd():
            torch.where(inr_e[:, None], torch.nn.functional.embedding(idc, El), 0.0)

        def torch_embed_bwd():
            torch.zeros((v_loc, lw.h), dtype=f32, device=dev).index_add_(0, id_in, dY_in)

        rr = {k: [] for k in ("fwd", "tfwd", "bwd", "tbwd")}
        for _ in range(3):
            rr["fwd"].append(time_graph(lambda: T.tp_vocab_embed_fwd(idl, El, 0, out=outl), 16))
            rr["tfwd"].append(time_graph(torch_embed_fwd, 16))
            rr["bwd"].append(time_fn(lambda: T.tp_vocab_embed_bwd(idl, dYe, 0, v_loc, dE_i=dEl), reps)[1])
            rr["tbwd"].append(time_fn(torch_embed_bwd, reps)[1])
        for k in ("fwd", "bwd"):
            res[f"embed_{k}"].update({"side_by_side_ms": round(float(np.median(rr[k])), 5),
                                      "torch_eager_ms": round(float(np.median(rr["t" + k])), 5)})
        log(f"[bench] embedding vs eager torch side by side: fwd {res['embed_fwd']['side_by_side_ms']} vs "
            f"{res['embed_fwd']['torch_eager_ms']} ms, bwd {res['embed_bwd']['side_by_side_ms']} vs "
            f"{res['embed_bwd']['torch_eager_ms']} ms")
        del dY_in
    except Exception as e:  # noqa: BLE001  (context only: the rows above stand)
        res["embed_fwd"]["torch_eager_error"] = f"{type(e).__name__}: {e}"[:300]
    del El, outl, dYe, dEl

    # --- GPT-style GeLU MLP shard, t = 4, forward ---
    g = synth.WORKLOADS["gpt_gelu_t4"]
    dg = synth.mlp_inputs(g.seed, g.N, g.h, g.F, g.t, "gelu")
    Xg, Ag, Bg = to_dev(dg["X"]), to_dev(dg["W_in"]), to_dev(dg["W_out"])
    Zg = torch.empty((g.N, g.f), dtype=bf, device=dev)
    Hg = torch.empty((g.N, g.f), dtype=bf, device=dev)
    Pg = torch.empty((g.N, g.h), dtype=f32, device=dev)
    flg = 2 * 2 * g.N * g.h * g.f
    ms = time_fn(lambda: T.tp_mlp_shard_fwd(Xg, Ag, Bg, "gelu", Z=Zg, H_save=Hg, P=Pg), reps)[0]
    res["gpt_gelu_mlp_fwd_t4"] = {"ms": round(ms, 4), "gflop": round(flg / 1e9, 2),
                                  "tflops": round(flg / (ms * 1e-3) / 1e12, 1)}
    return res


def mm_fp32_out(torch):
    """(mm, label): torch.mm writing fp32 outputs of a bf16 product when torch
    offers it on this device (checked on a small product), else the bf16 one."""
    try:
        a = torch.ones((64, 64), dtype=torch.bfloat16, device="cuda:0")
        c = torch.mm(a, a, out_dtype=torch.float32)
        torch.cuda.synchronize()
        if c.dtype == torch.float32 and float(c[0, 0]) == 64.0:
            return (lambda x, y: torch.mm(x, y, out_dtype=torch.float32)), "fp32 where ours are fp32"
    except (RuntimeError, TypeError):
        pass
    return (lambda x, y: torch.mm(x, y)), "bf16 (no fp32 outputs in this torch)"


def vendor_reference(torch, dev, time_fn, reps, N, h, f):
    """Context only: torch.matmul (the ROCm BLAS library) on the step's GEMM
    shapes, bf16 in and out, plain product without the epilogues. Not part of
    the measured path. (The attention projections are compared with it side
    by side in their own rows.)"""
    shapes = {"gemm1_gate_up": (N, h, 2 * f), "gemm2_down": (N, f, h), "dx": (N, 2 * f, h),
              "dw_gate_up": (h, N, 2 * f), "dw_down": (f, N, h)}
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    res = {}
    for name, (M, K, Nn) in shapes.items():
        a = torch.randn((M, K), device=dev, generator=g).to(torch.bfloat16)
        b = torch.randn((K, Nn), device=dev, generator=g).to(torch.bfloat16)
        ms = time_fn(lambda: a @ b, reps)[0]
        res[name] = {"ms": round(ms, 4), "tflops": round(2 * M * K * Nn / (ms * 1e-3) / 1e12, 1)}
        del a, b
    log(f"[bench] vendor BLAS reference: " + ", ".join(f"{k} {v['tflops']}" for k, v in res.items()))
    return res


def probe_rows(rows, value, np):
    """The matrix cores' sustained rate on this GPU with no memory traffic
    (random and all-zero operands), beside the step's rate, and one CU's
    store throughput (what a GEMM tile's epilogue costs): both from the
    stand-alone probes built beside the library."""
    mr = mfma_rate()
    med = {k: float(np.median([r["tflops"] for r in mr if r.get("data") == k])) for k in ("random", "zeros")}
    rows["mfma_rate_no_memory"] = {"random_tflops": round(med["random"], 1), "zeros_tflops": round(med["zeros"], 1),
                                   "step_frac_of_random": round(value / med["random"], 3)}
    clk = device_clock(mr)
    if clk:
        rows["mfma_rate_no_memory"]["device_max_sclk_mhz"] = clk["max_sclk_mhz"]
    log(f"[bench] MFMA rate without memory traffic: {rows['mfma_rate_no_memory']}")
    # one CU's store throughput: what a GEMM tile's epilogue costs
    sr = [r for r in run_probe("store_rate") if "pattern" in r]
    pick = lambda pat, w, n: next(r for r in sr if r["pattern"] == pat and r["waves"] == w and r["workgroups"] == n)  # noqa: E731
    rows["store_rate_per_cu"] = {
        "fp32_epilogue_gbs_per_cu": {f"{n}_cus_{w}_waves": pick("epilogue_fp32", w, n)["gbs_per_workgroup"]
                                     for n in (32, 256) for w in (4, 8, 16)},
        "fp32_mfma_layout_gbs_per_cu": {f"{n}_cus": pick("mfma_layout_fp32", 8, n)["gbs_per_workgroup"] for n in (32, 256)},
        "fp32_rows_gbs_per_cu_256": pick("rows_fp32", 8, 256)["gbs_per_workgroup"],
        "bf16_epilogue_gbs_per_cu_256": pick("epilogue_bf16", 8, 256)["gbs_per_workgroup"],
        "us_per_256x256_fp32_tile_all_cus": {
            "swapped": round(262144 / (pick("epilogue_fp32", 8, 256)["gbs_per_workgroup"] * 1e3), 2),
            "mfma_layout": round(262144 / (pick("mfma_layout_fp32", 8, 256)["gbs_per_workgroup"] * 1e3), 2)}}
    log(f"[bench] store rate per CU: {rows['store_rate_per_cu']}")


def run_probe(name, *args):
    """Run a stand-alone probe built beside the library (a child process on
    the same GPU); returns its JSON records."""
    import subprocess
    exe = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tensor_sharded_matmul_amd", name)
    if not os.path.exists(exe):
        raise RuntimeError(f"{exe} is not built; run `python -m tensor_sharded_matmul_amd.build`")
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=120)
    if r.returncode != 0:
        raise RuntimeError(f"{name} failed ({r.returncode}): {r.stderr.strip()[-500:]}")
    return [json.loads(line) for line in r.stdout.splitlines() if line.startswith("{")]


def mfma_rate(iters=20000, reps=3):
    """The MFMA rate probe's records {data, rep, ms, tflops} (and the device
    header)."""
    return run_probe("mfma_rate", iters, reps)


def device_clock(records):
    """The CU count and peak engine clock the probe read from the runtime."""
    return next((r for r in records if "max_sclk_mhz" in r), None)


def cpu_baseline(d, dY_bits, n_tok, synth, np):
    """The fp64 oracle as it stands, timed on the host cores: the measured
    workload's forward and backward (the backward from the forward's saved
    tensors, as the GPU step does; the first n_tok tokens, 4096 = all), then
    as legs the GPT GeLU shard forward and the Llama-3-70B attention
    projections forward + backward at prefill size."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 0) for i in threadpool_info()
                       if i.get("internal_api") == "openblas"), default=os.cpu_count())
    except Exception:
        threads = os.cpu_count()
    X = synth.bf16_to_f64(d["X"][:n_tok])
    W_in = synth.bf16_to_f64(d["W_in"])
    W_out = synth.bf16_to_f64(d["W_out"])
    dY = synth.bf16_to_f64(dY_bits[:n_tok])
    h, n_w = W_in.shape
    f = W_out.shape[0]
    t0 = time.perf_counter()
    Z, H, _ = O.mlp_shard_fwd(X, W_in, W_out, "swiglu")
    O.mlp_shard_bwd_saved(X, W_in, W_out, H, Z, dY, "swiglu")
    dt = time.perf_counter() - t0
    # GEMM1 + GEMM2 forward; dZ, dX, dW_in, dW_out backward: 3x the forward
    flops = 3 * (2 * n_tok * n_w * h + 2 * n_tok * h * f)
    del X, W_in, W_out, dY, Z, H
    log(f"[bench] oracle fp64 on {n_tok} tokens: {dt:.2f}s, {flops / dt / 1e9:.1f} GFLOP/s, "
        f"{threads} threads")
    legs = {}
    g = synth.WORKLOADS["gpt_gelu_t4"]
    dg = synth.mlp_inputs(g.seed, g.N, g.h, g.F, g.t, "gelu")
    og = {k: synth.bf16_to_f64(v) for k, v in dg.items()}
    t0 = time.perf_counter()
    O.mlp_shard_fwd(og["X"], og["W_in"], og["W_out"], "gelu")
    dtg = time.perf_counter() - t0
    flg = 2 * 2 * g.N * g.h * g.f
    legs["gpt_gelu_mlp_fwd_t4"] = {"s": round(dtg, 3), "gflop": round(flg / 1e9, 2),
                                   "tflops": round(flg / dtg / 1e12, 4)}
    del dg, og
    q = synth.WORKLOADS["llama70b_qkv_t8"]
    dq = synth.qkv_inputs(q.seed, q.N, q.h, q.n_h, q.n_kv, q.d_h, q.t)
    Wr = synth.bf16_to_f64(O.qkv_regroup(dq["W_qkv"], q.n_h, q.n_kv, q.d_h, q.t, 0))
    oq = {k: synth.bf16_to_f64(dq[k]) for k in ("X", "O", "W_O", "dQKV", "dY")}
    t0 = time.perf_counter()
    O.col_linear(oq["X"], Wr)
    O.row_linear_partial(oq["O"], oq["W_O"])
    O.col_linear_bwd(oq["X"], Wr, oq["dQKV"])
    O.row_linear_bwd(oq["O"], oq["W_O"], oq["dY"])
    dtq = time.perf_counter() - t0
    flq = 3 * (2 * q.N * q.h * Wr.shape[1] + 2 * q.N * oq["W_O"].shape[0] * q.h)
    legs["attn_proj_fwd_bwd_prefill"] = {"s": round(dtq, 3), "gflop": round(flq / 1e9, 2),
                                         "tflops": round(flq / dtq / 1e12, 4)}
    log(f"[bench] oracle legs: {legs}")
    return {"value": round(flops / dt / 1e12, 4), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the measured step (MLP shard fwd + bwd from saved tensors) on {n_tok} of 4096 tokens, "
                      f"fp64 numpy/OpenBLAS: {dt:.2f} s for {flops / 1e9:.1f} GFLOP",
            "legs": legs}


if __name__ == "__main__":
    sys.exit(main())
