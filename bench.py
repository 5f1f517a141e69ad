"""Throughput of the causal prefill attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the whole path over one batch of synthetic inputs
that already sit in HBM: the input step (per-tensor FP8 quantization of Q, K
and V, or the BF16 cast) and then the attention kernel (causal tile walk,
Q.K^T, online softmax, P.V, O and LSE epilogue). The default workload is the
long-context headline shape: B=1, S=32768, H=32, d=128, causal, FP8 e4m3
with per-tensor scales, Q, K, V ~ N(0, 1).

FP8 input step: by default Q and K are rotated by Hadamard blocks before the
per-tensor cast (attn_quantize_fp8_qkv_hadamard), which keeps the LSE within
its bar on heavy-tailed activations; ``--no-hadamard`` takes the unrotated
step (attn_quantize_fp8_qkv). The attention kernel is the same either way.

Prints ONE JSON line. ``value`` is the algorithmic causal FLOP count
B*Hq*S^2*(d_qk+d_v) divided by the measured time of a whole step, in TFLOP/s.
The attention kernel alone is reported beside it and in ``roofline``, whose
duration comes from HIP events recorded on the stream the kernel runs on.
For FP8, the input step folds Q's scale so that the score factor is a power
of two; ``attention_plain_q_scale`` times the same attention on the literal
per-tensor step (Q and K unrotated under their plain absmax scales, the
kernel's fma form) beside it.
``cpu_baseline`` times the fp64 CPU oracle on the first four query heads of
batch 0 of the same workload (all S query rows each), on this host's cores.

Only one GPU is used: ``--gpus`` above 1 exits with an error.
"""

from __future__ import annotations

import argparse
import dataclasses
import math
import hashlib
import json
import os
import shutil
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
PEAK_TFLOPS = {"fp8": 5000.0, "bf16": 2500.0}
HBM_GBS = 8000.0
METRIC = "causal prefill attention TFLOP/s (FP8, d=128, S=32K) and % of dense FP8 MFMA peak"
HEADLINE = "mha_fp8_32k"
KERNEL_SOURCES = ["attn_fwd_kernel.h", "common.h", "attn_fwd_launch.h"]


def code_only(text: str) -> str:
    """C/C++ source without comments, blank space collapsed to single spaces."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """Hash of the attention kernel's sources with comments and blank space removed
    (a comment edit does not invalidate the stored counter readings)."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "bf16_causal_prefill_fwd_amd", "csrc", name)) as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str, src_hash: str):
    """HBM bytes per attention launch from the committed PMC summary.

    profiles/attn_fwd_<workload>_traffic.txt holds ``key: value`` lines written
    from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) scaled by a plain
    copy of known size. It only counts if it was taken on the current kernel
    sources (same source hash); otherwise the traffic is unknown (None).
    """
    path = os.path.join(ROOT, "profiles", f"attn_fwd_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.lstrip().startswith("#"):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("kernel_source_sha256_16") != src_hash:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def algorithmic_bytes(w) -> float:
    """Q, K, V read once, O (bf16) and LSE (fp32) written once."""
    eb = 1 if w.dtype == "fp8" else 2
    qkv = w.B * w.S * (w.Hq * w.d_qk + w.Hkv * w.d_qk + w.Hkv * w.d_v) * eb
    out = w.B * w.S * w.Hq * w.d_v * 2 + w.B * w.Hq * w.S * 4
    return float(qkv + out)


def _amd_smi_sample(smi: str):
    """One reading of the gfx clocks (MHz, one per XCD) and socket power (W), or None."""
    try:
        out = subprocess.run([smi, "metric", "-g", "0", "--clock", "--power", "--json"],
                             capture_output=True, text=True, timeout=10)
        d = json.loads(out.stdout)
        g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        clks = [v["clk"]["value"] for k, v in g["clock"].items()
                if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)
                and isinstance(v["clk"].get("value"), (int, float))]
        pw = g.get("power", {}).get("socket_power", {}).get("value")
        if not clks:
            return None
        return sum(clks) / len(clks), min(clks), (float(pw) if isinstance(pw, (int, float)) else None)
    except Exception:
        return None


def sustained(seconds: float, attention, flops: float, stream, peak_tflops: float) -> dict:
    """Back-to-back attention launches for `seconds`, with SCLK and power sampled meanwhile.

    The pages report that the clock depends on the data (bit toggling), so the
    sustained rate and the clock it ran at are recorded together.
    """
    import threading

    import torch

    smi = shutil.which("amd-smi") or ("/opt/rocm/bin/amd-smi" if os.path.exists("/opt/rocm/bin/amd-smi") else None)
    samples = []
    stop = threading.Event()

    def poll():
        while not stop.is_set():
            r = _amd_smi_sample(smi)
            if r is None:
                return
            samples.append((time.perf_counter() - t0,) + r)
            stop.wait(0.2)

    th = threading.Thread(target=poll, daemon=True) if smi else None
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if th:
        th.start()
    e0.record(stream)
    launches = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            attention()
        launches += 10
        torch.cuda.synchronize()
    e1.record(stream)
    torch.cuda.synchronize()
    stop.set()
    if th:
        th.join(timeout=15)
    ms = e0.elapsed_time(e1)
    rec = {"seconds": round(ms / 1e3, 2), "launches": launches,
           "attention_tflops": round(launches * flops / (ms * 1e-3) / 1e12, 2),
           "sclk_mhz": None, "socket_power_w": None,
           "sampling": "amd-smi metric --clock --power, mean over XCDs, every ~0.3 s, after the first second"}
    # readings from the first second show the clock still ramping from idle
    settled = [x[1:] for x in samples if x[0] >= 1.0]
    if settled:
        import numpy as np
        samples = settled
        mean_clk = np.array([x[0] for x in samples])
        rec["sclk_mhz"] = {"median": round(float(np.median(mean_clk)), 1), "min": round(float(mean_clk.min()), 1),
                           "max": round(float(mean_clk.max()), 1), "samples": len(samples)}
        # the dense peak scales with the clock (2.4 GHz for the datasheet figure)
        rec["frac_of_peak_at_measured_sclk"] = round(
            rec["attention_tflops"] / (peak_tflops * float(np.median(mean_clk)) / 2400.0), 4)
        pws = [x[2] for x in samples if x[2] is not None]
        if pws:
            rec["socket_power_w"] = {"median": float(np.median(pws)), "max": float(max(pws))}
            # whole-socket energy (HBM and idle parts included) per unit of work
            rec["tflop_per_joule"] = round(rec["attention_tflops"] / float(np.median(pws)), 4)
    return rec


def plain_q_scale_leg(steps: int, w, q32, k32, codes, scales, o, flags: int, flops: float, peak: float,
                      sm_scale: float, stream) -> dict:
    """The FP8 attention again, on the literal per-tensor input step: Q and K
    unrotated, under their plain absmax scales.

    The default input step rotates Q and K and folds Q's scale so that the
    score factor q_scale * k_scale * softmax_scale * log2(e) is a power of
    two, which lets the kernel apply it through the MFMA operand scales. With
    the plain scales the factor is generally not a power of two and the
    kernel applies it with one fma per score. Same V codes and scale; own Q
    and K codes, O and LSE buffers.
    """
    import numpy as np
    import torch

    from bf16_causal_prefill_fwd_amd import ops

    print(f"# plain absmax Q scale: {steps} attention launches", file=sys.stderr, flush=True)
    q_plain = torch.empty_like(codes[0])
    k_plain = torch.empty_like(codes[1])
    scales_plain = torch.empty(3, dtype=torch.float32, device=q32.device)
    ops.attn_quantize_fp8(q32, out=q_plain, scale=scales_plain[0:1], stream=stream)
    ops.attn_quantize_fp8(k32, out=k_plain, scale=scales_plain[1:2], stream=stream)
    scales_plain[2:].copy_(scales[2:])
    o_plain = torch.empty_like(o)
    lse_plain = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=q32.device)

    def run():
        ops.attn_prefill_fwd(q_plain, k_plain, codes[2], causal=w.causal, out=o_plain, lse=lse_plain,
                             d_scales=scales_plain, stream=stream, flags=flags)

    for _ in range(3):
        run()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        e0.record(stream)
        run()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    sc = scales_plain.cpu().tolist()
    c = sc[0] * sc[1] * sm_scale * math.log2(math.e)
    mant, _ = math.frexp(c)
    avg = float(np.mean(ms))
    tflops = flops / (avg * 1e-3) / 1e12
    return {
        "q_scale": sc[0],
        "score_factor_power_of_two": bool(abs(mant - 0.5) < 2.0 ** -19),
        "attention_ms": round(avg, 4),
        "attention_ms_min": round(float(np.min(ms)), 4),
        "attention_tflops": round(tflops, 2),
        "attention_frac_of_peak": round(tflops / peak, 4),
        "note": "Q and K unrotated under their plain absmax/448 scales (attn_quantize_fp8), the literal "
                "per-tensor input step; the headline's input step rotates Q and K and folds Q's scale",
    }


def cpu_baseline(w, q, k, v, n_heads: int = 4, hadamard: bool = False, o_gpu=None, lse_gpu=None) -> dict:
    """The fp64 oracle on the first query heads of batch 0, every query row.

    n_heads whole causal head slices (about 10-15 s of CPU work at the 32K
    shape on a 16-core host) with the kv heads they read, quantized as the
    GPU input step does (with ``hadamard``, Q and K rotated first). Given the
    GPU's O and LSE for the same slices (numpy, [S, n_heads, d_v] and
    [n_heads, S]), their errors against this exact result are reported too.
    Also times the whole tiny configuration (B=1, S=512, H=2) on one thread.
    """
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import causal_attention, dequantize_fp8, encode_with_scale, per_tensor_scale, \
        per_tensor_scale_folded, bf16_encode, bf16_decode, prefill_reference
    from oracle.rotation import hadamard_encode, hadamard_scales
    from bf16_causal_prefill_fwd_amd.workloads import make_inputs

    G = w.Hq // w.Hkv
    nh = min(n_heads, w.Hq)
    nkv = max(1, nh // G)
    sm = 1.0 / math.sqrt(w.d_qk)
    t0 = time.perf_counter()
    if w.dtype == "fp8" and hadamard:
        kcs, ks = hadamard_scales(k)
        qcs, qs = hadamard_scales(q, k_scale=ks, softmax_scale=sm)
        vs = per_tensor_scale(v)
        sl = [dequantize_fp8(hadamard_encode(q[:1, :, 0:nh], qcs), qs),
              dequantize_fp8(hadamard_encode(k[:1, :, 0:nkv], kcs), ks),
              dequantize_fp8(encode_with_scale(v[:1, :, 0:nkv], vs), vs)]
    elif w.dtype == "fp8":
        ks, vs = per_tensor_scale(k), per_tensor_scale(v)
        scales = [per_tensor_scale_folded(q, ks, sm), ks, vs]
        cuts = ((q, nh), (k, nkv), (v, nkv))
        sl = [dequantize_fp8(encode_with_scale(x[:1, :, 0:n], s), s) for (x, n), s in zip(cuts, scales)]
    else:
        sl = [bf16_decode(bf16_encode(x[:1, :, 0:n])) for x, n in ((q, nh), (k, nkv), (v, nkv))]
    O, L = causal_attention(*sl, causal=w.causal)
    dt = time.perf_counter() - t0
    flops = nh * (float(w.S) ** 2 * (w.d_qk + w.d_v) if w.causal else 2.0 * float(w.S) ** 2 * (w.d_qk + w.d_v))
    threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    rec = {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"fp64 oracle (input step + exact softmax attention) on batch 0, query heads 0-{nh - 1} "
                   f"(kv heads 0-{nkv - 1}, G={G}), all {w.S} rows: {nh}/{w.B * w.Hq} of the workload, "
                   f"{flops / 1e9:.1f} GFLOP in {dt:.2f} s; host os.cpu_count()={os.cpu_count()}"),
    }
    if o_gpu is not None:
        import numpy as np
        og = np.asarray(o_gpu, dtype=np.float64)
        err = {"o_rel_l2": float(np.linalg.norm(og - O[0]) / np.linalg.norm(O[0])),
               "o_worst_row_rel_l2": float(np.max(np.linalg.norm(og - O[0], axis=-1)
                                                  / np.linalg.norm(O[0], axis=-1))),
               "bars": {"o_rel_l2": 3e-2 if w.dtype == "fp8" else 5e-3, "lse_max_abs": 1e-2}}
        if lse_gpu is not None:
            err["lse_max_abs"] = float(np.max(np.abs(np.asarray(lse_gpu, dtype=np.float64) - L[0])))
        rec["gpu_error_on_sample"] = err
    # the tiny configuration in full, one BLAS thread
    tq, tk, tv = make_inputs("tiny_mha_fp8", seed=0)
    with threadpool_limits(limits=1):
        t1 = time.perf_counter()
        prefill_reference(tq, tk, tv, "fp8", fold_q=True, hadamard=True)
        t1 = time.perf_counter() - t1
    tiny_flops = 2 * 512 ** 2 * 256
    rec["tiny_one_thread"] = {"workload": "tiny_mha_fp8 (B=1, S=512, H=2, d=128, FP8)", "seconds": round(t1, 3),
                              "gflops": round(tiny_flops / t1 / 1e9, 2), "threads": 1}
    return rec


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--hadamard", dest="hadamard", action="store_true", default=None,
                    help="FP8: rotate Q and K by Hadamard blocks in the input step "
                         "(attn_quantize_fp8_qkv_hadamard; the default for FP8 workloads)")
    ap.add_argument("--no-hadamard", dest="hadamard", action="store_false",
                    help="FP8: the unrotated input step (attn_quantize_fp8_qkv)")
    ap.add_argument("--p-block-scale", action="store_true",
                    help="FP8: per (row, 64-key block) power-of-two scaling of P (ATTN_FLAG_P_BLOCK_SCALE)")
    ap.add_argument("--p-rounded-sum", action="store_true",
                    help="FP8, with --p-block-scale: O divided by the row sum of the rounded P from one more "
                         "MFMA per step (ATTN_FLAG_P_ROUNDED_SUM)")
    ap.add_argument("--seq-len", type=int, default=None, help="override the workload's sequence length")
    ap.add_argument("--heads", type=int, default=None,
                    help="override the head count: Hq = Hkv = HEADS (multi-head attention)")
    ap.add_argument("--dist", choices=("gauss", "outlier", "outlier_shared", "mla"), default=None,
                    help="override the workload's input distribution (same shape), e.g. to compare the "
                         "clock and energy of Gaussian and heavy-tailed inputs")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-plain-q-scale", action="store_true",
                    help="skip the second FP8 attention timing with Q under its plain absmax scale (keeps a "
                         "profiled run to the headline's launches)")
    ap.add_argument("--sustain-s", type=float, default=10.0,
                    help="seconds of back-to-back attention launches with SCLK sampling (0 = skip)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the path has no multi-GPU mode", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from bf16_causal_prefill_fwd_amd import ops
    from bf16_causal_prefill_fwd_amd.workloads import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (none visible)", file=sys.stderr)
        return 2
    w = WORKLOADS[args.workload]
    base = w
    if args.dist is not None:
        w = dataclasses.replace(w, dist=args.dist)
    if args.seq_len is not None:
        if args.seq_len < 1:
            print("--seq-len must be >= 1", file=sys.stderr)
            return 2
        w = dataclasses.replace(w, S=args.seq_len)
    if args.heads is not None:
        if args.heads < 1:
            print("--heads must be >= 1", file=sys.stderr)
            return 2
        w = dataclasses.replace(w, Hq=args.heads, Hkv=args.heads)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"# workload {w.name}: generating inputs (seed {args.seed})", file=sys.stderr, flush=True)
    q, k, v = make_inputs(w, seed=args.seed)
    q32, k32, v32 = (torch.from_numpy(x).to(dev) for x in (q, k, v))

    # preallocated buffers: nothing is allocated inside the timed region
    if w.dtype == "fp8":
        codes = [torch.empty(t.shape, dtype=torch.uint8, device=dev) for t in (q32, k32, v32)]
    else:
        codes = [torch.empty(t.shape, dtype=torch.bfloat16, device=dev) for t in (q32, k32, v32)]
    scales = torch.empty(3, dtype=torch.float32, device=dev)
    o = torch.empty((w.B, w.S, w.Hq, w.d_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    sm_scale = 1.0 / math.sqrt(w.d_qk)

    if args.p_rounded_sum and not args.p_block_scale:
        print("--p-rounded-sum needs --p-block-scale", file=sys.stderr)
        return 2
    if (args.hadamard or args.p_block_scale or args.p_rounded_sum) and w.dtype != "fp8":
        print("--hadamard, --p-block-scale and --p-rounded-sum apply to FP8 workloads only", file=sys.stderr)
        return 2
    if args.hadamard is None:
        args.hadamard = w.dtype == "fp8"
    flags = (ops.ATTN_FLAG_P_BLOCK_SCALE if args.p_block_scale else 0) | \
        (ops.ATTN_FLAG_P_ROUNDED_SUM if args.p_rounded_sum else 0)

    def input_step():
        if w.dtype == "fp8":
            ops.attn_quantize_fp8_qkv(q32, k32, v32, sm_scale, out=codes, scales=scales, stream=stream,
                                      hadamard=args.hadamard)
        else:
            for i, t in enumerate((q32, k32, v32)):
                ops.attn_cast_bf16(t, out=codes[i], stream=stream)

    def attention():
        if w.dtype == "fp8":
            ops.attn_prefill_fwd(*codes, causal=w.causal, out=o, lse=lse, d_scales=scales, stream=stream,
                                 flags=flags)
        else:
            ops.attn_prefill_fwd(*codes, causal=w.causal, out=o, lse=lse, stream=stream)

    n_ev = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_ev)]
    print(f"# warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        input_step()
        attention()
    torch.cuda.synchronize()

    print(f"# timing {args.steps} steps", file=sys.stderr, flush=True)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        input_step()
        ev[i][1].record(stream)
        attention()
        ev[i][2].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0

    step_ms = t_start.elapsed_time(t_end) / args.steps
    attn_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in range(n_ev)]
    inp_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(n_ev)]
    attn_avg = float(np.mean(attn_ms))
    flops = w.causal_flops if w.causal else 2.0 * w.causal_flops
    value = flops / (step_ms * 1e-3) / 1e12
    attn_tflops = flops / (attn_avg * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    assert torch.isfinite(lse).all().item(), "non-finite LSE"

    if args.copy_calib_mib > 0:
        n = args.copy_calib_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    src_hash = kernel_source_hash()
    # the stored counter readings are for the workload as defined (shape and inputs)
    traffic = traffic_from_profile(w.name, src_hash) if w == base else None
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "S": w.S, "Hq": w.Hq, "Hkv": w.Hkv, "d_qk": w.d_qk,
                   "d_v": w.d_v, "causal": w.causal, "dist": w.dist, "seed": args.seed,
                   "hadamard": bool(args.hadamard), "p_block_scale": bool(args.p_block_scale),
                   "p_rounded_sum": bool(args.p_rounded_sum),
                   "step": "input step (quantize/cast Q,K,V) + attention"},
        "attention_ms": round(attn_avg, 4),
        "attention_ms_min": round(float(np.min(attn_ms)), 4),
        "attention_ms_median": round(float(np.median(attn_ms)), 4),
        "attention_tflops": round(attn_tflops, 2),
        "attention_frac_of_peak": round(attn_tflops / peak, 4),
        "input_step_ms": round(float(np.mean(inp_ms)), 4),
        "wall_s_timed": round(wall, 4),
        "roofline": {
            "bound": "mfma",
            "kernel": f"attn_fwd_kernel ({w.dtype}, d_qk={w.d_qk}, d_v={w.d_v})",
            "achieved": round(attn_tflops, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / peak, 4),
            "traffic": None if traffic is None else round(traffic),
            "algorithmic_flops_per_launch": flops,
            "algorithmic_bytes_per_launch": algorithmic_bytes(w),
            "kernel_source_sha256_16": src_hash,
        },
        "pages_context": {"tflops": 2672.0, "hardware": "MI355X", "note": "FP8 d=128 32K Gaussian, "
                          "attention alone, batch and heads not stated on the pages"},
    }
    if args.sustain_s > 0:
        print(f"# sustained run: {args.sustain_s:g} s of attention launches", file=sys.stderr, flush=True)
        rec["sustained"] = sustained(args.sustain_s, attention, flops, stream, peak)
    else:
        rec["sustained"] = None
    rec["attention_plain_q_scale"] = None
    if w.dtype == "fp8" and not args.no_plain_q_scale:
        rec["attention_plain_q_scale"] = plain_q_scale_leg(args.steps, w, q32, k32, codes, scales, o, flags, flops,
                                                           peak, sm_scale, stream)
    if not args.no_cpu_baseline:
        print("# cpu baseline (fp64 oracle, four head slices)", file=sys.stderr, flush=True)
        nh = min(4, w.Hq)
        rec["cpu_baseline"] = cpu_baseline(w, q, k, v, n_heads=nh, hadamard=args.hadamard,
                                           o_gpu=o[0, :, 0:nh].float().cpu().numpy(),
                                           lse_gpu=lse[0, 0:nh].cpu().numpy())
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
