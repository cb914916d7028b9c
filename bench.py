"""Benchmark of the W8A8 scaled-quantized Linear on one MI355X.

A step is one pass of the hot path over the video-DiT FFN pair (X [75600,
5120] BF16, W_up [13824, 5120], W_down [5120, 13824], activation qmax 448):

    quantise X per token -> FP8 GEMM with GELU-tanh epilogue -> G [75600, 13824]
    -> quantise G per token -> FP8 GEMM -> Y [75600, 5120]

with the weights quantised per output channel once, before timing (they are
cached on first use).  Inputs are seeded synthetic data already resident in
HBM.  The JSON line reports whole-step TFLOP/s (4 M N K flops per step), the
roofline of the dominant kernel (the up-projection GEMM, timed with HIP events
on the stream it runs on), the oracle timed on host cores on a row sample,
and per-workload extras (image-DiT FFN-up fused Linear, block-scaled FP8,
INT8, quantiser GB/s).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-extras] [--no-cpu] [--no-clock]

Measurement helpers (no bench line): --kernel-pass REPS launches every timed
kernel REPS times for rocprofv3 counter passes; --copy-calibration copies
1 GiB (the FETCH_SIZE / WRITE_SIZE scale); --summarize-trace,
--summarize-counters and --traffic-record turn rocprofv3 CSVs into the
tables and the traffic record kept under profiles/.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0     # MI355X dense FP8 MFMA
INT8_PEAK_TOPS = 5000.0      # MI355X dense INT8 MFMA
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def dev_bf16(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


class EventTimer:
    """Per-kernel durations from HIP events recorded on the launch stream."""

    def __init__(self, torch, stream):
        self.torch = torch
        self.stream = stream
        self.pairs: dict[str, list] = {}

    def run(self, name, fn):
        s = self.torch.cuda.Event(enable_timing=True)
        e = self.torch.cuda.Event(enable_timing=True)
        s.record(self.stream)
        out = fn()
        e.record(self.stream)
        self.pairs.setdefault(name, []).append((s, e))
        return out

    def ms(self, name) -> list[float]:
        return [s.elapsed_time(e) for s, e in self.pairs.get(name, [])]

    def clear(self):
        self.pairs.clear()


def measured_traffic(prefix: str, grid: int, source: str = "gemm.hip"):
    """HBM bytes per dispatch of the library kernel whose name starts with
    `prefix` and whose grid has `grid` threads, from the committed rocprofv3
    counter record, or None when the kernel's source file has changed since
    it was taken (or the record holds no such kernel)."""
    import hashlib

    rec_path = os.path.join(ROOT, "profiles", "traffic_kernel_pass.json")
    src = os.path.join(ROOT, "int8_w8a8_quantized_amd", "csrc", source)
    try:
        rec = json.load(open(rec_path))
        key = source.split(".")[0] + "_source_sha256"
        if hashlib.sha256(open(src, "rb").read()).hexdigest() != rec[key]:
            return None
        for name, r in rec["kernels"].items():
            if name.startswith(prefix) and name.endswith(f" grid={grid}"):
                return int(r["read_bytes"] + r["write_bytes"])
    except (OSError, KeyError, ValueError):
        pass
    return None


def quant_bytes(m, k, group=0):
    return 3 * m * k + 4 * m * (k // group if group else 1)


def time_calls(torch, stream, fn, reps=20, warmup=5):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = []
    for _ in range(reps):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record(stream)
        fn()
        e.record(stream)
        evs.append((s, e))
    torch.cuda.synchronize()
    t = sorted(s.elapsed_time(e) for s, e in evs)
    return t[len(t) // 2], t[0]


INFINITY_CACHE_BYTES = 256 << 20   # MI355X last-level (Infinity) cache


def cache_note(nbytes):
    """Whether a kernel's input alone fits the Infinity Cache (a repeated
    call then reads it from there: a "hot" figure)."""
    fits = nbytes <= INFINITY_CACHE_BYTES
    return f"{'hot' if fits else 'cold'} (input {nbytes / 2**20:.0f} MiB, Infinity Cache 256 MiB)"


def time_cold(torch, stream, x, call, reps=20, warmup=5):
    """Median / min of call(x_i) over rotating copies x_i of x whose total
    size is at least twice the Infinity Cache, so each call reads its input
    from HBM (a "cold" figure)."""
    n = max(2, -(-2 * INFINITY_CACHE_BYTES // (x.numel() * x.element_size())))
    copies = [x.clone() for _ in range(n)]
    i = [0]

    def fn():
        call(copies[i[0] % n])
        i[0] += 1

    out = time_calls(torch, stream, fn, reps, warmup)
    del copies
    torch.cuda.empty_cache()
    return out, n


def sample_sclk(torch, fn, seconds=3.0):
    """Shader clock while fn runs back to back: amd-smi sampled from a second
    thread, averaged over the XCDs, after a 0.5 s ramp.  None without amd-smi."""
    import shutil
    import subprocess
    import threading

    if shutil.which("amd-smi") is None:
        return None
    samples, stop = [], threading.Event()

    def worker():
        t_start = time.perf_counter()
        while not stop.is_set():
            try:
                r = subprocess.run(["amd-smi", "metric", "--clock", "--json"], capture_output=True,
                                   text=True, timeout=10)
                d = json.loads(r.stdout)
                d = d["gpu_data"][0] if isinstance(d, dict) else d[0]
                clk = [v["clk"]["value"] for k, v in d["clock"].items() if k.startswith("gfx_")]
                if clk and time.perf_counter() - t_start > 0.5:
                    samples.append(float(np.mean(clk)))
            except Exception:  # noqa: BLE001 -- an unreadable sample is skipped
                time.sleep(0.1)

    th = threading.Thread(target=worker, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=15)
    if not samples:
        return None
    return {"median_mhz": round(float(np.median(samples)), 1), "min_mhz": round(min(samples), 1),
            "max_mhz": round(max(samples), 1), "samples": len(samples),
            "during": "the up GEMM + GELU run back to back for 3 s (amd-smi, mean over 8 XCDs)"}


def quality_report(torch, x, w_up, w_dn, g, y, rows):
    """E_max / E_rel of the quantised step's outputs on the first `rows`
    tokens against FP32 GEMMs of the unquantised BF16 operands."""
    def gelu_tanh(t):
        return 0.5 * t * (1.0 + torch.tanh(0.7978845608028654 * (t + 0.044715 * t * t * t)))

    def measures(got, ref):
        d = (got.double() - ref.double())
        return {"E_max": float(d.abs().max()), "E_rel": float(d.norm() / ref.double().norm())}

    xr = x[:rows].float()
    g_ref = gelu_tanh(xr @ w_up.float().t().contiguous())
    y_ref = g_ref.bfloat16().float() @ w_dn.float().t().contiguous()
    out = {"rows": rows, "reference": "FP32 GEMMs of the unquantised BF16 operands",
           "up_gelu": measures(g[:rows].float(), g_ref), "pair": measures(y[:rows].float(), y_ref)}
    del xr, g_ref, y_ref
    torch.cuda.empty_cache()
    return out


def quality_linear(torch, x, w, y, rows, gelu=False):
    """E_max / E_rel (TeleFuser "Quantization", "Validation") of a quantised
    Linear's BF16 output y on the first `rows` rows against the FP32 GEMM of
    the unquantised BF16 operands (GELU-tanh after it when gelu)."""
    r = min(rows, x.shape[0])
    ref = x[:r].float() @ w.float().t().contiguous()
    if gelu:
        ref = 0.5 * ref * (1.0 + torch.tanh(0.7978845608028654 * (ref + 0.044715 * ref ** 3)))
    d = y[:r].double() - ref.double()
    out = {"rows": r, "E_max": float(d.abs().max()), "E_rel": float(d.norm() / ref.double().norm())}
    del ref, d
    return out


def vendor_reference(torch, stream, qx, sx, wq_up, ws_up, qg, sg, wq_dn, ws_dn):
    """The vendor library's FP8 GEMM on the same codes and scales:
    torch._scaled_mm (hipBLASLt) with row-wise activation and column-wise
    weight scales and BF16 output, no bias and no GELU; median of 20 calls
    for the up and down projections of the step."""
    out = {"library": "torch._scaled_mm (hipBLASLt), row/column scales, BF16 out, no epilogue"}
    f8 = torch.float8_e4m3fn
    for name, a, sa, b, sb in (("up", qx, sx, wq_up, ws_up), ("down", qg, sg, wq_dn, ws_dn)):
        A, B = a.view(f8), b.view(f8).t()
        M, K, N = A.shape[0], A.shape[1], B.shape[1]

        def fn():
            return torch._scaled_mm(A, B, scale_a=sa[:, None], scale_b=sb[None, :],
                                    out_dtype=torch.bfloat16)
        try:
            fn()
            med, _ = time_calls(torch, stream, fn)
        except Exception as e:  # noqa: BLE001 -- reported, not fatal
            out[name] = {"error": str(e)[:200]}
            continue
        tf = 2.0 * M * N * K / med / 1e9
        out[name] = {"ms": med, "tflops": tf, "frac_fp8_peak": tf / FP8_PEAK_TFLOPS}
        torch.cuda.empty_cache()
    return out


def hbm_reference(torch, stream, g):
    """What plain streaming kernels reach on the quantisers' traffic: torch's
    BF16 -> E4M3FN cast of G (2 bytes read, 1 written per element: the
    quantiser's mix without the absmax) and a device copy of G (1:1); median
    of 20, bytes as moved."""
    out = {}
    f8 = torch.empty(g.shape, dtype=torch.float8_e4m3fn, device="cuda")
    med, _ = time_calls(torch, stream, lambda: f8.copy_(g))
    out["cast_bf16_to_e4m3fn_2to1"] = {"ms": med, "gbs": 3 * g.numel() / med / 1e6}
    del f8
    g2 = torch.empty_like(g)
    med, _ = time_calls(torch, stream, lambda: g2.copy_(g))
    out["copy_1to1"] = {"ms": med, "gbs": 4 * g.numel() / med / 1e6}
    del g2
    for v in out.values():
        v["frac_hbm"] = v["gbs"] / HBM_PEAK_GBS
    out["tensor"] = f"G [{g.shape[0]}, {g.shape[1]}] BF16 ({2 * g.numel() / 2**20:.0f} MiB)"
    torch.cuda.empty_cache()
    return out


def extras(torch, tfq, synth, stream):
    """Secondary workloads, each timed on its own (median of 20 after 5 warmup)."""
    out = {}
    # image-DiT FFN-up: one fused call (quantise X + GEMM)
    log("extras: c3_image_dit")
    d = synth.make("c3_image_dit")
    M, K, N = d["spec"].M, d["spec"].K, d["spec"].N
    x, w = dev_bf16(d["x"], torch), dev_bf16(d["w"], torch)
    del d
    wq, ws = tfq.tfq_quantize_weight_per_channel(w, "fp8", 448.0)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    need = tfq.tfq_quant_linear_workspace_bytes(M, K, "fp8", 0)
    wsp = torch.empty(need, dtype=torch.uint8, device="cuda")
    med, best = time_calls(torch, stream, lambda: tfq.tfq_quant_linear_fused(
        x, wq, ws, "fp8", 448.0, 0, None, None, y, wsp))
    fl = 2.0 * M * N * K
    out["c3_image_dit_fused_linear"] = {"ms": med, "ms_min": best, "tflops": fl / med / 1e9,
                                        "frac_fp8_peak": fl / med / 1e9 / FP8_PEAK_TFLOPS,
                                        "quality": quality_linear(torch, x, w, y, 2048)}
    qa, sa = tfq.tfq_quantize_rows(x, "fp8", 448.0)
    med, _ = time_calls(torch, stream, lambda: tfq.tfq_quantize_rows(x, "fp8", 448.0, 0, qa, sa))
    gbs = quant_bytes(M, K) / med / 1e6
    out["c3_quantize_x"] = {"ms": med, "gbs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
                            "cache": cache_note(M * K * 2)}
    (med, _), n = time_cold(torch, stream, x, lambda t: tfq.tfq_quantize_rows(t, "fp8", 448.0, 0,
                                                                              qa, sa))
    gbs = quant_bytes(M, K) / med / 1e6
    out["c3_quantize_x_cold"] = {"ms": med, "gbs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
                                 "cache": f"cold ({n} rotating input copies)"}
    med, _ = time_calls(torch, stream, lambda: tfq.tfq_scaled_mm_fp8(qa, sa, wq, ws, 0, None,
                                                                      None, y))
    out["c3_gemm"] = {"ms": med, "tflops": fl / med / 1e9,
                      "frac_fp8_peak": fl / med / 1e9 / FP8_PEAK_TFLOPS}
    del x, w, wq, ws, y, wsp, qa, sa

    # block-scaled FP8
    log("extras: c5_block_fp8")
    d = synth.make("c5_block_fp8")
    M, K, N = d["spec"].M, d["spec"].K, d["spec"].N
    x, w = dev_bf16(d["x"], torch), dev_bf16(d["w"], torch)
    del d
    wq, ws = tfq.tfq_quantize_weight_per_channel(w, "fp8", 448.0, 128)
    qa, sa = tfq.tfq_quantize_rows(x, "fp8", 448.0, 128)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    med, _ = time_calls(torch, stream, lambda: tfq.tfq_quantize_rows(x, "fp8", 448.0, 128, qa, sa))
    gbs = quant_bytes(M, K, 128) / med / 1e6
    out["c5_quantize_x_groups"] = {"ms": med, "gbs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
                                   "cache": cache_note(M * K * 2)}
    (med, _), n = time_cold(torch, stream, x, lambda t: tfq.tfq_quantize_rows(t, "fp8", 448.0, 128,
                                                                              qa, sa))
    gbs = quant_bytes(M, K, 128) / med / 1e6
    out["c5_quantize_x_groups_cold"] = {"ms": med, "gbs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
                                        "cache": f"cold ({n} rotating input copies)"}
    fl = 2.0 * M * N * K
    med, _ = time_calls(torch, stream, lambda: tfq.tfq_scaled_mm_fp8(qa, sa, wq, ws, 128, None,
                                                                      None, y))
    out["c5_block_gemm"] = {"ms": med, "tflops": fl / med / 1e9,
                            "frac_fp8_peak": fl / med / 1e9 / FP8_PEAK_TFLOPS,
                            "quality": quality_linear(torch, x, w, y, 2048)}
    del x, w, wq, ws, y, qa, sa

    # INT8
    log("extras: c2_int8")
    d = synth.make("c2_int8")
    M, K, N = d["spec"].M, d["spec"].K, d["spec"].N
    x, w = dev_bf16(d["x"], torch), dev_bf16(d["w"], torch)
    del d
    wq, ws = tfq.tfq_quantize_weight_per_channel(w, "int8", 127.0)
    qa, sa = tfq.tfq_quantize_rows(x, "int8", 127.0)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    med, _ = time_calls(torch, stream, lambda: tfq.tfq_quantize_rows(x, "int8", 127.0, 0, qa, sa))
    gbs = quant_bytes(M, K) / med / 1e6
    out["c2_quantize_x"] = {"ms": med, "gbs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
                            "cache": cache_note(M * K * 2)}
    (med, _), n = time_cold(torch, stream, x, lambda t: tfq.tfq_quantize_rows(t, "int8", 127.0, 0,
                                                                              qa, sa))
    gbs = quant_bytes(M, K) / med / 1e6
    out["c2_quantize_x_cold"] = {"ms": med, "gbs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
                                 "cache": f"cold ({n} rotating input copies)"}
    fl = 2.0 * M * N * K
    med, _ = time_calls(torch, stream, lambda: tfq.tfq_scaled_mm_int8(qa, sa, wq, ws, None, None,
                                                                       True, False, y))
    out["c2_int8_gemm"] = {"ms": med, "tops": fl / med / 1e9,
                           "frac_int8_peak": fl / med / 1e9 / INT8_PEAK_TOPS,
                           "quality": quality_linear(torch, x, w, y, 2048)}
    del x, w, wq, ws, y, qa, sa

    # the tiny FP8 Linear (parity workload; quality only, it is launch-bound)
    d = synth.make("c1_tiny_fp8")
    x, w = dev_bf16(d["x"], torch), dev_bf16(d["w"], torch)
    wq, ws = tfq.tfq_quantize_weight_per_channel(w, "fp8", 448.0)
    y = tfq.tfq_quant_linear_fused(x, wq, ws, "fp8", 448.0)
    qa, sa = tfq.tfq_quantize_rows(x, "fp8", 448.0)
    # a 128 x 256 quantisation (98 KB): the event-timed cost of a call whose
    # data movement is negligible, for reading the small quantisers above
    med, _ = time_calls(torch, stream, lambda: tfq.tfq_quantize_rows(x, "fp8", 448.0, 0, qa, sa))
    out["c1_tiny_fp8"] = {"quality": quality_linear(torch, x, w, y, 128),
                          "quantize_x_ms": med}
    return out


FP4_PEAK_TFLOPS = 10100.0  # MI355X dense FP4 (and FP6) MFMA


def mx_pair(torch, tfq, stream, x, w_up, w_dn, g, y, bits=8):
    """The same FFN pair in MXFP8 (bits 8), MXFP6 with E2M3 elements (bits 6)
    or MXFP4 (bits 4): E8M0 scale per 32 elements, scales applied by the
    scaled MFMA; each call timed on its own (median of 20)."""
    log(f"extras: c4 FFN pair in MXFP{bits}")
    M, K = x.shape
    N, N2 = w_up.shape[0], w_dn.shape[0]
    quant = {8: tfq.tfq_quantize_mx, 4: tfq.tfq_quantize_mxfp4,
             6: lambda t, *o: tfq.tfq_quantize_mxfp6(t, "e2m3", *o)}[bits]
    mm = {8: tfq.tfq_scaled_mm_mxfp8, 4: tfq.tfq_scaled_mm_mxfp4,
          6: lambda *a: tfq.tfq_scaled_mm_mxfp6(*a[:4], "e2m3", *a[4:])}[bits]
    peak = FP8_PEAK_TFLOPS if bits == 8 else FP4_PEAK_TFLOPS
    wq_up, ws_up = quant(w_up)
    wq_dn, ws_dn = quant(w_dn)
    qx, sx = quant(x)
    qg, sg = quant(g)
    out = {}
    ms_qx, _ = time_calls(torch, stream, lambda: quant(x, qx, sx))
    ms_up, _ = time_calls(torch, stream, lambda: mm(qx, sx, wq_up, ws_up, None, "gelu_tanh", g))
    ms_qg, _ = time_calls(torch, stream, lambda: quant(g, qg, sg))
    ms_dn, _ = time_calls(torch, stream, lambda: mm(qg, sg, wq_dn, ws_dn, None, None, y))
    # 2 B in, then 1 B (MXFP8), 3/4 B (MXFP6) or 1/2 B (MXFP4) of code and
    # 1/32 B of scale per element
    mxq = lambda m, k: 2 * m * k + m * k * bits // 8 + m * k // 32  # noqa: E731
    fl = 2.0 * M * N * K
    out["quant_x"] = {"ms": ms_qx, "gbs": mxq(M, K) / ms_qx / 1e6}
    out["gemm_up_gelu"] = {"ms": ms_up, "tflops": fl / ms_up / 1e9,
                           "frac_peak": fl / ms_up / 1e9 / peak}
    out["quant_g"] = {"ms": ms_qg, "gbs": mxq(M, N) / ms_qg / 1e6}
    out["gemm_down"] = {"ms": ms_dn, "tflops": 2.0 * M * N2 * N / ms_dn / 1e9,
                        "frac_peak": 2.0 * M * N2 * N / ms_dn / 1e9 / peak}
    step = ms_qx + ms_up + ms_qg + ms_dn
    out["step_ms_sum_of_medians"] = step
    out["step_tflops"] = 4.0 * M * N * K / step / 1e9
    # g and y now hold this format's up and down outputs
    out["quality"] = quality_report(torch, x, w_up, w_dn, g, y, rows=2048)
    return out


def moe_layer(torch, tfq, stream):
    """A routed FFN-up layer at video-DiT size: 75600 tokens, 8 experts of
    [13824, 5120], top-2 routing with skewed expert loads.  Synthetic and
    seeded, generated on the GPU (torch generator, seed 0); the routing (a
    sort by expert) is set up outside the timed calls.  Timed: the gathered
    per-row quantisation of the 151200 routed rows and the grouped GEMM with
    the GELU epilogue (median of 20 each)."""
    log("extras: moe_video_dit_ffn_up (8 experts, top-2)")
    T, K, N, E, topk = 75600, 5120, 13824, 8, 2
    g = torch.Generator(device="cuda").manual_seed(0)
    x = torch.randn((T, K), generator=g, device="cuda").to(torch.bfloat16)
    p = torch.rand(E, generator=g, device="cuda") ** 3 + 0.02  # skewed expert popularity
    choice = torch.multinomial(p.expand(T, E), topk, replacement=False, generator=g)
    expert = choice.reshape(-1)
    order = torch.sort(expert, stable=True).indices
    row_index = (order // topk).to(torch.int32)
    loads = torch.bincount(expert, minlength=E)
    off = torch.zeros(E + 1, dtype=torch.int32, device="cuda")
    off[1:] = torch.cumsum(loads, 0).to(torch.int32)
    M = T * topk
    wq = torch.empty((E, N, K), dtype=torch.uint8, device="cuda")
    ws = torch.empty((E, N), dtype=torch.float32, device="cuda")
    for e in range(E):
        w = (torch.randn((N, K), generator=g, device="cuda") * 0.015).to(torch.bfloat16)
        tfq.tfq_quantize_weight_per_channel(w, "fp8", 448.0, 0, wq[e], ws[e])
        del w
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ms_q, _ = time_calls(torch, stream, lambda: tfq.tfq_quantize_rows_gather(
        x, row_index, "fp8", 448.0, 0, qa, sa))
    ms_g, _ = time_calls(torch, stream, lambda: tfq.tfq_grouped_scaled_mm_fp8(
        qa, sa, wq, ws, off, None, "gelu_tanh", y))
    fl = 2.0 * M * N * K
    out = {"tokens": T, "experts": E, "topk": topk, "K": K, "N": N,
           "expert_rows": loads.tolist(),
           "gather_quantize": {"ms": ms_q, "gbs": (2 * M * K + M * K + 4 * M) / ms_q / 1e6},
           "grouped_gemm_gelu": {"ms": ms_g, "tflops": fl / ms_g / 1e9,
                                 "frac_fp8_peak": fl / ms_g / 1e9 / FP8_PEAK_TFLOPS}}
    del x, wq, ws, qa, sa, y
    torch.cuda.empty_cache()
    return out


def kv_cache(torch, tfq, stream):
    """FP8 KV cache at video-DiT attention size: K [75600 tokens, 40 heads,
    128] BF16 stored into a cache (slots in reverse token order) and loaded
    back to BF16 in a random order; synthetic N(0,1), torch generator seed 0.
    HBM bytes per call: store 2 + 1 per element + 4 per vector + 4 per token;
    load 1 + 2 per element + 4 per vector + 4 per token."""
    log("extras: kv_cache_video_dit (75600 x 40 x 128)")
    T, H, D = 75600, 40, 128
    g = torch.Generator(device="cuda").manual_seed(0)
    kv = torch.randn((T, H, D), generator=g, device="cuda").to(torch.bfloat16)
    slot = torch.arange(T - 1, -1, -1, dtype=torch.int32, device="cuda")
    order = torch.randperm(T, generator=g, device="cuda").to(torch.int32)
    cache = torch.empty((T, H, D), dtype=torch.uint8, device="cuda")
    scale = torch.empty((T, H), dtype=torch.float32, device="cuda")
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    E = T * H * D
    ms_s, _ = time_calls(torch, stream, lambda: tfq.tfq_kv_cache_store(kv, slot, cache, scale))
    ms_l, _ = time_calls(torch, stream, lambda: tfq.tfq_kv_cache_load(cache, scale, order,
                                                                       out=out))
    res = {"store": {"ms": ms_s, "gbs": (3 * E + 4 * T * H + 4 * T) / ms_s / 1e6},
           "load_bf16": {"ms": ms_l, "gbs": (3 * E + 4 * T * H + 4 * T) / ms_l / 1e6}}
    for k in res:
        res[k]["frac_hbm"] = res[k]["gbs"] / HBM_PEAK_GBS
    del kv, cache, scale, out
    torch.cuda.empty_cache()
    return res


def cpu_baseline(d, rows_sample: int):
    """The oracle on host cores over a row sample of the same FFN-pair step:
    quantise the sampled X rows, up GEMM + GELU, BF16 round, quantise G rows,
    down GEMM.  Returns (TFLOP/s, seconds, threads)."""
    import oracle as orc
    import synth

    x = np.ascontiguousarray(d["x"][:rows_sample])
    wq_up, ws_up = orc.quantize_rows(d["w"], "fp8", 448.0)
    wq_dn, ws_dn = orc.quantize_rows(d["w_down"], "fp8", 448.0)
    t0 = time.perf_counter()
    qx, sx = orc.quantize_rows(x, "fp8", 448.0)
    g = orc.linear_ref(qx, sx, wq_up, ws_up, "fp8", gelu=True)
    gb = synth.to_bf16_bits(g.astype(np.float32))
    qg, sg = orc.quantize_rows(gb, "fp8", 448.0)
    orc.linear_ref(qg, sg, wq_dn, ws_dn, "fp8")
    sec = time.perf_counter() - t0
    M, N = rows_sample, d["w"].shape[0]
    K = d["w"].shape[1]
    flops = 4.0 * M * N * K
    return flops / sec / 1e12, sec, orc.num_threads()


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_per_config(synth, d_c4, g_host):
    """The oracle on the host cores for every workload: the quantiser at full
    size (X of each workload, and the video-DiT G), GB/s over the same
    algorithmic bytes as the GPU; the Linear on all rows of the tiny and INT8
    workloads and on a 256-row sample of the image-DiT and block-scaled ones
    (seconds for the sample and the linear extrapolation to all rows).  About
    10 s on 16 host cores."""
    import oracle as orc

    out = {"quantize": {}, "linear": {}}

    def tq(name, bits, qtype, qmax, group=0):
        t0 = time.perf_counter()
        res = orc.quantize_rows(bits, qtype, qmax, group)
        sec = time.perf_counter() - t0
        m, k = bits.shape
        out["quantize"][name] = {"gbs": round(quant_bytes(m, k, group) / sec / 1e9, 3),
                                 "seconds": round(sec, 3), "sample": f"full [{m}, {k}]"}
        return res

    tq("c4_video_dit_x", d_c4["x"], "fp8", 448.0)
    if g_host is not None:
        tq("c4_video_dit_g", g_host, "fp8", 448.0)
    for wl, qt, qmax, grp, rows in (("c1_tiny_fp8", "fp8", 448.0, 0, None),
                                    ("c2_int8", "int8", 127.0, 0, None),
                                    ("c3_image_dit", "fp8", 448.0, 0, 256),
                                    ("c5_block_fp8", "fp8", 448.0, 128, 256)):
        d = synth.make(wl)
        qa, sa = tq(wl + "_x", d["x"], qt, qmax, grp)
        if grp:
            qw, sw = orc.quantize_blocks(d["w"], qt, qmax, grp)
        else:
            qw, sw = orc.quantize_rows(d["w"], qt, qmax)
        M, K, N = d["spec"].M, d["spec"].K, d["spec"].N
        sel = None if rows is None else np.arange(rows)
        t0 = time.perf_counter()
        if qt == "int8":
            orc.int8_linear(qa, sa, qw, sw, rows=sel)
        else:
            orc.linear_ref(qa, sa, qw, sw, "fp8", grp, rows=sel)
        sec = time.perf_counter() - t0
        r = M if rows is None else rows
        out["linear"][wl] = {"tflops": round(2.0 * r * N * K / sec / 1e12, 6), "seconds": round(sec, 3),
                             "sample": f"{r} of {M} rows" + (" (all)" if r == M else ""),
                             "seconds_all_rows_extrapolated": round(sec * M / r, 1)}
        del d, qa, sa, qw, sw
    return out


def kernel_pass(torch, tfq, synth, reps):
    """Every kernel bench.py times, `reps` launches in a row, on the same
    seeded inputs and with the heuristic launch configurations: a short
    program for rocprofv3 counter passes (the full bench runs each workload
    for minutes under a counter pass).  Order: video-DiT FFN pair (quantise X,
    up GEMM + GELU, quantise G, down GEMM), the same pair's GEMMs in MXFP8,
    MXFP6 E2M3 and MXFP4, image-DiT fused Linear (quantise + GEMM),
    block-scaled FP8 (1x128-group quantise + GEMM), INT8 (quantise + GEMM)."""
    tfq.tfq_set_autotune(0)
    d = synth.make("c4_video_dit")
    x, w_up, w_dn = (dev_bf16(d[k], torch) for k in ("x", "w", "w_down"))
    del d
    wq_up, ws_up = tfq.tfq_quantize_weight_per_channel(w_up, "fp8", 448.0)
    wq_dn, ws_dn = tfq.tfq_quantize_weight_per_channel(w_dn, "fp8", 448.0)
    qx, sx = tfq.tfq_quantize_rows(x, "fp8", 448.0)
    g = tfq.tfq_scaled_mm_fp8(qx, sx, wq_up, ws_up, 0, None, "gelu_tanh")
    qg, sg = tfq.tfq_quantize_rows(g, "fp8", 448.0)
    y = tfq.tfq_scaled_mm_fp8(qg, sg, wq_dn, ws_dn)
    for name, fn in (("c4 quantise X", lambda: tfq.tfq_quantize_rows(x, "fp8", 448.0, 0, qx, sx)),
                     ("c4 up GEMM + GELU", lambda: tfq.tfq_scaled_mm_fp8(
                         qx, sx, wq_up, ws_up, 0, None, "gelu_tanh", g)),
                     ("c4 quantise G", lambda: tfq.tfq_quantize_rows(g, "fp8", 448.0, 0, qg, sg)),
                     ("c4 down GEMM", lambda: tfq.tfq_scaled_mm_fp8(qg, sg, wq_dn, ws_dn, 0, None,
                                                                     None, y))):
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        log(f"kernel pass: {name} x{reps}")
    del qx, sx, qg, sg, wq_up, ws_up, wq_dn, ws_dn
    torch.cuda.empty_cache()
    # the same pair in MXFP8, MXFP6 E2M3 and MXFP4 (GEMMs only)
    for bits in (8, 6, 4):
        quant = {8: tfq.tfq_quantize_mx, 4: tfq.tfq_quantize_mxfp4,
                 6: lambda t: tfq.tfq_quantize_mxfp6(t, "e2m3")}[bits]
        mm = {8: tfq.tfq_scaled_mm_mxfp8, 4: tfq.tfq_scaled_mm_mxfp4,
              6: lambda *a: tfq.tfq_scaled_mm_mxfp6(*a[:4], "e2m3", *a[4:])}[bits]
        qa, sa = quant(x)
        qu, su = quant(w_up)
        for _ in range(reps):
            mm(qa, sa, qu, su, None, "gelu_tanh", g)
        qg, sg = quant(g)
        qd, sd = quant(w_dn)
        for _ in range(reps):
            mm(qg, sg, qd, sd, None, None, y)
        torch.cuda.synchronize()
        log(f"kernel pass: MXFP{bits} up and down GEMMs x{reps}")
        del qa, sa, qu, su, qg, sg, qd, sd
        torch.cuda.empty_cache()
    del x, g, y, w_up, w_dn
    torch.cuda.empty_cache()
    for wl, qt, qmax, blk in (("c3_image_dit", "fp8", 448.0, 0), ("c5_block_fp8", "fp8", 448.0, 128),
                              ("c2_int8", "int8", 127.0, 0)):
        d = synth.make(wl)
        x, w = dev_bf16(d["x"], torch), dev_bf16(d["w"], torch)
        del d
        wq, ws = tfq.tfq_quantize_weight_per_channel(w, qt, qmax, blk)
        for _ in range(reps):
            if wl == "c3_image_dit":
                tfq.tfq_quant_linear_fused(x, wq, ws, qt, qmax)
            else:
                qa, sa = tfq.tfq_quantize_rows(x, qt, qmax, blk)
                if qt == "int8":
                    tfq.tfq_scaled_mm_int8(qa, sa, wq, ws)
                else:
                    tfq.tfq_scaled_mm_fp8(qa, sa, wq, ws, blk)
        torch.cuda.synchronize()
        log(f"kernel pass: {wl} x{reps}")
        del x, w, wq, ws
        torch.cuda.empty_cache()


def read_counters(paths, library_only=True):
    """{kernel key: {counter: [values]}}, {kernel key: {dispatch: seconds}}
    from rocprofv3 counter_collection.csv files; the key is the demangled
    name without namespace and argument list, plus the grid size."""
    import csv
    import re
    from collections import defaultdict

    vals = defaultdict(lambda: defaultdict(list))
    durs = defaultdict(dict)
    for path in paths:
        for r in csv.DictReader(open(path)):
            k = r["Kernel_Name"]
            if library_only and "tfq::" not in k:
                continue
            k = re.sub(r"^void |tfq::\(anonymous namespace\)::|tfq::", "", k)
            k = re.sub(r"\(.*\)$", "", k).strip()
            key = f"{k} grid={r['Grid_Size']}"
            vals[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
            durs[key][(path, r["Dispatch_Id"])] = (int(r["End_Timestamp"])
                                                   - int(r["Start_Timestamp"])) * 1e-9
    return vals, durs


def traffic_record(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    """HBM bytes per dispatch of every library kernel from a FETCH_SIZE and a
    WRITE_SIZE pass (KiB per dispatch), each scaled by what the same counter
    reads for a 1 GiB device copy.  Prints the JSON record measured_traffic
    reads (with the kernel sources' hashes, so a changed kernel reads as
    unmeasured)."""
    import hashlib

    def copy_kib(path, counter):
        vals, _ = read_counters([path], library_only=False)
        v = [x for k, cs in vals.items() if "copy" in k for x in cs.get(counter, [])]
        return float(np.median(v))

    f_fac = (1 << 30) / (copy_kib(copy_fetch_csv, "FETCH_SIZE") * 1024)
    w_fac = (1 << 30) / (copy_kib(copy_write_csv, "WRITE_SIZE") * 1024)
    fv, _ = read_counters([fetch_csv])
    wv, _ = read_counters([write_csv])
    kernels = {}
    for k in sorted(set(fv) & set(wv)):
        fk, wk = float(np.mean(fv[k]["FETCH_SIZE"])), float(np.mean(wv[k]["WRITE_SIZE"]))
        kernels[k] = {"fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                      "read_bytes": int(fk * 1024 * f_fac), "write_bytes": int(wk * 1024 * w_fac)}
    src = os.path.join(ROOT, "int8_w8a8_quantized_amd", "csrc")
    sha = lambda f: hashlib.sha256(open(os.path.join(src, f), "rb").read()).hexdigest()  # noqa: E731
    rec = {"note": "HBM bytes per dispatch: rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (separate "
                   "runs, KiB per dispatch) scaled by a 1 GiB device copy's readings",
           "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4),
           "gemm_source_sha256": sha("gemm.hip"), "quantize_source_sha256": sha("quantize.hip"),
           "kernels": kernels}
    print(json.dumps(rec, indent=1))


def summarize_trace(stats_csv):
    """Markdown table of a rocprofv3 --stats kernel_stats.csv: the library's
    kernels one by one, everything else (torch's kernels of the error
    report and set-up) summed in one line."""
    import csv
    import re

    def short(name):
        name = re.sub(r"^void |tfq::\(anonymous namespace\)::|tfq::", "", name)
        return re.sub(r"\(.*\)$", "", name).strip()

    # per-dispatch durations from the kernel trace next to the stats file,
    # for the median (and the median of the grid's largest dispatches)
    trace = stats_csv.replace("_kernel_stats.csv", "_kernel_trace.csv")
    durs = {}
    if trace != stats_csv and os.path.exists(trace):
        for r in csv.DictReader(open(trace)):
            if "tfq::" in r["Kernel_Name"]:
                durs.setdefault(short(r["Kernel_Name"]), []).append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    rows, other = [], [0, 0]
    for r in csv.DictReader(open(stats_csv)):
        name = r["Name"]
        if "tfq::" not in name:
            other[0] += int(r["Calls"])
            other[1] += int(r["TotalDurationNs"])
            continue
        n = short(name)
        med = float(np.median(durs[n])) if n in durs else float("nan")
        rows.append((n, int(r["Calls"]), float(r["AverageNs"]) / 1e3, med, float(r["MinNs"]) / 1e3,
                     float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    print("| kernel | calls | average (us) | median (us) | min (us) | max (us) | share of kernel time |")
    print("|---|---|---|---|---|---|---|")
    for n, c, a, md, lo, hi, pc in rows:
        print(f"| {n} | {c} | {a:.1f} | {md:.1f} | {lo:.1f} | {hi:.1f} | {pc:.2f}% |")
    print(f"| (other kernels) | {other[0]} | | | | | total {other[1] / 1e6:.1f} ms |")


def summarize_counters(paths):
    """Per-kernel means of rocprofv3 --pmc CSVs (counter_collection.csv of
    one or more passes), keyed by kernel name and grid size, with derived
    figures.  MI355X sums these counters over its units, so:
      clock = GRBM_GUI_ACTIVE / 8 XCDs / duration;
      MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / (SQ_CYCLES / 32 SEs)
        (the share of shader cycles each SIMD's matrix core is busy);
      SQ_BUSY_CYCLES / (SQ_CYCLES): the share of cycles the sequencers hold waves;
      wait share = SQ_WAIT_ANY / SQ_WAVE_CYCLES (per wave);
      LDS bank conflicts: SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS (conflict
        cycles per cycle of LDS instruction activity).
    GRBM_GUI_ACTIVE also counts the GPU's busy time around a dispatch, so
    the clock figure reads high (even above 2.4 GHz) for kernels of tens of
    microseconds; it is meaningful for the GEMMs.  Prints a markdown table."""
    vals, durs = read_counters(paths)
    rows = []
    for key, cs in vals.items():
        m = {c: float(np.mean(v)) for c, v in cs.items()}
        dur = float(np.mean(list(durs[key].values())))
        row = {"kernel": key, "dispatches": len(durs[key]), "us": dur * 1e6}
        if "GRBM_GUI_ACTIVE" in m:
            row["clock_ghz"] = m["GRBM_GUI_ACTIVE"] / 8 / dur / 1e9
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m and "SQ_CYCLES" in m:
            row["mfma_busy"] = m["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 / (m["SQ_CYCLES"] / 32)
        if "SQ_BUSY_CYCLES" in m and "SQ_CYCLES" in m:
            row["sq_busy"] = m["SQ_BUSY_CYCLES"] / m["SQ_CYCLES"]
        if "SQ_WAIT_ANY" in m and "SQ_WAVE_CYCLES" in m:
            row["wait_any_per_wave"] = m["SQ_WAIT_ANY"] / m["SQ_WAVE_CYCLES"]
        if "SQ_LDS_BANK_CONFLICT" in m and "SQ_ACTIVE_INST_LDS" in m:
            row["lds_conflict_per_lds_active"] = m["SQ_LDS_BANK_CONFLICT"] / max(
                m["SQ_ACTIVE_INST_LDS"], 1.0)
        row["raw"] = m
        rows.append(row)
    rows.sort(key=lambda r: -r["us"] * r["dispatches"])
    print("| kernel | dispatches | us | clock GHz | MFMA busy | SQ busy | wait/wave "
          "| LDS conflict / LDS active |")
    print("|---|---|---|---|---|---|---|---|")
    f = lambda r, k, fmt: (fmt % r[k]) if k in r else "-"  # noqa: E731
    for r in rows:
        print(f"| {r['kernel']} | {r['dispatches']} | {r['us']:.1f} | {f(r, 'clock_ghz', '%.3f')} "
              f"| {f(r, 'mfma_busy', '%.3f')} | {f(r, 'sq_busy', '%.3f')} "
              f"| {f(r, 'wait_any_per_wave', '%.3f')} | {f(r, 'lds_conflict_per_lds_active', '%.4f')} |")
    print()
    print("Raw per-dispatch means:")
    print()
    for r in rows:
        print(f"* {r['kernel']}: " + ", ".join(f"{c} {v:.4g}" for c, v in sorted(r["raw"].items())))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--qmax", type=float, default=448.0)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-autotune", action="store_true",
                    help="use the fixed heuristic GEMM configurations instead of tuning each "
                         "shape on its first call (during warm-up)")
    ap.add_argument("--cpu-rows", type=int, default=256)
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the 3 s shader-clock sample (amd-smi) after the timed steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device-to-device copy three times (the reference "
                         "kernel for scaling FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--kernel-pass", type=int, default=0, metavar="REPS",
                    help="only launch every timed kernel REPS times in a row (for rocprofv3 "
                         "counter passes) and exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                    help="print per-kernel means and derived figures of rocprofv3 --pmc CSVs "
                         "and exit (no GPU needed)")
    ap.add_argument("--traffic-record", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="print the HBM traffic record of rocprofv3 FETCH_SIZE / WRITE_SIZE "
                         "passes (bench and 1 GiB copy) and exit (no GPU needed)")
    ap.add_argument("--summarize-trace", metavar="STATS_CSV",
                    help="print the library kernels of a rocprofv3 kernel_stats.csv as a "
                         "markdown table and exit (no GPU needed)")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.traffic_record:
        traffic_record(*args.traffic_record)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import int8_w8a8_quantized_amd as tfq
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copied 1 GiB three times")
        return
    if args.kernel_pass:
        kernel_pass(torch, tfq, synth, args.kernel_pass)
        return

    # per-shape GEMM tuning: the first warm-up step tunes every shape of the step
    tfq.tfq_set_autotune(0 if args.no_autotune else 1)
    log("generating c4_video_dit inputs (seeded synthetic)")
    t0 = time.perf_counter()
    d = synth.make("c4_video_dit")
    spec = d["spec"]
    M, K, N, N2 = spec.M, spec.K, spec.N, spec.n_down
    log(f"inputs ready in {time.perf_counter() - t0:.1f}s: X [{M},{K}] W_up [{N},{K}] "
        f"W_down [{N2},{N}]")
    x = dev_bf16(d["x"], torch)
    w_up = dev_bf16(d["w"], torch)
    w_dn = dev_bf16(d["w_down"], torch)
    # one-time weight quantisation (cached on first use), outside the timed region
    wq_up, ws_up = tfq.tfq_quantize_weight_per_channel(w_up, "fp8", 448.0)
    wq_dn, ws_dn = tfq.tfq_quantize_weight_per_channel(w_dn, "fp8", 448.0)
    qx = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sx = torch.empty((M,), dtype=torch.float32, device="cuda")
    g = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    qg = torch.empty((M, N), dtype=torch.uint8, device="cuda")
    sg = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N2), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()

    timer = EventTimer(torch, stream)

    def step(qmax):
        timer.run("quant_x", lambda: tfq.tfq_quantize_rows(x, "fp8", qmax, 0, qx, sx))
        timer.run("gemm_up_gelu", lambda: tfq.tfq_scaled_mm_fp8(qx, sx, wq_up, ws_up, 0, None,
                                                                 "gelu_tanh", g))
        timer.run("quant_g", lambda: tfq.tfq_quantize_rows(g, "fp8", qmax, 0, qg, sg))
        timer.run("gemm_down", lambda: tfq.tfq_scaled_mm_fp8(qg, sg, wq_dn, ws_dn, 0, None, None,
                                                              y))

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step(args.qmax)
    torch.cuda.synchronize()
    timer.clear()
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(args.qmax)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    flops_step = 4.0 * M * N * K
    value = flops_step / (ms_step * 1e-3) / 1e12

    per = {k: float(np.mean(timer.ms(k))) for k in ("quant_x", "gemm_up_gelu", "quant_g",
                                                       "gemm_down")}
    # (the oracle's quantiser is timed on this G at the end)
    g_host = None if args.no_cpu else g.view(torch.int16).cpu().numpy().view(np.uint16)
    up_flops = 2.0 * M * N * K
    achieved = up_flops / (per["gemm_up_gelu"] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": "scaled_gemm fp8 (up projection + GELU epilogue)",
                "achieved": round(achieved, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
                "traffic": measured_traffic("gemm_pipe_kernel<0, 1, true, false, false",
                                            -(-M // 256) * -(-N // 256) * 256),
                "algorithmic_bytes": M * K + N * K + 4 * M + 4 * N + 2 * M * N}
    kernels = {
        "quant_x": {"ms": per["quant_x"], "gbs": quant_bytes(M, K) / per["quant_x"] / 1e6},
        "gemm_up_gelu": {"ms": per["gemm_up_gelu"], "tflops": achieved},
        "quant_g": {"ms": per["quant_g"], "gbs": quant_bytes(M, N) / per["quant_g"] / 1e6},
        "gemm_down": {"ms": per["gemm_down"],
                      "tflops": 2.0 * M * N2 * N / (per["gemm_down"] * 1e-3) / 1e12},
    }
    for kk, nb in (("quant_x", M * K * 2), ("quant_g", M * N * 2)):
        kernels[kk]["frac_hbm"] = kernels[kk]["gbs"] / HBM_PEAK_GBS
        kernels[kk]["cache"] = cache_note(nb)
    for kk, (n_, k_, epi_) in (("gemm_up_gelu", (N, K, "gelu_tanh")), ("gemm_down", (N2, N, None))):
        cfg = tfq.tfq_autotune_lookup("fp8", M, n_, k_, epi_)
        kernels[kk]["config"] = None if cfg is None else {"kernel": cfg[0], "band": cfg[1]}
    log(f"step {ms_step:.3f} ms -> {value:.1f} TFLOP/s; per kernel {json.dumps(per)}")

    # operator error against the unquantised product, E_max = max|y_q - y| and
    # E_rel = ||y_q - y|| / ||y|| (TeleFuser "Quantization", "Validation"), on
    # the first rows of the step just timed (qmax 448); the reference is two
    # FP32 GEMMs of the BF16 inputs (GELU-tanh between them)
    quality = quality_report(torch, x, w_up, w_dn, g, y, rows=2048)

    # the reduced-qmax sweep (LightX2V "模型量化技术", "MiniMax-H3 FP8 FP16
    # 累加"): the same step at activation qmax 14 and 7, 3 timed steps each,
    # with per-kernel times and the operator error of each
    sweep = {}
    for q in (14.0, 7.0):
        step(q)
        torch.cuda.synchronize()
        timer.clear()
        t1 = time.perf_counter()
        for _ in range(3):
            step(q)
        torch.cuda.synchronize()
        per_q = {k: float(np.mean(timer.ms(k))) for k in ("quant_x", "gemm_up_gelu", "quant_g",
                                                            "gemm_down")}
        sweep[str(q)] = {"ms_per_step": (time.perf_counter() - t1) * 1e3 / 3, "kernels_ms": per_q,
                         "quality": quality_report(torch, x, w_up, w_dn, g, y, rows=2048)}
    timer.clear()
    sclk = None
    if not args.no_clock:
        log("shader clock under the up GEMM (amd-smi)")
        sclk = sample_sclk(torch, lambda: tfq.tfq_scaled_mm_fp8(qx, sx, wq_up, ws_up, 0, None,
                                                                "gelu_tanh", g))
    if sclk is not None:
        sclk["frac_fp8_peak_at_this_clock"] = round(
            achieved / (FP8_PEAK_TFLOPS * sclk["median_mhz"] / 2400.0), 4)
    roofline["sclk"] = sclk

    ext = {}
    if not args.no_extras:
        ext["vendor_reference"] = vendor_reference(torch, stream, qx, sx, wq_up, ws_up, qg, sg,
                                                   wq_dn, ws_dn)
        ext["hbm_reference"] = hbm_reference(torch, stream, g)
        ext["c4_mxfp8_pair"] = mx_pair(torch, tfq, stream, x, w_up, w_dn, g, y, 8)
        torch.cuda.synchronize()
        ext["c4_mxfp6_e2m3_pair"] = mx_pair(torch, tfq, stream, x, w_up, w_dn, g, y, 6)
        torch.cuda.synchronize()
        ext["c4_mxfp4_pair"] = mx_pair(torch, tfq, stream, x, w_up, w_dn, g, y, 4)
        torch.cuda.synchronize()
        del x, g, qg, y, qx
        torch.cuda.empty_cache()
        ext.update(extras(torch, tfq, synth, stream))
        ext["moe_video_dit_ffn_up"] = moe_layer(torch, tfq, stream)
        ext["kv_cache_video_dit"] = kv_cache(torch, tfq, stream)

    cpu = None
    if not args.no_cpu:
        log(f"cpu baseline: oracle on {args.cpu_rows} rows of the same step")
        tf, sec, thr = cpu_baseline(d, args.cpu_rows)
        cpu = {"value": round(tf, 6), "unit": "TFLOP/s", "cores": thr, "kind": "oracle",
               "sample": f"{args.cpu_rows} of {M} token rows of the FFN-pair step (quantise X, "
                         f"up GEMM + GELU, quantise G, down GEMM), {sec:.1f} s; all {M} rows "
                         f"extrapolated: {sec * M / args.cpu_rows:.0f} s",
               "cpu_model": cpu_model(), "nproc": os.cpu_count()}
        log("cpu baseline: oracle per workload (quantisers at full size, Linear samples)")
        cpu["per_config"] = cpu_baseline_per_config(synth, d, g_host)

    # operator error by workload and activation qmax
    all_quality = {"c4_video_dit": {str(args.qmax): quality,
                                    **{k: v["quality"] for k, v in sweep.items()}}}
    for key, wl in (("c3_image_dit_fused_linear", "c3_image_dit"), ("c5_block_gemm", "c5_block_fp8"),
                    ("c2_int8_gemm", "c2_int8"), ("c1_tiny_fp8", "c1_tiny_fp8")):
        if key in ext and "quality" in ext[key]:
            all_quality[wl] = {"448.0" if wl != "c2_int8" else "127.0": ext[key]["quality"]}
    out = {
        "metric": "FP8 W8A8 Linear TFLOP/s (% FP8 MFMA peak) + quantize GB/s at DiT shapes",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3fn (fp32 accumulate)",
        "data": "synthetic (seeded; Student-t(4) activations, N(0,0.015) weights)",
        "config": {"workload": "video-DiT FFN pair: X[75600,5120] -> W_up[13824,5120] + "
                               "GELU-tanh -> W_down[5120,13824], per-token/per-channel E4M3FN",
                   "M": M, "K": K, "N_up": N, "N_down": N2, "act_qmax": args.qmax,
                   "autotune": not args.no_autotune,
                   "frac_fp8_peak": round(value / FP8_PEAK_TFLOPS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "quality": all_quality,
        "kernels": kernels,
        "qmax_sweep": sweep,
        "extras": ext,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
