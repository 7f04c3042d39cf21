"""Benchmark of the fused attention forward on one MI355X.

One step = one pass of the whole hot path on one batch of synthetic input:
  * prefill, Llama-2-7B-shaped causal attention (B=4, H=32, N=2048, d=128), and
  * decode, paged GQA (B=8, Hq=32, Hkv=8, d=128, 16-token pages, lengths U[1024, 131072]).
Inputs are seeded, synthetic and resident in HBM before timing starts.  W untimed warmup
steps, then K timed steps bracketed by device synchronisation; each kernel launch is
also bracketed by HIP events on the stream it runs on.

Prints ONE JSON line.  `value` is the prefill throughput in TFLOP/s (algorithmic FLOPs
4*d per visible query-key pair); the decode half of the metric (KV GB/s) is reported in
the `decode` object.  Each carries a `roofline` (dense bf16 MFMA peak for prefill, HBM
peak for decode).  `cpu_baseline` times the CPU oracle over the same prefill and decode
workloads on this host's cores (a process pool).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import attn_inputs as ai  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 4096 FLOP/clk x 2.4 GHz)
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense FP8 MFMA (twice the bf16 rate)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "prefill attention TFLOPS and decode KV GB/s at 1 MI355X, % of roofline"
PREFILL_CFG = "llama2_7b_prefill"
DECODE_CFG = "paged_gqa_decode"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the other workloads (non-causal, 32K and fp16 prefill, contiguous and "
                        "FP8-cache decode, varlen prefill, backward, chunked prefill)")
    p.add_argument("--settle-ms", type=float, default=300.0,
                   help="after the W warmup steps, keep running untimed steps until the warmup "
                        "has lasted this long: the GPU raises its clocks over tens of ms of "
                        "load after an idle spell, and the timed steps should see the steady state")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="after the timed region, run one plain device copy of this many MiB "
                        "(a reference dispatch of known traffic for counter calibration)")
    return p.parse_args()


def to_dev(bits):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def to_dev16(bits):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16)
    return t.cuda()


def kernel_sources_digest() -> str:
    h = hashlib.sha256()
    cdir = os.path.join(ROOT, "io_aware_exact_attention_amd", "csrc")
    for name in sorted(os.listdir(cdir)):
        with open(os.path.join(cdir, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def device_clock_mhz():
    """Peak shader clock of device 0 in MHz, from hipDeviceGetAttribute with
    hipDeviceAttributeClockRate (kHz), asked of the HIP runtime already loaded for the
    library (never a second copy); the enum's value is read from the installed HIP header.
    None when any step is unavailable."""
    try:
        import ctypes
        hdr = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include", "hip",
                           "hip_runtime_api.h")
        src = open(hdr).read()
        i = src.index("typedef enum hipDeviceAttribute_t {")
        body = src[i:src.index("} hipDeviceAttribute_t;", i)]
        body = re.sub(r"/\*.*?\*/", "", re.sub(r"//[^\n]*", "", body), flags=re.S)
        val, names = -1, {}
        for ent in body[body.index("{") + 1:].split(","):
            ent = ent.strip()
            if not ent:
                continue
            if "=" in ent:
                n, e = (x.strip() for x in ent.split("=", 1))
                val = int(e, 0) if re.fullmatch(r"0x[0-9a-fA-F]+|\d+", e) else names[e]
            else:
                n, val = ent, val + 1
            names[n] = val
        lib = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
        khz = ctypes.c_int(0)
        if lib.hipDeviceGetAttribute(ctypes.byref(khz), names["hipDeviceAttributeClockRate"], 0):
            return None
        return khz.value / 1000.0 if khz.value > 0 else None
    except Exception:
        return None


def recorded_traffic(kernel: str):
    """HBM bytes per launch recorded from rocprofv3 counter runs in profiles/, if they
    were taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    if not os.path.exists(path):
        return None
    digest = kernel_sources_digest()
    for line in open(path):
        m = re.match(r"\|\s*" + re.escape(kernel) + r"\s*\|\s*([0-9a-f]+)\s*\|\s*(\d+)\s*\|", line)
        if m and m.group(1) == digest:
            return int(m.group(2))
    return None


def decode_traffic():
    """Split + merge kernel traffic of one decode step, when both were recorded."""
    a = recorded_traffic("decode_split_kernel<128,paged>")
    b = recorded_traffic("decode_merge_kernel<128>")
    return a + b if a is not None and b is not None else None


# ------------------------------------------------------------------------------ workloads
def prefill_setup(name, keep_host=False):
    import torch
    cfg = ai.CONFIGS[name]
    q, k, v = ai.prefill_inputs(cfg)
    if cfg.fp8:   # E4M3 codes stay bytes; O is bf16
        conv = lambda c: torch.from_numpy(np.ascontiguousarray(c)).cuda()
    else:
        conv = to_dev16 if cfg.f16 else to_dev
    dq, dk, dv = conv(q), conv(k), conv(v)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda") if cfg.fp8 else \
        torch.empty_like(dq)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    if keep_host:
        return cfg, (dq, dk, dv, o, lse), (q, k, v)
    return cfg, (dq, dk, dv, o, lse)


def decode_setup(name, keep_host=False):
    import torch
    cfg = ai.CONFIGS[name]
    lens = ai.decode_lengths(cfg)
    q = ai.decode_q(cfg)
    if cfg.paged:
        lay = ai.paged_layout(lens, cfg.page_size, cfg.seed)
        kc = ai.build_paged_cache(cfg, ai.T_K, lens, lay, pad_bits=np.uint16(0))
        vc = ai.build_paged_cache(cfg, ai.T_V, lens, lay, pad_bits=np.uint16(0))
        table = torch.from_numpy(lay.block_table).cuda()
        maxlen = int(lens.max())
    else:
        maxlen = cfg.fixed_len
        kc = ai.build_contig_cache(cfg, ai.T_K, lens, maxlen, pad_bits=np.uint16(0))
        vc = ai.build_contig_cache(cfg, ai.T_V, lens, maxlen, pad_bits=np.uint16(0))
        table = None
    dq = to_dev(q)
    if cfg.kv_fp8:   # E4M3 codes stay bytes
        dkc, dvc = torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda()
    else:
        dkc, dvc = to_dev(kc), to_dev(vc)
    host = (q, kc, vc, lay.block_table, lens) if keep_host and cfg.paged else None
    del kc, vc
    o = torch.empty_like(dq)
    lse = torch.empty((cfg.B, cfg.Hq), dtype=torch.float32, device="cuda")
    seq = torch.from_numpy(lens).cuda()
    if keep_host:
        return cfg, lens, maxlen, (dq, dkc, dvc, table, seq, o, lse), host
    return cfg, lens, maxlen, (dq, dkc, dvc, table, seq, o, lse)


def settle(fn, t_start: float, settle_ms: float) -> int:
    """Run fn (untimed) until settle_ms have passed since t_start (the start of the
    warmup); returns the number of extra calls.  Synchronises every 8 calls so that the
    time waited is GPU time."""
    import torch
    extra = 0
    torch.cuda.synchronize()
    while (time.perf_counter() - t_start) * 1e3 < settle_ms:
        for _ in range(8):
            fn()
        extra += 8
        torch.cuda.synchronize()
    return extra


SETTLE_MS = 300.0


def time_kernel(fn, steps, warmup):
    """Average microseconds per call, from HIP events on the current stream."""
    import torch
    t0 = time.perf_counter()
    for _ in range(warmup):
        fn()
    settle(fn, t0, SETTLE_MS)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(steps)]
    return float(np.mean(per)), float(np.median(per)), float(np.min(per))


# ------------------------------------------------------------------------------ CPU baseline
def cpu_baseline(prefill_host, decode_host):
    """The fp64 oracle as it stands, on this host's cores: a process pool (one BLAS thread
    per worker) over the prefill workload's (b, head, 1,024-row block) units and the paged
    decode workload's (sequence, KV head) units, inputs placed in shared memory first.
    Throughput is the GPU's algorithmic work (FLOPs, bytes) over the pool's wall time."""
    from oracle import pool
    cfg = ai.CONFIGS[PREFILL_CFG]
    q, k, v = prefill_host
    heads = [(b, h) for b in range(cfg.B) for h in range(cfg.Hq)]
    rp = pool.time_prefill(q, k, v, cfg.scale, cfg.causal, heads)
    flops = ai.prefill_flops(cfg)
    dcfg = ai.CONFIGS[DECODE_CFG]
    dq, kp, vp, table, lens = decode_host
    units = [(b, h) for b in range(dcfg.B) for h in range(dcfg.Hkv)]
    rd = pool.time_decode(dq, kp, vp, table, lens, dcfg.scale, units)
    dbytes = ai.decode_bytes(dcfg, lens)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    return {"value": round(flops / rp["seconds"] / 1e12, 4), "unit": "TFLOP/s",
            "cores": cores, "workers": rp["workers"], "kind": "oracle",
            "cpu_model": pool.cpu_model(),
            "sample": f"the whole {PREFILL_CFG} workload ({len(heads)} heads, {rp['units']} "
                      f"units of up to 1,024 query rows), {rp['seconds']:.2f} s wall on "
                      f"{rp['workers']} worker processes of numpy fp64 three-pass attention "
                      "(full rows even where causal masks them); FLOPs counted as for the GPU "
                      "(4*d per visible pair)",
            "decode": {"value": round(dbytes / rd["seconds"] / 1e9, 3), "unit": "GB/s",
                       "workers": rd["workers"],
                       "sample": f"the whole {DECODE_CFG} workload ({rd['units']} (sequence, "
                                 f"KV head) units, sum(len)={int(lens.sum())}), "
                                 f"{rd['seconds']:.2f} s wall; bytes counted as for the GPU "
                                 "(bf16 K and V of the live tokens plus q, o, lse, lengths and "
                                 "block-table entries)"}}


# ------------------------------------------------------------------------------ main
def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the attention kernels "
              "here have no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    if not args.no_cpu:
        # the oracle pool's workers fork from a server started before the GPU is touched
        from oracle import pool
        pool.start()
    import torch
    import io_aware_exact_attention_amd as mi

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    pcfg, (q, k, v, o, lse), prefill_host = prefill_setup(PREFILL_CFG, keep_host=True)
    dcfg, lens, maxlen, (dq, dkc, dvc, table, seq, do, dlse), decode_host = decode_setup(
        DECODE_CFG, keep_host=True)
    if args.no_cpu:
        prefill_host = decode_host = None
    ws = mi.decode_workspace(dcfg.B, dcfg.Hq, dcfg.d, maxlen, 0)

    def prefill_call():
        mi.attn_fwd_prefill(q, k, v, o, lse, pcfg.causal, pcfg.scale, stream)

    def decode_call():
        mi.attn_fwd_decode(dq, dkc, dvc, table, seq, do, dlse, maxlen, dcfg.scale, 0, ws,
                           stream=stream)

    global SETTLE_MS
    SETTLE_MS = args.settle_ms

    def step_call():
        prefill_call()
        decode_call()

    # warmup (W steps, then untimed steps until the warmup has lasted settle_ms), then K
    # timed steps (prefill + decode), each launch bracketed by events
    t_warm = time.perf_counter()
    for _ in range(args.warmup):
        step_call()
    settle_steps = settle(step_call, t_warm, args.settle_ms)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps + 1)]
    t_wall0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        prefill_call()
        ev[2 * i + 1].record(stream)
        decode_call()
        ev[2 * i + 2].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    p_us = [ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e3 for i in range(args.steps)]
    d_us = [ev[2 * i + 1].elapsed_time(ev[2 * i + 2]) * 1e3 for i in range(args.steps)]
    p_avg, d_avg = float(np.mean(p_us)), float(np.mean(d_us))

    p_flops = ai.prefill_flops(pcfg)
    p_tflops = p_flops / (p_avg * 1e-6) / 1e12
    d_bytes = ai.decode_bytes(dcfg, lens)
    d_gbs = d_bytes / (d_avg * 1e-6) / 1e9
    props = torch.cuda.get_device_properties(0)
    clk_mhz = device_clock_mhz()

    out = {
        "metric": METRIC,
        "value": round(p_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"ms": args.settle_ms, "extra_untimed_steps": settle_steps},
        "ms_per_step": round(t_wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded i.i.d. N(0,1) draws rounded to bf16",
        "config": {
            "workload": "prefill llama2_7b_prefill (causal, B=4, H=32, N=2048, d=128) + decode "
                        "paged_gqa_decode (B=8, Hq=32, Hkv=8, d=128, page 16, "
                        f"sum(len)={int(lens.sum())}, max len={maxlen})",
            "prefill": {"B": pcfg.B, "Hq": pcfg.Hq, "Hkv": pcfg.Hkv, "Nq": pcfg.Nq,
                        "Nk": pcfg.Nk, "d": pcfg.d, "causal": pcfg.causal},
            "decode": {"B": dcfg.B, "Hq": dcfg.Hq, "Hkv": dcfg.Hkv, "d": dcfg.d,
                       "page_size": dcfg.page_size, "lengths": lens.tolist(),
                       "num_splits": mi.attn_decode_num_splits(dcfg.B, dcfg.Hq, dcfg.Hkv,
                                                               dcfg.d, maxlen, 0)},
        },
        "roofline": {"bound": "mfma", "achieved": round(p_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(p_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic("prefill_kernel<128,causal>"),
                     "kernel": "prefill_kernel<128, causal>",
                     "us_per_launch": round(p_avg, 2),
                     "us_median": round(float(np.median(p_us)), 2),
                     "us_min": round(float(np.min(p_us)), 2), "flops_per_launch": p_flops},
        "decode": {
            "value": round(d_gbs, 1), "unit": "GB/s", "us_per_step": round(d_avg, 2),
            "us_median": round(float(np.median(d_us)), 2), "us_min": round(float(np.min(d_us)), 2),
            "roofline": {"bound": "hbm", "achieved": round(d_gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(d_gbs / PEAK_HBM_GBS, 4),
                         "traffic": decode_traffic(),
                         "kernel": "decode_split_kernel<128, paged> + decode_merge_kernel<128>",
                         "bytes_per_launch": d_bytes},
        },
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "max_clock_mhz": clk_mhz,
                   # dense bf16 MFMA peak recomputed from this device: CUs x 4096 FLOP/clk x
                   # its peak clock (the roofline above uses the published figure)
                   "peak_bf16_tflops_from_clock": (
                       round(props.multi_processor_count * 4096 * clk_mhz * 1e6 / 1e12, 1)
                       if clk_mhz else None),
                   "kernel_sources": kernel_sources_digest()},
    }

    if not args.no_extra:
        extra = {}
        del q, k, v, o, lse
        for name in ("llama2_7b_prefill_noncausal", "long_prefill_32k", "llama2_7b_prefill_f16",
                     "llama2_7b_prefill_fp8"):
            cfg, (eq, ek, ev_, eo, el) = prefill_setup(name)
            if cfg.fp8:
                qs, ks, vs = ai.prefill_scales(cfg)
                call = lambda: mi.attn_fwd_prefill_fp8(eq, ek, ev_, eo, el, cfg.causal,
                                                       cfg.scale, qs, ks, vs, stream)
            else:
                fwd = mi.attn_fwd_prefill_f16 if cfg.f16 else mi.attn_fwd_prefill
                call = lambda: fwd(eq, ek, ev_, eo, el, cfg.causal, cfg.scale, stream)
            # (the 32K prefill: 10 timed launches, 7 ms each)
            avg, med, mn = time_kernel(
                call, 10 if name == "long_prefill_32k" else args.steps, args.warmup)
            tf = ai.prefill_flops(cfg) / (avg * 1e-6) / 1e12
            extra[name] = {"us": round(avg, 2), "us_min": round(mn, 2), "TFLOP/s": round(tf, 2),
                           "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
            if cfg.fp8:
                # same shape and FLOPs as the bf16 causal prefill timed above
                extra[name]["speedup_vs_bf16"] = round(p_avg / avg, 3)
                # half the FLOPs (Q.K^T) on the FP8 MFMA, half (P.V) on the bf16 one
                mixed = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
                extra[name]["peak_mixed_tflops"] = round(mixed, 1)
                extra[name]["frac_mixed"] = round(tf / mixed, 4)
            del eq, ek, ev_, eo, el
            torch.cuda.empty_cache()
        del dq, dkc, dvc, table, seq, do, dlse, ws
        torch.cuda.empty_cache()
        cfg, clens, cmax, (cq, ckc, cvc, ctab, cseq, co, cl) = decode_setup("gqa_decode_contig")
        cws = mi.decode_workspace(cfg.B, cfg.Hq, cfg.d, cmax, 0)
        avg, med, mn = time_kernel(
            lambda: mi.attn_fwd_decode(cq, ckc, cvc, None, cseq, co, cl, cmax, cfg.scale, 0, cws,
                                       stream=stream), args.steps, args.warmup)
        gbs = ai.decode_bytes(cfg, clens) / (avg * 1e-6) / 1e9
        extra["gqa_decode_contig"] = {"us": round(avg, 2), "us_min": round(mn, 2),
                                      "GB/s": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)}
        del cq, ckc, cvc, cseq, co, cl, cws
        torch.cuda.empty_cache()
        # the paged decode workload over an FP8 E4M3 cache (same lengths and pages)
        cfg, flens, fmax, (fq, fkc, fvc, ftab, fseq, fo, fl) = decode_setup("paged_gqa_decode_fp8")
        fws = mi.decode_workspace(cfg.B, cfg.Hq, cfg.d, fmax, 0)
        avg, med, mn = time_kernel(
            lambda: mi.attn_fwd_decode_fp8(fq, fkc, fvc, ftab, fseq, fo, fl, fmax, cfg.scale,
                                           ai.FP8_K_SCALE, ai.FP8_V_SCALE, 0, fws,
                                           stream=stream), args.steps, args.warmup)
        gbs = ai.decode_bytes(cfg, flens) / (avg * 1e-6) / 1e9
        extra["paged_gqa_decode_fp8"] = {"us": round(avg, 2), "us_min": round(mn, 2),
                                         "GB/s": round(gbs, 1),
                                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                                         "speedup_vs_bf16_cache": round(d_avg / avg, 3)}
        del fq, fkc, fvc, ftab, fseq, fo, fl, fws
        torch.cuda.empty_cache()
        # ragged batch of 16 prompts (256..4096 tokens) packed along tokens, causal
        cfg = ai.CONFIGS["varlen_prefill"]
        vl = ai.varlen_lengths(cfg.seed, cfg.B, *cfg.len_range)
        vq, vk, vv, vcq, vck = ai.varlen_inputs(cfg.seed, vl, vl, cfg.Hq, cfg.Hkv, cfg.d)
        vq, vk, vv = to_dev(vq).reshape(vq.shape), to_dev(vk).reshape(vk.shape), \
            to_dev(vv).reshape(vv.shape)
        vcq, vck = torch.from_numpy(vcq).cuda(), torch.from_numpy(vck).cuda()
        vo = torch.empty_like(vq)
        vlse = torch.empty((cfg.Hq, vq.shape[0]), dtype=torch.float32, device="cuda")
        mx = int(vl.max())
        avg, med, mn = time_kernel(
            lambda: mi.attn_fwd_prefill_varlen(vq, vk, vv, vo, vlse, vcq, vck, mx, mx, True,
                                               cfg.scale, stream), args.steps, args.warmup)
        fl = ai.varlen_flops(vl, vl, cfg.Hq, cfg.d, True)
        tf = fl / (avg * 1e-6) / 1e12
        extra["varlen_prefill"] = {"us": round(avg, 2), "us_min": round(mn, 2),
                                   "TFLOP/s": round(tf, 2), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                                   "lengths": [int(x) for x in vl]}
        bf16_varlen_us = avg
        del vq, vk, vv, vo
        torch.cuda.empty_cache()
        # the same ragged batch over FP8 inputs
        vq, vk, vv, _, _ = ai.varlen_inputs(cfg.seed, vl, vl, cfg.Hq, cfg.Hkv, cfg.d, fp8=True)
        vq, vk, vv = (torch.from_numpy(x).cuda() for x in (vq, vk, vv))
        vo = torch.empty(vq.shape, dtype=torch.bfloat16, device="cuda")
        avg, med, mn = time_kernel(
            lambda: mi.attn_fwd_prefill_varlen_fp8(vq, vk, vv, vo, vlse, vcq, vck, mx, mx, True,
                                                   cfg.scale, ai.FP8_Q_SCALE, ai.FP8_K_SCALE,
                                                   ai.FP8_V_SCALE, stream), args.steps, args.warmup)
        tf = fl / (avg * 1e-6) / 1e12
        extra["varlen_prefill_fp8"] = {"us": round(avg, 2), "us_min": round(mn, 2),
                                       "TFLOP/s": round(tf, 2),
                                       "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                                       "speedup_vs_bf16": round(bf16_varlen_us / avg, 3)}
        del vq, vk, vv, vcq, vck, vo, vlse
        torch.cuda.empty_cache()
        # backward of the causal Llama-2-shaped prefill (dQ, dK, dV from the stored LSE)
        cfg, (bq, bk, bv, bo, bl) = prefill_setup("llama2_7b_prefill")
        bdo = to_dev(ai.prefill_dout(cfg))
        mi.attn_fwd_prefill(bq, bk, bv, bo, bl, cfg.causal, cfg.scale, stream)
        gq, gk, gv = torch.empty_like(bq), torch.empty_like(bk), torch.empty_like(bv)
        bws = torch.empty(mi.attn_bwd_workspace_bytes(cfg.B, cfg.Hq, cfg.Nq), dtype=torch.uint8,
                          device="cuda")
        avg, med, mn = time_kernel(
            lambda: mi.attn_bwd(bq, bk, bv, bo, bl, bdo, gq, gk, gv, cfg.causal, cfg.scale, bws,
                                stream), args.steps, args.warmup)
        tf = ai.backward_flops(cfg) / (avg * 1e-6) / 1e12
        extra["llama2_7b_backward"] = {"us": round(avg, 2), "us_min": round(mn, 2),
                                       "TFLOP/s": round(tf, 2),
                                       "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                                       "flops": ai.backward_flops(cfg)}
        del bq, bk, bv, bo, bl, bdo, gq, gk, gv, bws
        torch.cuda.empty_cache()
        # chunked prefill against a paged cache (512 new tokens per sequence)
        cfg = ai.CONFIGS["chunked_prefill_paged"]
        plens = ai.decode_lengths(cfg)
        lay = ai.paged_layout(plens, cfg.page_size, cfg.seed)
        pq = to_dev(ai.chunk_q(cfg))
        pkc = to_dev(ai.build_paged_cache(cfg, ai.T_K, plens, lay, pad_bits=np.uint16(0)))
        pvc = to_dev(ai.build_paged_cache(cfg, ai.T_V, plens, lay, pad_bits=np.uint16(0)))
        ptab = torch.from_numpy(lay.block_table).cuda()
        plen_d = torch.from_numpy(plens).cuda()
        po = torch.empty_like(pq)
        pl = torch.empty(pq.shape[:3], dtype=torch.float32, device="cuda")
        pmax = int(plens.max())
        avg, med, mn = time_kernel(
            lambda: mi.attn_fwd_prefill_paged(pq, pkc, pvc, ptab, plen_d, po, pl, pmax, True,
                                              cfg.scale, stream=stream), args.steps, args.warmup)
        tf = ai.chunk_prefill_flops(cfg, plens) / (avg * 1e-6) / 1e12
        extra["chunked_prefill_paged"] = {"us": round(avg, 2), "us_min": round(mn, 2),
                                          "TFLOP/s": round(tf, 2),
                                          "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                                          "chunk": cfg.chunk, "kv_lens": [int(x) for x in plens]}
        bf16_chunk_us = avg
        del pq, pkc, pvc, po, pl
        torch.cuda.empty_cache()
        # the same chunked prefill over FP8 queries and an FP8 paged cache
        cfg = ai.CONFIGS["chunked_prefill_paged_fp8"]
        u8 = lambda c: torch.from_numpy(np.ascontiguousarray(c)).cuda()
        pq = u8(ai.chunk_q(cfg))
        pkc = u8(ai.build_paged_cache(cfg, ai.T_K, plens, lay, pad_bits=np.uint8(0)))
        pvc = u8(ai.build_paged_cache(cfg, ai.T_V, plens, lay, pad_bits=np.uint8(0)))
        po = torch.empty(pq.shape, dtype=torch.bfloat16, device="cuda")
        pl = torch.empty(pq.shape[:3], dtype=torch.float32, device="cuda")
        avg, med, mn = time_kernel(
            lambda: mi.attn_fwd_prefill_paged_fp8(pq, pkc, pvc, ptab, plen_d, po, pl, pmax, True,
                                                  cfg.scale, ai.FP8_Q_SCALE, ai.FP8_K_SCALE,
                                                  ai.FP8_V_SCALE, stream=stream),
            args.steps, args.warmup)
        tf = ai.chunk_prefill_flops(cfg, plens) / (avg * 1e-6) / 1e12
        extra["chunked_prefill_paged_fp8"] = {"us": round(avg, 2), "us_min": round(mn, 2),
                                              "TFLOP/s": round(tf, 2),
                                              "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                                              "speedup_vs_bf16": round(bf16_chunk_us / avg, 3)}
        out["other_workloads"] = extra

    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib * 2**20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(prefill_host, decode_host)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
