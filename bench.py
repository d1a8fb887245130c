#!/usr/bin/env python3
"""Benchmark of the KDA forward hot path on one MI355X.

One step = one chunkwise prefill (``kda_chunk_fwd``) of the long-context
workload (B=1, H=32, T=131072, d_k=d_v=128, C=64, bf16 storage) with every
input already resident in HBM.  The same run also times the small prefill
workload (B=2, H=8, T=2048, report only), the batched decode step
(``kda_decode_step``: 128 sessions x 32 heads, 268 MB fp32 state updated in
place, a fresh seeded token set every step), the same prefill through the
scalar-gate entry point, the packed
varlen workload (8 sequences through cu_seqlens), the backward (fp32
storage, d = 128), and the fp64 CPU oracle on a bounded sample of the prefill
workload.

Prints ONE JSON line.  ``value`` is prefill tokens/s; the ``decode`` object
carries the decode state bandwidth.  Roofline fractions use the algorithmic
bytes of the operator (inputs read once, outputs written once) over measured
time, against MI355X's 8 TB/s HBM.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s + decode state GB/s (KDA, H=32, d=128) and % of roofline"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0


def prefill_alg_bytes(T_total, H, dk, dv, n_seqs, has_s0=True):
    """q, k, v (bf16), g (fp32), beta (fp32) read once, o (bf16) written once,
    plus the fp32 initial state read and final state written once."""
    per_th = 2 * dk + 2 * dk + 2 * dv + 4 * dk + 4 + 2 * dv
    state = n_seqs * H * dk * dv * 4
    return T_total * H * per_th + state * (2 if has_s0 else 1)


def prefill_f32_alg_bytes(T_total, H, dk, dv, n_seqs, has_s0=True):
    """As prefill_alg_bytes with q, k, v and o stored in fp32."""
    per_th = 4 * dk + 4 * dk + 4 * dv + 4 * dk + 4 + 4 * dv
    state = n_seqs * H * dk * dv * 4
    return T_total * H * per_th + state * (2 if has_s0 else 1)


def scalar_gate_alg_bytes(T_total, H, dk, dv, n_seqs, has_s0=True):
    """As prefill_alg_bytes with one fp32 log-decay per (token, head)."""
    per_th = 2 * dk + 2 * dk + 2 * dv + 4 + 4 + 2 * dv
    state = n_seqs * H * dk * dv * 4
    return T_total * H * per_th + state * (2 if has_s0 else 1)


def prefill_alg_flops(T_total, H, C, d):
    """Dense chunk contractions per token-head: A, H, W, U, H Z (C^2 d terms)
    and W S, Qbar S, Ktil^T Z (C d^2 terms): 2 (5 C d + 3 d^2)."""
    return T_total * H * 2 * (5 * C * d + 3 * d * d)


def decode_alg_bytes(N, H, dk, dv):
    """Per (session, head): state read + write (fp32), q, k, v, o (bf16), g
    (fp32), beta (fp32)."""
    return N * H * (2 * dk * dv * 4 + 2 * dk + 2 * dk + 2 * dv + 4 * dk + 4 + 2 * dv)


def _counter_record(key):
    """The committed rocprofv3 counter record for one workload, or None when it
    is missing or the kernel sources have changed since it was taken."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
            rec = json.load(f)[key]
        h = hashlib.sha256()
        for name in rec["sources"]:
            with open(os.path.join(ROOT, "gated_delta_rule_80_amd", "csrc", name), "rb") as f:
                h.update(f.read())
    except (OSError, KeyError, ValueError):
        return None
    return rec if h.hexdigest() == rec["sources_sha256"] else None


def measured_traffic(key):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    runs (scaled by a plain copy of known size), or None when the kernel
    sources have changed since those counters were taken."""
    rec = _counter_record(key)
    return rec["hbm_bytes_per_launch"] if rec else None


def measured_mfma(key):
    """Per kernel: the fraction of SIMD cycles with the matrix unit busy
    (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE per XCD x 1024 SIMDs) and the
    MFMA FLOPs issued (SQ_INSTS_VALU_MFMA_MOPS_* x 512), from the committed
    counter run; None when the sources have changed since."""
    rec = _counter_record(key)
    if not rec or "mfma_counters" not in rec:
        return None
    return {k: {"busy_frac": v["mfma_busy_frac"],
                "flop": v["mfma_flop_f16"] + v["mfma_flop_bf16"] + v["mfma_flop_f32"]}
            for k, v in rec["mfma_counters"].items()}


def cpu_model():
    """The host CPU as /proc/cpuinfo names it, with its family / model /
    stepping numbers (some hosts report only a generic model name) and the
    logical CPU count."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" not in line:
                    if fields:
                        break           # the first processor's block is enough
                    continue
                key, val = (x.strip() for x in line.split(":", 1))
                fields.setdefault(key, val)
    except OSError:
        pass
    name = fields.get("model name") or platform.processor() or "unknown"
    ids = ", ".join("%s %s" % (k, fields[k]) for k in ("vendor_id", "cpu family", "model",
                                                        "stepping") if k in fields)
    return "%s (%s; %d logical CPUs)" % (name, ids or "no cpuinfo ids", os.cpu_count() or 0)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=32768)
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--skip-small-prefill", action="store_true")
    ap.add_argument("--skip-fp32-prefill", action="store_true")
    ap.add_argument("--skip-scalar-gate", action="store_true")
    ap.add_argument("--skip-varlen", action="store_true")
    ap.add_argument("--skip-backward", action="store_true")
    ap.add_argument("--skip-layer-forms", action="store_true")
    ap.add_argument("--prefill-order", choices=("overlapped", "serial"), default="overlapped",
                    help="order of the bf16 prefill's two kernels (kda_set_prefill_overlap): "
                         "side by side where the library applies it (default), or one after "
                         "the other; hardware counter runs need the serial order, since "
                         "counter collection runs the dispatches one at a time")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="finally run a plain device copy kernel over this many MiB three times: "
                         "the known-size reference for hardware byte counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: the whole KDA path runs on a single MI355X "
              "(no sharding or collectives); --gpus %d is not supported" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_80_amd as K
    import kda_workloads as W

    K.lib()  # fail loudly if the HIP library is missing
    K.set_prefill_overlap(1 if args.prefill_order == "overlapped" else 0)
    dev = torch.device("cuda:0")
    w5 = W.WORKLOADS[5]
    print("[bench] generating %s" % w5.description, file=sys.stderr, flush=True)
    inp = W.make_workload(5)
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    B, T, H, dk = d["q"].shape
    dv = d["v"].shape[-1]
    N = inp["n_seqs"]
    ws = torch.empty(K.workspace_bytes(B, T, H, dk, dv, w5.chunk, N), dtype=torch.uint8,
                     device=dev)
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    fs = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)

    def step():
        K.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=d["scale"],
                    initial_state=d["initial_state"], chunk_size=w5.chunk, workspace=ws, out=o,
                    final_state=fs)

    print("[bench] prefill warmup %d, timed %d" % (args.warmup, args.steps), file=sys.stderr,
          flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    ms_per_step = wall * 1e3 / args.steps
    avg_launch_ms = sum(launch_ms) / len(launch_ms)
    T_total = B * T
    tokens_per_s = T_total / (ms_per_step * 1e-3)
    alg_bytes = prefill_alg_bytes(T_total, H, dk, dv, N)
    alg_flops = prefill_alg_flops(T_total, H, w5.chunk, dk)
    achieved = alg_bytes / (avg_launch_ms * 1e-3) / 1e9
    ok = bool(torch.isfinite(o.float()).all().item()) and bool(torch.isfinite(fs).all().item())

    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "precision": "bf16 storage; fp16 MFMA operands with fp32 accumulation; fp32 state",
        "data": "synthetic",
        "config": {"workload": "long-context prefill B=1 H=32 T=131072 d_k=d_v=128 C=64 bf16, "
                               "z~U(4,12), S0~N(0,0.01^2)",
                   "global_batch": B, "seq_len": T, "heads": H, "d_k": dk, "d_v": dv,
                   "chunk": w5.chunk, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm",
                     "kernel": ("kda_chunk_fwd = kda_intra_kernel beside kda_inter_kernel<2>, "
                                "records handed over through L2 (overlapped order)"
                                if args.prefill_order == "overlapped" else
                                "kda_chunk_fwd = kda_intra_kernel then kda_inter_kernel<1> "
                                "(serial order)"),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("kda_chunk_fwd:T131072_H32"),
                     "traffic_order": "serial: the counters are collected with one dispatch at "
                                      "a time, so they measure the two kernels one after the "
                                      "other; side by side the chain reads the records from L2 "
                                      "and moves at most these bytes",
                     "alg_bytes_per_launch": alg_bytes,
                     "avg_launch_ms": round(avg_launch_ms, 4),
                     "mfma_frac_alg": round(alg_flops / (avg_launch_ms * 1e-3) / 1e12
                                            / BF16_MFMA_PEAK_TFLOPS, 4),
                     "mfma_counters": measured_mfma("kda_chunk_fwd:T131072_H32")},
        "outputs_finite": ok,
    }

    if not args.skip_small_prefill:
        # Workload 2, report only: B=2 rows of 2048 tokens, H=8.  Sixteen chains
        # of 32 chunks cannot fill the chip; this leg shows the latency floor.
        w2 = W.WORKLOADS[2]
        print("[bench] small prefill: %s" % w2.description, file=sys.stderr, flush=True)
        inp2 = W.make_workload(2)
        d2 = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp2.items()}
        B2, T2, H2, dk2 = d2["q"].shape
        ws2 = torch.empty(K.workspace_bytes(B2, T2, H2, dk2, dv, w2.chunk, B2), dtype=torch.uint8,
                          device=dev)
        o2 = torch.empty((B2, T2, H2, dv), dtype=torch.bfloat16, device=dev)
        fs2 = torch.empty((B2, H2, dk2, dv), dtype=torch.float32, device=dev)

        def pstep():
            K.chunk_fwd(d2["q"], d2["k"], d2["v"], d2["g"], d2["beta"], scale=d2["scale"],
                        initial_state=d2["initial_state"], chunk_size=w2.chunk, workspace=ws2,
                        out=o2, final_state=fs2)

        for _ in range(5):
            pstep()
        torch.cuda.synchronize()
        n_p = 50
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n_p):
            pstep()
        e1.record(stream)
        torch.cuda.synchronize()
        pms = e0.elapsed_time(e1) / n_p
        ptok = B2 * T2
        pbytes = prefill_alg_bytes(ptok, H2, dk2, dv, B2)
        pgbs = pbytes / (pms * 1e-3) / 1e9
        result["small_prefill"] = {
            "value": round(ptok / (pms * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(pms, 4), "steps": n_p,
            "config": {"workload": "prefill B=2 H=8 T=2048 d_k=d_v=128 C=64 bf16, "
                                   "S0~N(0,0.01^2) (report only)"},
            "roofline": {"bound": "hbm", "kernel": "kda_chunk_fwd", "achieved": round(pgbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(pgbs / HBM_PEAK_GBS, 4), "alg_bytes_per_launch": pbytes,
                         "traffic": measured_traffic("kda_chunk_fwd:B2_T2048_H8")}}
        del d2, inp2, ws2, o2, fs2

    if not args.skip_fp32_prefill:
        # Workload 2's shape with fp32 storage, report only: the fp32 path at
        # d = 128 (chunk factors and state chain on fp32 MFMA).
        print("[bench] fp32 prefill: B=2 H=8 T=2048 d=128, fp32 storage", file=sys.stderr,
              flush=True)
        inpf = W.make_prefill(H=8, dk=128, dv=128, dtype="f32", z_range=(2.0, 9.0), seed=1002,
                              B=2, T=2048, s0_std=0.01)
        df = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inpf.items()}
        Bf, Tf, Hf, dkf = df["q"].shape
        wsf = torch.empty(K.workspace_bytes(Bf, Tf, Hf, dkf, dkf, 64, Bf, torch.float32),
                          dtype=torch.uint8, device=dev)
        of = torch.empty((Bf, Tf, Hf, dkf), dtype=torch.float32, device=dev)
        fsf = torch.empty((Bf, Hf, dkf, dkf), dtype=torch.float32, device=dev)

        def fstep():
            K.chunk_fwd(df["q"], df["k"], df["v"], df["g"], df["beta"], scale=df["scale"],
                        initial_state=df["initial_state"], chunk_size=64, workspace=wsf,
                        out=of, final_state=fsf)

        for _ in range(3):
            fstep()
        torch.cuda.synchronize()
        n_f = 20
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n_f):
            fstep()
        e1.record(stream)
        torch.cuda.synchronize()
        fms = e0.elapsed_time(e1) / n_f
        fbytes = prefill_f32_alg_bytes(Bf * Tf, Hf, dkf, dkf, Bf)
        fgbs = fbytes / (fms * 1e-3) / 1e9
        result["fp32_prefill"] = {
            "value": round(Bf * Tf / (fms * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(fms, 4), "steps": n_f,
            "config": {"workload": "prefill B=2 H=8 T=2048 d_k=d_v=128 C=64 fp32 storage, "
                                   "S0~N(0,0.01^2) (report only)"},
            "roofline": {"bound": "hbm", "kernel": "kda_bwd_prep_kernel (chunk factors) and "
                         "kda_fwd_f32_chain_kernel, fp32 MFMA", "achieved": round(fgbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(fgbs / HBM_PEAK_GBS, 4), "alg_bytes_per_launch": fbytes,
                         "traffic": measured_traffic("kda_chunk_fwd:f32_B2_T2048_H8")}}
        del df, inpf, wsf, of, fsf

    if not args.skip_decode:
        w3 = W.WORKLOADS[3]
        print("[bench] decode: %s" % w3.description, file=sys.stderr, flush=True)
        state = W.make_decode_state(w3).to(dev)
        # Fresh seeded tokens for every one of the workload's steps, drawn on the
        # host and held on the device (about 5 MB per step) before the timing.
        n_tok = max(1, min(w3.steps, args.decode_steps))
        toks = [{k: (v.to(dev) if isinstance(v, torch.Tensor) else v)
                 for k, v in W.make_decode_step(s, w3).items()} for s in range(n_tok)]
        od = torch.empty((w3.n_sessions, w3.H, w3.dv), dtype=torch.bfloat16, device=dev)

        def dstep(i):
            t = toks[i % n_tok]
            K.decode_step(t["q"], t["k"], t["v"], t["g"], t["beta"], state, scale=w3.scale,
                          out=od)

        for i in range(8):
            dstep(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.decode_steps):
            dstep(i)
        e1.record(stream)
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / args.decode_steps
        dbytes = decode_alg_bytes(w3.n_sessions, w3.H, w3.dk, w3.dv)
        dgbs = dbytes / (dms * 1e-3) / 1e9
        result["decode"] = {
            "value": round(dgbs, 1), "unit": "GB/s", "ms_per_step": round(dms, 5),
            "steps": args.decode_steps,
            "config": {"workload": "batched decode 128 sessions x 32 heads d=128, fp32 state "
                                   "268 MB in place, bf16 tokens, a fresh seeded token set for "
                                   "each of the %d steps (cycled beyond that)" % n_tok},
            "roofline": {"bound": "hbm", "kernel": "kda_decode_kernel<128,128,bf16>",
                         "achieved": round(dgbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(dgbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("kda_decode_step:N128_H32"),
                         "alg_bytes_per_launch": dbytes},
        }
        del state, toks

    if not args.skip_scalar_gate:
        # The same long-context prefill through the scalar-gate entry point, gated
        # by the first channel's log-decay of every (token, head).
        gs = d["g"][..., 0].contiguous()
        print("[bench] scalar-gate prefill", file=sys.stderr, flush=True)

        def sstep():
            K.chunk_fwd_scalar_gate(d["q"], d["k"], d["v"], gs, d["beta"], scale=d["scale"],
                                    initial_state=d["initial_state"], chunk_size=w5.chunk,
                                    workspace=ws, out=o, final_state=fs)

        for _ in range(3):
            sstep()
        torch.cuda.synchronize()
        n_s = max(1, args.steps // 2)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n_s):
            sstep()
        e1.record(stream)
        torch.cuda.synchronize()
        sms = e0.elapsed_time(e1) / n_s
        sbytes = scalar_gate_alg_bytes(T_total, H, dk, dv, N)
        sgbs = sbytes / (sms * 1e-3) / 1e9
        result["scalar_gate"] = {
            "value": round(T_total / (sms * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(sms, 4), "steps": n_s,
            "config": {"workload": "long-context prefill B=1 H=32 T=131072 d=128 C=64 bf16 "
                                   "with one log-decay per (token, head)"},
            "roofline": {"bound": "hbm", "kernel": "kda_chunk_fwd_scalar_gate",
                         "achieved": round(sgbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(sgbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("kda_chunk_fwd_scalar_gate:T131072_H32"),
                         "alg_bytes_per_launch": sbytes}}
        del gs

    if not args.skip_layer_forms:
        # The same long-context prefill with the layer's input steps done in the
        # kernels (gate and beta as logits, q and k L2-normalised), then the
        # output stage (RMS norm x weight x sigmoid gate) on its output.
        print("[bench] prefill with every input form, then the output stage", file=sys.stderr,
              flush=True)
        gen = torch.Generator(device=dev).manual_seed(11)
        z = (4.0 + 8.0 * torch.rand(d["g"].shape, generator=gen, device=dev)).contiguous()
        bl = torch.randn(d["beta"].shape, generator=gen, device=dev).contiguous()
        ogate = torch.randn(o.shape, generator=gen, device=dev).to(torch.bfloat16).contiguous()
        wgt = (1.0 + 0.1 * torch.randn(dv, generator=gen, device=dev)).contiguous()
        out_stage = torch.empty_like(o)

        def fstep():
            K.chunk_fwd_ex(d["q"], d["k"], d["v"], z, bl, gate="per_channel", gate_is_logit=True,
                           beta_is_logit=True, l2norm_qk=True, scale=d["scale"],
                           initial_state=d["initial_state"], chunk_size=w5.chunk, workspace=ws,
                           out=o, final_state=fs)

        def ostep():
            K.output_rmsnorm_gate(o, ogate, wgt, eps=1e-6, out=out_stage)

        for _ in range(3):
            fstep()
            ostep()
        torch.cuda.synchronize()
        n_f = max(1, args.steps // 2)
        times = []
        for fn in (fstep, ostep):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n_f):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / n_f)
        fms, oms = times
        obytes = 3 * T_total * H * dv * 2 + dv * 4   # o and gate read, out written (bf16)
        ogbs = obytes / (oms * 1e-3) / 1e9
        fgbs = alg_bytes / (fms * 1e-3) / 1e9
        result["layer_forms"] = {
            "value": round(T_total / (fms * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(fms, 4), "steps": n_f,
            "config": {"workload": "long-context prefill as above through kda_chunk_fwd_ex with "
                                   "logit gate, logit beta and in-kernel q/k L2 norm; then "
                                   "kda_output_rmsnorm_gate on its output"},
            "roofline": {"bound": "hbm", "kernel": "kda_chunk_fwd_ex", "achieved": round(fgbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(fgbs / HBM_PEAK_GBS, 4), "alg_bytes_per_launch": alg_bytes,
                         "traffic": measured_traffic("kda_chunk_fwd_ex:T131072_H32_all_forms")},
            "output_stage": {"ms": round(oms, 4), "achieved": round(ogbs, 1), "unit": "GB/s",
                             "frac": round(ogbs / HBM_PEAK_GBS, 4),
                             "kernel": "kda_output_rmsnorm_gate_kernel",
                             "alg_bytes_per_launch": obytes,
                             "traffic": measured_traffic("kda_output_rmsnorm_gate:T131072_H32")}}
        del z, bl, ogate, wgt, out_stage

    if not args.skip_varlen:
        # The packed workload: 8 sequences of seeded lengths in one buffer with
        # cu_seqlens, zero initial states, one final state per sequence.
        w4 = W.WORKLOADS[4]
        print("[bench] varlen prefill: %s" % w4.description, file=sys.stderr, flush=True)
        inp4 = W.make_workload(4)
        d4 = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp4.items()}
        B4, T4, H4, dk4 = d4["q"].shape
        N4 = inp4["n_seqs"]
        ws4 = torch.empty(K.workspace_bytes(B4, T4, H4, dk4, dv, w4.chunk, N4), dtype=torch.uint8,
                          device=dev)
        o4 = torch.empty((B4, T4, H4, dv), dtype=torch.bfloat16, device=dev)
        fs4 = torch.empty((N4, H4, dk4, dv), dtype=torch.float32, device=dev)

        def vstep():
            K.chunk_fwd(d4["q"], d4["k"], d4["v"], d4["g"], d4["beta"], scale=d4["scale"],
                        initial_state=None, cu_seqlens=d4["cu_seqlens"], chunk_size=w4.chunk,
                        workspace=ws4, out=o4, final_state=fs4)

        for _ in range(3):
            vstep()
        torch.cuda.synchronize()
        n_v = max(1, args.steps // 2)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n_v):
            vstep()
        e1.record(stream)
        torch.cuda.synchronize()
        vms = e0.elapsed_time(e1) / n_v
        vtok = B4 * T4
        vbytes = prefill_alg_bytes(vtok, H4, dk4, dv, N4, has_s0=False)
        vgbs = vbytes / (vms * 1e-3) / 1e9
        lens = [int(x) for x in (inp4["cu_seqlens"][1:] - inp4["cu_seqlens"][:-1]).tolist()]
        result["varlen"] = {
            "value": round(vtok / (vms * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(vms, 4), "steps": n_v,
            "config": {"workload": "varlen packed prefill, 8 sequences of lengths %s (%d "
                                   "tokens), H=32 d=128 C=64 bf16, zero initial states"
                                   % (lens, vtok)},
            "roofline": {"bound": "hbm", "kernel": "kda_chunk_fwd (cu_seqlens)",
                         "achieved": round(vgbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(vgbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("kda_chunk_fwd:varlen8_H32"),
                         "alg_bytes_per_launch": vbytes}}
        del d4, inp4, ws4, o4, fs4

    if not args.skip_backward:
        # Gradients through kda_chunk_bwd at the layer's width (bf16 q, k, v and
        # d_o, fp32 gradients, d = 128, C = 16), one sequence of 8192 tokens
        # per head, 32 heads.
        print("[bench] backward (bf16 storage, d=128, C=16, B=1 H=32 T=8192)", file=sys.stderr,
              flush=True)
        gen = torch.Generator(device=dev).manual_seed(7)
        Tb, Hb, db, Cb = 8192, 32, 128, 16
        rnd = lambda *sh: torch.randn(*sh, generator=gen, device=dev)  # noqa: E731
        bf = torch.bfloat16
        qb = torch.nn.functional.normalize(rnd(1, Tb, Hb, db), dim=-1).to(bf).contiguous()
        kb = torch.nn.functional.normalize(rnd(1, Tb, Hb, db), dim=-1).to(bf).contiguous()
        vb, dob = rnd(1, Tb, Hb, db).to(bf), rnd(1, Tb, Hb, db).to(bf)
        gb = (-0.05 * torch.rand(1, Tb, Hb, db, generator=gen, device=dev)).contiguous()
        bb = torch.sigmoid(rnd(1, Tb, Hb)).contiguous()
        s0b, dfb = 0.1 * rnd(1, Hb, db, db), rnd(1, Hb, db, db)
        wsb = torch.empty(K.workspace_bytes_bwd(1, Tb, Hb, db, Cb, 1, bf), dtype=torch.uint8,
                          device=dev)

        def bstep():
            return K.chunk_bwd(qb, kb, vb, gb, bb, dob, initial_state=s0b, d_final_state=dfb,
                               chunk_size=Cb, workspace=wsb)

        for _ in range(2):
            bstep()
        torch.cuda.synchronize()
        n_b = max(1, args.steps // 4)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n_b):
            grads = bstep()
        e1.record(stream)
        torch.cuda.synchronize()
        bms = e0.elapsed_time(e1) / n_b
        # inputs q, k, v, d_o (bf16), g (fp32) and beta read once, gradients
        # (fp32) written once, states read (s0, d_final) and written (d_s0) once
        bbytes = Tb * Hb * (4 * 2 * db + 4 * db + 4) + Tb * Hb * (4 * 4 * db + 4) + \
            3 * Hb * db * db * 4
        bgbs = bbytes / (bms * 1e-3) / 1e9
        result["backward"] = {
            "value": round(Tb / (bms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(bms, 4),
            "steps": n_b,
            "config": {"workload": "gradients of the chunked prefill, B=1 H=32 T=8192 d=128 C=16, "
                                   "bf16 q/k/v/d_o, fp32 gradients, log-decays U(-0.05, 0), "
                                   "through kda_chunk_bwd"},
            "roofline": {"bound": "hbm", "kernel": "kda_bwd_prep_kernel, kda_bwd_chain_mfma_kernel "
                         "and kda_bwd_grad_kernel (fp32 MFMA for every contraction); the "
                         "states stored at every other chunk boundary dominate the traffic",
                         "achieved_hbm_gbs": round(bgbs, 2), "hbm_frac": round(bgbs / HBM_PEAK_GBS, 5),
                         "alg_bytes_per_launch": bbytes,
                         "traffic": measured_traffic("kda_chunk_bwd:T8192_H32_d128_C16")},
            "outputs_finite": bool(all(torch.isfinite(t).all().item() for t in grads.values()))}
        del qb, kb, vb, dob, gb, bb, s0b, dfb, wsb, grads

    if not args.no_cpu_baseline:
        import numpy as np
        import oracle
        S = min(args.cpu_sample_tokens, T)
        print("[bench] cpu oracle on the first %d tokens x %d heads" % (S, H), file=sys.stderr,
              flush=True)
        a = {n: W.to64(inp[n][:, :S]).reshape(S, H, -1) for n in ("q", "k", "v", "g")}
        bta = W.to64(inp["beta"][:, :S]).reshape(S, H)
        s0 = W.to64(inp["initial_state"])
        threads = len(os.sched_getaffinity(0))
        oracle.load_c_oracle()
        t0 = time.perf_counter()
        oracle.prefill(a["q"], a["k"], a["v"], a["g"], bta, inp["scale"], s0, [0, S],
                       col_block=32, n_threads=threads)
        cpu_s = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": round(S / cpu_s, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": "first %d tokens of the long-context prefill workload, all %d heads, "
                      "fp64 token recurrence, %.1f s" % (S, H, cpu_s),
            "cpu": cpu_model()}
        del np

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)  # reads n*4 bytes, writes n*4 bytes
        torch.cuda.synchronize()
        del src, dst

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
