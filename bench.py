#!/usr/bin/env python3
"""MXFP8 flash attention benchmark on one MI355X.

One step = the whole hot path on one batch of the B4 H32 L4096 d128 causal bf16 workload:
mx_quantize of Q, K and V (ROW + SEQ views), the forward (O, LSE) and the backward (G
views + D, the dK/dV kernel, the dQ kernel). Inputs are resident in HBM before the timed region.
The step is timed over 3 rounds of 20 (the value is the median round's rate); each line also
records the GPU clocks, ROCm and hipcc versions and the identity of the built sources.

FLOPs are causal-adjusted (FLAMIA notes section 6 visible-pair count): forward 4 d per
visible pair, backward 10 d (five GEMMs). `value` is the step's fwd+bwd FLOPs over the
step's wall time (quantisation included). The per-kernel lines come from HIP events that
the library records immediately around each launch of the named kernel, on its stream.

    python bench.py [--steps K] [--warmup W] [--rounds R] [--dq f32|f16] [--no-cpu-baseline] [--cpu-heads N]
    python bench.py --pmc-run      # one untimed step + a 1 GiB device copy, for counter runs
    python bench.py --workload c4  # 128 packed documents (log-normal lengths 32..2048), H4 d128 causal
    python bench.py --workload c5  # B1 H16 L16384 d128 non-causal (c5gqa: 16 query heads on 4 KV heads)
    python bench.py --workload x1  # cross-attention: 768 documents x 512 queries against
                                   # jagged keys/values (<= 14980), H3 d128, non-causal
    python bench.py --workload n1  # fused RMSNorm + quantise producer, x [262144, 512] bf16
    python bench.py --workload g1  # fused MXFP8 GEMM + quantise producer, 16384 x 12288 x 4096
    python bench.py --score mxfp4  # the mixed route: Q and K scored as MXFP4 (E2M1), everything else
                                   # MXFP8 (any attention workload; default c3)
    python bench.py --fwd strict   # the forward with the strict per-key V fold on the diagonal tiles
                                   # (causal workloads; V also quantised to its per-token view)
    python bench.py --bwd strict   # the backward with the strict dQ (per-query dS scales, K fold;
                                   # FP32 dQ; K also quantised to its per-token view)

`roofline.traffic` is the roofline kernel's HBM bytes per launch from rocprofv3 counters
(FETCH_SIZE and WRITE_SIZE, each scaled by its reading for the 1 GiB copy of --pmc-run),
stored in profiles/ with the hash of the kernel sources it was measured on; it is reported
only while those sources are unchanged, else null.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_attn_bwd_dkdv_c3.json")
# sources that determine the dK/dV kernel's code (hashed to validate recorded counters)
KERNEL_SOURCES = ["block_scaled_mxfp8_amd/csrc/attn_bwd.hip", "block_scaled_mxfp8_amd/csrc/mx_device.h",
                  "block_scaled_mxfp8_amd/csrc/mx_layout.h", "block_scaled_mxfp8_amd/csrc/mx_internal.h",
                  "block_scaled_mxfp8_amd/build.py"]


# the fused GEMM + quantise kernel (g1 workload)
GEMM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_gemm_quantize_g1.json")
GEMM_KERNEL_SOURCES = ["block_scaled_mxfp8_amd/csrc/gemm_quantize.hip", "block_scaled_mxfp8_amd/csrc/mx_device.h",
                       "block_scaled_mxfp8_amd/csrc/mx_layout.h", "block_scaled_mxfp8_amd/csrc/mx_gemm.h",
                       "block_scaled_mxfp8_amd/build.py"]

# the fused RMSNorm + quantise kernel (n1 workload)
NORM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_rmsnorm_quantize_n1.json")
NORM_KERNEL_SOURCES = ["block_scaled_mxfp8_amd/csrc/rmsnorm_quantize.hip", "block_scaled_mxfp8_amd/csrc/mx_device.h",
                       "block_scaled_mxfp8_amd/csrc/mx_layout.h", "block_scaled_mxfp8_amd/csrc/mx_norm.h",
                       "block_scaled_mxfp8_amd/build.py"]


def kernel_sources_sha256(sources=None):
    h = hashlib.sha256()
    for rel in (KERNEL_SOURCES if sources is None else sources):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def recorded_traffic(path=None, sources=None):
    """Bytes per launch of the recorded kernel (default: dK/dV) from its counter record, or
    None if absent or stale."""
    try:
        with open(TRAFFIC_FILE if path is None else path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != kernel_sources_sha256(sources):
        return None
    return int(rec["fetch_kib"] * rec["fetch_scale"] * 1024 + rec["write_kib"] * rec["write_scale"] * 1024)

# every source the library is built from (the identity recorded in each line)
ALL_SOURCES = sorted(os.path.relpath(p, ROOT) for p in
                     __import__("glob").glob(os.path.join(ROOT, "block_scaled_mxfp8_amd", "csrc", "*")))

PEAK_MXFP8_TFLOPS = 5000.0      # MI355X dense MXFP8 MFMA, AMD's published figure
PEAK_MXFP4_TFLOPS = 10100.0     # MI355X dense MXFP4 MFMA


def mixed_peak(fp4_share):
    """Peak of work whose FLOPs are fp4_share MXFP4 products and the rest MXFP8 ones (each at its
    own peak): the harmonic mix, FLOPs over the time the two parts need at their peaks."""
    return 1.0 / (fp4_share / PEAK_MXFP4_TFLOPS + (1.0 - fp4_share) / PEAK_MXFP8_TFLOPS)
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--dq", choices=["f32", "f16", "f16prefix"], default="f32",
                    help="dQ accumulation of the timed step (f16prefix: FP16 sums with the per-row prefix boost; "
                         "attention workloads without cross keys)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-steps", type=int, default=10, help="launches averaged per kernel line")
    ap.add_argument("--pmc-run", action="store_true", help="one untimed step + a 1 GiB copy (counter collection)")
    ap.add_argument("--recompute-dq", action="store_true",
                    help="minimal workspace: the dQ pass rebuilds dS instead of reading the stored codes")
    ap.add_argument("--rounds", type=int, default=3, help="timed rounds of --steps steps (value: the median)")
    ap.add_argument("--cpu-heads", type=int, default=24,
                    help="(batch, head) pairs the CPU baseline times (0: all of them, the full tensor)")
    ap.add_argument("--score", choices=["mxfp8", "mxfp4"], default="mxfp8",
                    help="score operands of the attention workloads: MXFP8 (E4M3), or MXFP4 (E2M1; the mixed route)")
    ap.add_argument("--fwd", choices=["plain", "strict"], default="plain",
                    help="forward of the step: plain, or with the strict per-key V fold (causal only)")
    ap.add_argument("--bwd", choices=["plain", "strict"], default="plain",
                    help="backward of the step: plain, or with the strict dQ (causal, FP32 dQ)")
    ap.add_argument("--workload", choices=["c3", "c4", "c5", "c5gqa", "x1", "n1", "g1"], default="c3",
                    help="c3: the headline causal self-attention step; c4: 128 packed documents; c5/c5gqa: "
                         "B1 H16 L16384 non-causal (MHA / 16 on 4 KV heads); x1: the jagged cross-attention "
                         "step; n1: the fused RMSNorm + quantise producer; g1: the fused GEMM + quantise producer")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: measures one GPU; multi-GPU runs are not supported (use --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    if args.workload == "x1":
        run_cross(args)
        return
    if args.workload == "n1":
        run_norm(args)
        return
    if args.workload == "g1":
        run_gemm(args)
        return
    run_attention(args)


def environment():
    """GPU clock, toolchain and source identity recorded in every line."""
    import subprocess
    info = {"source_sha256": kernel_sources_sha256(ALL_SOURCES)[:16]}
    try:
        with open(os.path.join(ROOT, "block_scaled_mxfp8_amd", "build_info.json")) as f:
            b = json.load(f)
        info["build_git"] = b.get("git")
        info["hipcc"] = b.get("hipcc")
        info["build_source_sha256"] = b.get("source_sha256", "")[:16]
    except (OSError, ValueError):
        info["build_git"] = None
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        info["rocm"] = None
    try:
        out = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        card = next(iter(json.loads(out.stdout).values()))
        info["gpu_clocks"] = {k: v for k, v in card.items() if any(c in k.lower() for c in ("sclk", "mclk", "fclk"))}
    except Exception:  # noqa: BLE001 - informational
        info["gpu_clocks"] = None
    return info


def run_attention(args):
    """c3 (headline), c5, c5gqa (batched) and c4 (packed documents): one step = mx_quantize of
    Q, K, V (ROW + SEQ views) + the forward + the backward, inputs resident in HBM. The step is
    timed over --rounds rounds of --steps steps each, with no measurement hook installed; the
    value is the median round. One more round of --steps steps records HIP events around every
    launch of the backward's dK/dV kernel (on the stream it is launched on) for the roofline."""
    import numpy as np
    import torch

    import synth
    from block_scaled_mxfp8_amd import (MX_DQ_F16_BOOST, MX_DQ_F16_PREFIX, MX_DQ_F32, MX_VIEW_ROW_FP4, MX_VIEW_SEQ,
                                        MX_VIEW_SEQ_TOKEN,
                                        PROFILE_BWD_DKDV, PROFILE_BWD_DQ, PROFILE_BWD_PREP, PROFILE_FWD,
                                        PROFILE_QUANTIZE, load, mx_attn_bwd, mx_attn_bwd_strict, mx_attn_fwd,
                                        mx_attn_fwd_strict,
                                        mx_profile_kernel, mx_quantize, mx_quantize_token_block)
    from block_scaled_mxfp8_amd.flops import attn_flops, visible_pairs

    load()
    name = args.workload
    cfg = synth.CONFIGS[name]
    d = cfg["head_dim"]
    causal = cfg["causal"]
    dq_mode = {"f32": MX_DQ_F32, "f16": MX_DQ_F16_BOOST, "f16prefix": MX_DQ_F16_PREFIX}[args.dq]
    print(f"[bench] generating {name} inputs", file=sys.stderr, flush=True)
    x = synth.make_inputs(name)
    packed = "cu_seqlens" in x
    if packed:
        cu_np = x.pop("cu_seqlens")
        lengths = np.diff(cu_np)
        cu = torch.from_numpy(cu_np.astype(np.int32)).cuda()
        maxlen = int(lengths.max())
        H = cfg["heads"]
        pairs = visible_pairs(1, H, causal=causal, lengths=lengths)
        kw = dict(cu_seqlens=cu, max_seqlen=maxlen)
        desc = (f"{name}: {len(lengths)} packed documents (log-normal lengths {int(lengths.min())}..{maxlen}, "
                f"T {int(cu_np[-1])}), H{H} d{d} causal per document")
        cfg_line = {"documents": int(len(lengths)), "tokens": int(cu_np[-1]), "max_seqlen": maxlen, "heads": H}
    else:
        B, H, L = cfg["batch"], cfg["heads"], cfg["seqlen"]
        pairs = visible_pairs(B, H, L, causal=causal)
        kw = {}
        desc = (f"{name}: B{B} H{H}" + (f" Hkv{cfg['heads_kv']}" if cfg["heads_kv"] != H else "") +
                f" L{L} d{d} {'causal' if causal else 'non-causal'}")
        cfg_line = {"batch": B, "heads": H, "heads_kv": cfg["heads_kv"], "seqlen": L}
    t = {n: torch.from_numpy(x[n]).to(torch.bfloat16).cuda() for n in ("q", "k", "v", "g")}
    del x
    f_fwd = attn_flops(pairs, d)
    f_bwd = attn_flops(pairs, d, backward=True)
    ws = {}
    ds_store = not args.recompute_dq

    fp4 = args.score == "mxfp4"
    strict = args.fwd == "strict"
    bstrict = args.bwd == "strict"
    if (strict or bstrict) and (fp4 or not causal):
        sys.exit("--fwd/--bwd strict need a causal workload with MXFP8 scores")
    if bstrict and args.dq != "f32":
        sys.exit("--bwd strict accumulates dQ in FP32")
    qk_views = (MX_VIEW_ROW_FP4 | MX_VIEW_SEQ) if fp4 else 3
    v_tok = [None]
    k_tok = [None]

    def quant():
        if strict:   # the per-token V view of the diagonal tiles: a second pass over V
            v_tok[0] = mx_quantize(t["v"], views=MX_VIEW_SEQ_TOKEN, **kw)[1]
        if bstrict:  # the per-token K view of the strict dQ: a second pass over K
            k_tok[0] = mx_quantize(t["k"], views=MX_VIEW_SEQ_TOKEN, **kw)[1]
        return (mx_quantize(t["q"], views=qk_views, **kw), mx_quantize(t["k"], views=qk_views, **kw),
                mx_quantize(t["v"], **kw))

    def fwd(q_row, k_row, v_seq):
        if strict:
            return mx_attn_fwd_strict(q_row, k_row, v_seq, v_tok[0], **kw)
        return mx_attn_fwd(q_row, k_row, v_seq, causal=causal, **kw)

    def step(mode=dq_mode):
        (q_row, q_seq), (k_row, k_seq), (v_row, v_seq) = quant()
        o, lse = fwd(q_row, k_row, v_seq)
        key = "strict" if bstrict else mode    # (the strict call's workspace is the minimal one)
        if bstrict:
            dq, dk, dv, w = mx_attn_bwd_strict(q_row, q_seq, k_row, k_seq, k_tok[0], v_row, o, lse, t["g"],
                                               workspace=ws.get(key), **kw)
        else:
            dq, dk, dv, w = mx_attn_bwd(q_row, q_seq, k_row, k_seq, v_row, o, lse, t["g"], causal=causal,
                                        dq_mode=mode, workspace=ws.get(key), ds_store=ds_store, **kw)
        ws[key] = w
        return o, dq

    if args.pmc_run:
        step()
        step()
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1.0)
        b.copy_(a)          # calibration: 1 GiB read + 1 GiB written
        torch.cuda.synchronize()
        print("[bench] pmc run done", file=sys.stderr, flush=True)
        return
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    rounds = []
    for r in range(max(1, args.rounds)):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        rounds.append((time.perf_counter() - t0) * 1e3 / args.steps)
        print(f"[bench] round {r}: {args.steps} steps, {rounds[-1]:.3f} ms/step", file=sys.stderr, flush=True)
    ms_step = float(np.median(rounds))
    # roofline round: events around every launch of the dK/dV kernel (the step's dominant kernel)
    ev_main = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in ev_main:
        a.record()
        b.record()
    mx_profile_kernel(PROFILE_BWD_DKDV, ev_main)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_hooked = (time.perf_counter() - t0) * 1e3 / args.steps
    mx_profile_kernel(0, [])
    ms_bwd_main = float(np.mean([a.elapsed_time(b) for a, b in ev_main]))
    print(f"[bench] roofline round: {ms_hooked:.3f} ms/step, dK/dV {ms_bwd_main:.3f} ms", file=sys.stderr, flush=True)

    # per-kernel averages outside the timed region
    def kernel_ms(kind, fn, n=args.profile_steps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in ev:
            a.record()
            b.record()
        mx_profile_kernel(kind, ev)
        torch.cuda.synchronize()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        mx_profile_kernel(0, [])
        return float(np.mean([a.elapsed_time(b) for a, b in ev]))

    (q_row, q_seq), (k_row, k_seq), (v_row, v_seq) = quant()
    o, lse = fwd(q_row, k_row, v_seq)
    ms_fwd = kernel_ms(PROFILE_FWD, lambda: fwd(q_row, k_row, v_seq))
    ms_fwd_plain = kernel_ms(PROFILE_FWD, lambda: mx_attn_fwd(q_row, k_row, v_seq, causal=causal, **kw)) if strict else None
    ms_quant = kernel_ms(PROFILE_QUANTIZE, lambda: mx_quantize(t["q"], **kw), n=3 * args.profile_steps)
    ms_quant_tb = None
    if not packed and not fp4:   # the token-block variant of the quantiser (same bytes; one exponent per 32 tokens x d)
        ms_quant_tb = kernel_ms(PROFILE_QUANTIZE, lambda: mx_quantize_token_block(t["q"]), n=3 * args.profile_steps)

    def bwd(mode):
        return lambda: mx_attn_bwd(q_row, q_seq, k_row, k_seq, v_row, o, lse, t["g"], causal=causal, dq_mode=mode,
                                   workspace=ws.get(mode), ds_store=ds_store, **kw)

    res_bwd = {}
    if bstrict:   # the strict backward's own call (its workspace is the minimal one)
        def sbwd():
            r = mx_attn_bwd_strict(q_row, q_seq, k_row, k_seq, k_tok[0], v_row, o, lse, t["g"],
                                   workspace=ws.get("strict"), **kw)
            ws["strict"] = r[3]
        sbwd()
        s_dq = kernel_ms(PROFILE_BWD_DQ, sbwd)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s0.record()
        for _ in range(args.profile_steps):
            sbwd()
        s1.record()
        torch.cuda.synchronize()
        res_bwd["strict"] = dict(dq_ms=s_dq, call_ms=s0.elapsed_time(s1) / args.profile_steps)
    modes = [("f32", MX_DQ_F32), ("f16", MX_DQ_F16_BOOST)]
    if args.dq == "f16prefix":
        modes.append(("f16prefix", MX_DQ_F16_PREFIX))
    for nm, mode in modes:
        if mode not in ws:
            _, _, _, ws[mode] = bwd(mode)()
        main_ms = kernel_ms(PROFILE_BWD_DKDV, bwd(mode))
        prep = kernel_ms(PROFILE_BWD_PREP, bwd(mode))
        fin = kernel_ms(PROFILE_BWD_DQ, bwd(mode))
        # whole call, events around it on the current stream
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s0.record()
        for _ in range(args.profile_steps):
            bwd(mode)()
        s1.record()
        torch.cuda.synchronize()
        call = s0.elapsed_time(s1) / args.profile_steps
        res_bwd[nm] = dict(dkdv_ms=main_ms, prep_ms=prep, dq_ms=fin, call_ms=call)

    q_elems = int(t["q"].numel())
    quant_bytes = q_elems * (2 + 2 * (1 + 1 / 32))          # bf16 in, two views of codes + scales out
    tflops = lambda f, ms: f / (ms * 1e-3) / 1e12          # noqa: E731
    # algorithmic FLOPs per kernel: dK/dV kernel S, E, dV, dK (4 of the 5 products, 8 d per
    # visible pair); dQ kernel dQ (2 d; the recomputing variant also rebuilds S and E, 4 d more,
    # not counted in the step's FLOPs, which follow the method's 10 d per pair)
    f_dkdv = f_bwd * 4 // 5
    bwd_f32, bwd_f16 = res_bwd["f32"], res_bwd["f16"]
    value = tflops(f_fwd + f_bwd, ms_step)
    # peaks: MXFP8 everywhere, or (MXFP4 scores) the mix of the FP4 score products' FLOP share
    # (forward 1 of 2 products, backward 1 of 5, dK/dV kernel 1 of 4, whole step 2 of 7) with MXFP8
    pk_step = mixed_peak(2 / 7) if fp4 else PEAK_MXFP8_TFLOPS
    pk_fwd = mixed_peak(1 / 2) if fp4 else PEAK_MXFP8_TFLOPS
    pk_bwd = mixed_peak(1 / 5) if fp4 else PEAK_MXFP8_TFLOPS
    pk_dkdv = mixed_peak(1 / 4) if fp4 else PEAK_MXFP8_TFLOPS
    if fp4:
        metric = f"mixed MXFP4-score / MXFP8 attn fwd/bwd TFLOP/s (causal-adj) on {name}" + (
            " (B4 H32 L4096 d128)" if name == "c3" else "")
    elif strict or bstrict:
        metric = (f"MXFP8 attn fwd/bwd TFLOP/s (causal-adj) on {name}, strict option ("
                  + " and ".join(x for x, on in (("forward V fold", strict), ("dQ K fold + per-query dS scales", bstrict))
                                 if on) + ")")
    elif name == "c3":
        metric = "MXFP8 attn fwd/bwd TFLOP/s (causal-adj) at B4 H32 L4096 d128, % of peak"
    else:
        metric = f"MXFP8 attn fwd/bwd TFLOP/s (causal-adj) on {name}"
    line = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4 scores + mxfp8" if fp4 else "mxfp8",
        "data": "synthetic",
        "config": dict({"workload": desc + ", bf16 N(0,1)-based synthetic inputs, step = quantise Q/K/V + fwd + bwd"
                        + (" with Q and K scored as MXFP4" if fp4 else "")
                        + (", the forward with the strict per-key V fold (V also quantised per token)" if strict else "")
                        + (", the backward with the strict dQ (K also quantised per token)" if bstrict else ""),
                        "head_dim": d, "causal": causal, "dq": args.dq, "score": args.score, "fwd": args.fwd, "bwd": args.bwd,
                        "dq_pass": "rebuilds dS" if args.recompute_dq else "reads stored dS codes"}, **cfg_line),
        "timing": {"rounds": args.rounds, "steps_per_round": args.steps, "ms_per_step_rounds": [round(r, 4) for r in rounds],
                   "statistic": "median of rounds, wall clock, no measurement hook",
                   "ms_per_step_roofline_round": round(ms_hooked, 4)},
        "pct_of_peak": round(100 * value / pk_step, 2),
        "fwd_tflops": round(tflops(f_fwd, ms_fwd), 2),
        "fwd_pct_of_peak": round(100 * tflops(f_fwd, ms_fwd) / pk_fwd, 2),
        "bwd_tflops": round(tflops(f_bwd, bwd_f32["call_ms"]), 2),
        "bwd_pct_of_peak": round(100 * tflops(f_bwd, bwd_f32["call_ms"]) / pk_bwd, 2),
        "bwd_f16dq_tflops": round(tflops(f_bwd, bwd_f16["call_ms"]), 2),
        "bwd_f16dq_pct_of_peak": round(100 * tflops(f_bwd, bwd_f16["call_ms"]) / pk_bwd, 2),
        **({"bwd_strict_tflops": round(tflops(f_bwd, res_bwd["strict"]["call_ms"]), 2),
            "bwd_strict_call_ms": round(res_bwd["strict"]["call_ms"], 4),
            "attn_bwd_dq_strict_ms": round(res_bwd["strict"]["dq_ms"], 4)} if "strict" in res_bwd else {}),
        **({"bwd_f16prefix_tflops": round(tflops(f_bwd, res_bwd["f16prefix"]["call_ms"]), 2),
            "bwd_f16prefix_call_ms": round(res_bwd["f16prefix"]["call_ms"], 4),
            "bwd_f16prefix_prep_ms": round(res_bwd["f16prefix"]["prep_ms"], 4),
            "attn_bwd_dq_f16prefix_ms": round(res_bwd["f16prefix"]["dq_ms"], 4)} if "f16prefix" in res_bwd else {}),
        "peaks_tflops": {"step": round(pk_step, 1), "fwd": round(pk_fwd, 1), "bwd": round(pk_bwd, 1)},
        "quantize_gbs": round(quant_bytes / (ms_quant * 1e-3) / 1e9, 1),
        "quantize_token_block_gbs": None if ms_quant_tb is None else round(quant_bytes / (ms_quant_tb * 1e-3) / 1e9, 1),
        "kernels_ms": {"attn_fwd": round(ms_fwd, 4),
                       **({"attn_fwd_plain": round(ms_fwd_plain, 4)} if strict else {}),
                       "attn_bwd_dkdv": round(bwd_f32["dkdv_ms"], 4),
                       "attn_bwd_dq_f32": round(bwd_f32["dq_ms"], 4), "attn_bwd_dq_f16": round(bwd_f16["dq_ms"], 4),
                       "bwd_prep": round(bwd_f32["prep_ms"], 4), "quantize_one_tensor": round(ms_quant, 4)},
        "flops": {"fwd": f_fwd, "bwd": f_bwd, "visible_pairs": pairs},
        "pages_context": {"fa4_mx8_fwd_pflops_gb300": 2.85, "fa4_mx8_bwd_pflops_gb300_f16dq": 1.98,
                          "fa4_mx8_bwd_pflops_gb300_f32dq": 1.82},
        "roofline": {"kernel": f"attn_bwd_dkdv_kernel<{d}> (backward dK/dV)", "bound": "mfma",
                     "achieved": round(tflops(f_dkdv, ms_bwd_main), 2), "peak": round(pk_dkdv, 1),
                     "unit": "TFLOP/s", "frac": round(tflops(f_dkdv, ms_bwd_main) / pk_dkdv, 4),
                     "traffic": recorded_traffic() if name == "c3" and not fp4 and not strict and not bstrict else None},
        "env": environment(),
    }
    if not args.no_cpu_baseline and name == "c3" and not fp4 and not strict and not bstrict:
        line["cpu_baseline"] = cpu_baseline(t, args.cpu_heads)
    print(json.dumps(line), flush=True)


def run_cross(args):
    """x1: one step = mx_quantize of Q (per query document) and K, V (per key document) + the
    cross-attention forward and backward. FLOPs: 4 d (forward) and 10 d (backward) per
    (query, key) pair of every document and head."""
    import numpy as np
    import torch

    import synth
    from block_scaled_mxfp8_amd import (MX_DQ_F16_BOOST, MX_DQ_F32, PROFILE_BWD_DKDV, PROFILE_BWD_DQ,
                                        PROFILE_BWD_PREP, PROFILE_FWD, PROFILE_QUANTIZE, load, mx_attn_cross_bwd,
                                        mx_attn_cross_fwd, mx_profile_kernel, mx_quantize)
    from block_scaled_mxfp8_amd.flops import attn_flops

    load()
    cfg = synth.CONFIGS["x1"]
    H, d = cfg["heads"], cfg["head_dim"]
    if args.dq == "f16prefix":
        sys.exit("--dq f16prefix is measured on the self-attention workloads")
    dq_mode = MX_DQ_F32 if args.dq == "f32" else MX_DQ_F16_BOOST
    print("[bench] generating x1 inputs on the device", file=sys.stderr, flush=True)
    x = synth.make_cross_inputs_device()
    nq, nk = np.diff(x["cu_q"]), np.diff(x["cu_k"])
    cq, ck = torch.from_numpy(x["cu_q"]).cuda(), torch.from_numpy(x["cu_k"]).cuda()
    mq, mk = int(nq.max()), int(nk.max())
    pairs = H * int(np.sum(nq * nk))
    f_fwd, f_bwd = attn_flops(pairs, d), attn_flops(pairs, d, backward=True)
    ws = {}

    def quant():
        return (mx_quantize(x["q"], cu_seqlens=cq, max_seqlen=mq), mx_quantize(x["k"], cu_seqlens=ck, max_seqlen=mk),
                mx_quantize(x["v"], cu_seqlens=ck, max_seqlen=mk))

    def step(mode=dq_mode):
        (q_row, q_seq), (k_row, k_seq), (v_row, v_seq) = quant()
        o, lse = mx_attn_cross_fwd(q_row, k_row, v_seq, cq, ck, mq, mk)
        dq, dk, dv, w = mx_attn_cross_bwd(q_row, q_seq, k_row, k_seq, v_row, o, lse, x["g"], cq, ck, mq, mk,
                                          dq_mode=mode, workspace=ws.get(mode))
        ws[mode] = w
        return o, dq

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    steps = max(1, args.steps)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    print(f"[bench] timed {steps} steps: {ms_step:.3f} ms/step", file=sys.stderr, flush=True)

    def kernel_ms(kind, fn, n=3):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in ev:
            a.record()
            b.record()
        mx_profile_kernel(kind, ev)
        torch.cuda.synchronize()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        mx_profile_kernel(0, [])
        return float(np.mean([a.elapsed_time(b) for a, b in ev]))

    (q_row, q_seq), (k_row, k_seq), (v_row, v_seq) = quant()
    o, lse = mx_attn_cross_fwd(q_row, k_row, v_seq, cq, ck, mq, mk)
    fwd = lambda: mx_attn_cross_fwd(q_row, k_row, v_seq, cq, ck, mq, mk)  # noqa: E731
    bwd = lambda: mx_attn_cross_bwd(q_row, q_seq, k_row, k_seq, v_row, o, lse, x["g"], cq, ck, mq, mk,  # noqa: E731
                                    dq_mode=dq_mode, workspace=ws[dq_mode])
    ms = {"attn_fwd": kernel_ms(PROFILE_FWD, fwd), "attn_bwd_dkdv": kernel_ms(PROFILE_BWD_DKDV, bwd),
          "attn_bwd_dq": kernel_ms(PROFILE_BWD_DQ, bwd), "bwd_prep": kernel_ms(PROFILE_BWD_PREP, bwd),
          "quantize_kv": kernel_ms(PROFILE_QUANTIZE, lambda: mx_quantize(x["k"], cu_seqlens=ck, max_seqlen=mk))}
    tflops = lambda f, t: f / (t * 1e-3) / 1e12  # noqa: E731
    f_dkdv = f_bwd * 4 // 5
    line = {
        "metric": "MXFP8 cross-attn fwd/bwd TFLOP/s, 768 docs x 512 queries vs jagged KV (<= 14980), H3 d128",
        "value": round(tflops(f_fwd + f_bwd, ms_step), 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8",
        "data": "synthetic",
        "config": {"workload": "x1: cross-attention, 768 documents x 512 queries, key/value lengths U[1, 14980] "
                               f"(total {int(nk.sum())}, max {mk}), H3 d128, non-causal, bf16 N(0,1); step = "
                               "quantise Q/K/V + fwd + bwd", "dq": args.dq},
        "pct_of_peak": round(100 * tflops(f_fwd + f_bwd, ms_step) / PEAK_MXFP8_TFLOPS, 2),
        "fwd_tflops": round(tflops(f_fwd, ms["attn_fwd"]), 2),
        "kernels_ms": {k: round(v, 4) for k, v in ms.items()},
        "flops": {"fwd": f_fwd, "bwd": f_bwd, "pairs": pairs},
        "roofline": {"kernel": "attn_bwd_dkdv_kernel<128> (backward dK/dV)", "bound": "mfma",
                     "achieved": round(tflops(f_dkdv, ms["attn_bwd_dkdv"]), 2), "peak": PEAK_MXFP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops(f_dkdv, ms["attn_bwd_dkdv"]) / PEAK_MXFP8_TFLOPS, 4),
                     "traffic": None},
    }
    print(json.dumps(line), flush=True)


def run_norm(args):
    """n1: one step = mx_rmsnorm_quantize of x [262144, 512] bf16 into both MX views.
    Algorithmic bytes: x read once (2 B/elem), gamma (2 B/column), both views written
    (2 x (1 + 1/32) B/elem)."""
    import numpy as np
    import torch

    import synth
    from block_scaled_mxfp8_amd import PROFILE_RMSNORM, load, mx_profile_kernel, mx_rmsnorm_quantize

    load()
    cfg = synth.CONFIGS["n1"]
    rows, n = cfg["rows"], cfg["n"]
    eps = 1e-6
    print("[bench] generating n1 inputs on the device", file=sys.stderr, flush=True)
    x, gamma = synth.make_norm_inputs_device()
    nbytes = rows * n * 2 + n * 2 + 2 * (rows * n + rows * n // 32)
    step = lambda: mx_rmsnorm_quantize(x, gamma, eps)  # noqa: E731
    if args.pmc_run:
        step()
        buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        buf2 = torch.empty_like(buf)
        buf2.copy_(buf)
        torch.cuda.synchronize()
        print("[bench] pmc run done", file=sys.stderr, flush=True)
        return
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    steps = max(1, args.steps)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    print(f"[bench] timed {steps} steps: {ms_step:.4f} ms/step", file=sys.stderr, flush=True)
    # the kernel alone, from HIP events the library records around it on its launch stream
    nev = max(1, args.profile_steps)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nev)]
    for a, b in ev:
        a.record()
        b.record()
    mx_profile_kernel(PROFILE_RMSNORM, ev)
    torch.cuda.synchronize()
    for _ in range(nev):
        step()
    torch.cuda.synchronize()
    mx_profile_kernel(0, [])
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    gbs = lambda t: nbytes / (t * 1e-3) / 1e9  # noqa: E731
    line = {
        "metric": "fused RMSNorm + MXFP8 quantise (both scale layouts) effective throughput at N=512",
        "value": round(gbs(ms_step) / 1e3, 3),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16->mxfp8",
        "data": "synthetic",
        "config": {"workload": f"n1: x [{rows}, {n}] bf16 (N(0,1) x per-row 2^U(-3,3), 4 outlier channels x20), "
                               "gamma 1 + 0.25 N(0,1), eps 1e-6; step = RMSNorm + ROW and SEQ MX views",
                   "rows": rows, "n": n},
        "bytes_per_step": nbytes,
        "kernel_ms": round(k_ms, 5),
        "pages_context": {"fused_rmsnorm_quantize_tbs_blackwell_n512": [2.6, 4.0],
                          "unfused_tbs_blackwell_n512": [0.75, 0.87]},
        "roofline": {"kernel": "rmsnorm_quantize_kernel<bf16, n <= 512>", "bound": "hbm",
                     "achieved": round(gbs(k_ms), 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs(k_ms) / PEAK_HBM_GBS, 4),
                     "traffic": recorded_traffic(NORM_TRAFFIC_FILE, NORM_KERNEL_SOURCES)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_norm(x, gamma, eps)
    print(json.dumps(line), flush=True)


def run_gemm(args):
    """g1: one step = mx_gemm_quantize of A [16384, 4096] and B [12288, 4096] (ROW views) into
    both MX views of C = A B^T. FLOPs 2 m n k; algorithmic bytes: both operands read once
    ((1 + 1/32) B per element) and both views of C written (2 x (1 + 1/32) B per element)."""
    import numpy as np
    import torch

    import synth
    from block_scaled_mxfp8_amd import PROFILE_GEMM, QView, load, mx_gemm_quantize, mx_profile_kernel

    load()
    cfg = synth.CONFIGS["g1"]
    m, n, k = cfg["m"], cfg["n"], cfg["k"]
    print("[bench] generating g1 operands on the device", file=sys.stderr, flush=True)
    a = QView(*synth.make_gemm_operand_device(m, k, "a"))
    b = QView(*synth.make_gemm_operand_device(n, k, "b"))
    torch.cuda.synchronize()
    flops = 2.0 * m * n * k
    nbytes = (m + n) * k * 33 // 32 + 2 * (m * n * 33 // 32)
    step = lambda: mx_gemm_quantize(a, b)  # noqa: E731
    if args.pmc_run:
        step()
        buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        buf2 = torch.empty_like(buf)
        buf2.copy_(buf)
        torch.cuda.synchronize()
        print("[bench] pmc run done", file=sys.stderr, flush=True)
        return
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    steps = max(1, args.steps)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    print(f"[bench] timed {steps} steps: {ms_step:.4f} ms/step", file=sys.stderr, flush=True)
    # the kernel alone, from HIP events the library records around it on its launch stream
    nev = max(1, args.profile_steps)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nev)]
    for e0, e1 in ev:
        e0.record()
        e1.record()
    mx_profile_kernel(PROFILE_GEMM, ev)
    torch.cuda.synchronize()
    for _ in range(nev):
        step()
    torch.cuda.synchronize()
    mx_profile_kernel(0, [])
    k_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    tflops = lambda t: flops / (t * 1e-3) / 1e12  # noqa: E731
    line = {
        "metric": "fused MXFP8 GEMM + quantise (both scale layouts of the output) TFLOP/s",
        "value": round(tflops(ms_step), 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8",
        "data": "synthetic",
        "config": {"workload": f"g1: C [{m}, {n}] = A [{m}, {k}] B^T, B [{n}, {k}], MXFP8 ROW-view operands "
                               "(log-normal E4M3 codes, E8M0 scales U[123,131] / U[118,126]); step = GEMM + "
                               "ROW and SEQ MX views of C",
                   "m": m, "n": n, "k": k},
        "pct_of_peak": round(100 * tflops(ms_step) / PEAK_MXFP8_TFLOPS, 2),
        "bytes_per_step": nbytes,
        "kernel_ms": round(k_ms, 5),
        "pages_context": {"fused_gemm_quantize_pflops_b200": [0.91, 0.98], "separate_gemm_then_quantize_pflops_b200": 0.20},
        "roofline": {"kernel": "gemm_quantize_kernel", "bound": "mfma",
                     "achieved": round(tflops(k_ms), 1), "peak": PEAK_MXFP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops(k_ms) / PEAK_MXFP8_TFLOPS, 4),
                     "traffic": recorded_traffic(GEMM_TRAFFIC_FILE, GEMM_KERNEL_SOURCES)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_gemm(a, b)
    print(json.dumps(line), flush=True)


def cpu_baseline_gemm(a, b, rows=4096):
    """The float64 oracle (as it stands) on the first `rows` rows of A against the whole of B."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001 - only used to report the thread count
        cores = os.cpu_count()
    ac, asc = a.codes[:rows].cpu().numpy(), a.scales[:rows].cpu().numpy()
    bc, bsc = b.codes.cpu().numpy(), b.scales.cpu().numpy()
    n, k = bc.shape
    t0 = time.perf_counter()
    oracle.gemm_quantize(ac, asc, bc, bsc)
    sec = time.perf_counter() - t0
    return {"value": round(2.0 * rows * n * k / sec / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "sample": f"first {rows} of {a.codes.shape[0]} rows of A against all of B "
                                        f"({n} x {k}), float64 numpy, {sec:.1f} s"}


def cpu_baseline_norm(x, gamma, eps, rows=32768):
    """The float64 oracle (as it stands) on the first `rows` rows of the n1 input."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001 - only used to report the thread count
        cores = os.cpu_count()
    xs = x[:rows].float().cpu().numpy().astype(np.float64)
    g = gamma.float().cpu().numpy().astype(np.float64)
    t0 = time.perf_counter()
    oracle.rmsnorm_quantize(xs, g, float(np.float32(eps)))
    sec = time.perf_counter() - t0
    n = xs.shape[1]
    nbytes = rows * n * 2 + n * 2 + 2 * (rows * n + rows * n // 32)
    return {"value": round(nbytes / sec / 1e12, 6), "unit": "TB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {rows} of {x.shape[0]} rows (n {n}), float64 numpy, {sec:.1f} s"}


def cpu_baseline(t, heads=24):
    """The C++ oracle (oracle/cpp, as it stands) on a bounded sample of the same workload:
    forward and backward of the first `heads` (batch, head) pairs of the c3 step (every pair
    is the same work), scaled to the metric's unit; heads=0 times every pair (the full tensor)."""
    import numpy as np
    import torch

    from block_scaled_mxfp8_amd.flops import attn_flops
    from oracle import fast
    B, H, L, d = t["q"].shape
    n_pairs = B * H if heads <= 0 else min(heads, B * H)
    pairs = [(i // H, i % H) for i in range(n_pairs)]
    sec = 0.0
    for bh in pairs:
        q, k, v, g = (t[n][bh].to(torch.float64).cpu().numpy() for n in ("q", "k", "v", "g"))
        t0 = time.perf_counter()
        f = fast.head_forward(q, k, v, True)
        fast.head_backward(q, k, v, f["O_out"], f["lse"].astype(np.float32), g, True)
        sec += time.perf_counter() - t0
    fl = n_pairs * (attn_flops(L * (L + 1) // 2, d) + attn_flops(L * (L + 1) // 2, d, backward=True))
    cores = int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))
    return {"value": round(fl / sec / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"fwd+bwd of {n_pairs} of {B * H} (batch, head) pairs (L{L} d{d} causal; every pair is "
                      f"the same work), C++17/OpenMP oracle with matrix-core-model scores, {sec:.1f} s; "
                      f"full tensor at this rate: {sec * B * H / n_pairs:.0f} s"}


if __name__ == "__main__":
    main()
