"""Benchmark of the single-GPU MoE layer (forward pass) on MI355X.

One step = one pass of the whole layer over one batch of synthetic input:
router GEMM + top-k -> histogram/scan/permute -> grouped expert GEMMs (up with
the token-row gather and the activation fused) -> [shared expert] -> down
projection -> combine (fused into the down projection's epilogue for top-1
routing) -> [aux loss] -> [bias step], each a C-ABI call into libmoe_hip.so
on one HIP stream.
Inputs are resident in HBM before the timed region starts.

Prints ONE JSON line.  `value` is layer tokens/s; `roofline` describes the
dominant kernel (the grouped up-projection GEMM with the fused activation:
algorithmic FLOPs over kept rows / its HIP-event time on the launch stream
inside the timed region; `traffic` = rocprofv3 FETCH_SIZE + WRITE_SIZE bytes
per call, scaled by a copy kernel, when taken on the current source);
`cpu_baseline` is the fp64 oracle timed on a bounded sample on the host.
`measured_ceilings` are the chip's read-stream and bf16 MFMA rates measured in the
same run by the library's probes; each roofline carries `frac_of_measured` (the
same achieved rate against them) next to `frac` (against the published peaks).
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

METRIC = "MoE layer tokens/sec @DeepSeek-V3 & Mixtral shapes; % MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 vector
# sources the up-projection kernel is compiled from (the traffic counters are tied to them)
GEMM_SRC = [os.path.join(ROOT, "mixture_experts_layer_histogram_amd", "csrc", f)
            for f in ("grouped_gemm.hip", "gemm_tile.h", "moe_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mixtral_prefill")
    ap.add_argument("--also", default="deepseek_v3,mixtral_decode",
                    help="comma-separated workloads measured after the main one and reported as sub-objects "
                         "of the same JSON line (the metric's other shapes); '' for none")
    ap.add_argument("--also-steps", type=int, default=20, help="timed steps of each --also workload")
    ap.add_argument("--oracle-tokens", type=int, default=None,
                    help="tokens in the CPU-baseline sample (default: whole batch for prefill shapes)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fp8-experts", action="store_true",
                    help="routed experts with fp8 (E4M3) weights and per-row scales, quantised before timing")
    ap.add_argument("--capacity-layout", choices=["packed", "padded"], default=None,
                    help="override the workload's capacity layout (padded: [E, C] expert buffers)")
    ap.add_argument("--capacity-priority", choices=["slot", "choice"], default=None,
                    help="override which slots an over-full expert keeps")
    ap.add_argument("--backward", action="store_true",
                    help="a training step: the forward (its up-projection keeping the pre-activations) plus "
                         "moe_backward (dout = seeded noise, d_aux = 1 with an aux loss); reports the backward's "
                         "time and algorithmic TFLOP/s")
    ap.add_argument("--no-library-reference", action="store_true",
                    help="skip timing the vendor library (torch.matmul, hipBLASLt) on the dense equivalent of the "
                         "up projection (a comparison point for the roofline, reported as library_reference)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip measuring the chip's read-stream and MFMA ceilings with the library's probes "
                         "(reported as measured_ceilings, with frac_of_measured next to each roofline frac)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one device copy of this many MiB first (a known-size reference for the "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def src_hash(paths):
    """Hash of the kernel sources with comments and layout removed, so that a
    comment edit does not mark counters taken on the same code as stale."""
    h = hashlib.sha256()
    for path in paths:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch of the dominant kernel from rocprofv3 counters, if
    they were taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        ent = t.get(workload)
        if ent and ent.get("kernel_src_sha256_16") == src_hash(GEMM_SRC):
            return ent["bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        pass
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's layer; --gpus {args.gpus} is not supported "
              "(this build uses a single GPU and no collectives)", file=sys.stderr)
        sys.exit(2)

    import torch
    from workloads import BY_NAME

    cfg = BY_NAME[args.config]
    if args.capacity_layout or args.capacity_priority:
        if args.capacity_layout == "padded" and cfg.capacity is None:
            print("--capacity-layout padded needs a workload with a capacity factor", file=sys.stderr)
            sys.exit(2)
        cfg = cfg.scaled(capacity_layout=args.capacity_layout or cfg.capacity_layout,
                         capacity_priority=args.capacity_priority or cfg.capacity_priority)
    torch.cuda.set_device(0)
    result, inp = measure(cfg, args, args.steps, args.warmup, fp8_experts=args.fp8_experts,
                          backward=args.backward, calib_copy_mib=args.calib_copy_mib)
    also = [a for a in args.also.split(",") if a and a != cfg.name] if not (args.backward or args.fp8_experts) else []
    if also:
        result["other_shapes"] = {}
    for name in also:
        print(f"bench: also measuring {name}", file=sys.stderr, flush=True)
        sub, _ = measure(BY_NAME[name], args, args.also_steps, args.warmup)
        result["other_shapes"][name] = {k: sub[k] for k in ("value", "unit", "ms_per_step", "config", "roofline",
                                                            "expert_gemms", "up_call_ms_timed", "breakdown_ms")}
    if not args.no_library_reference and cfg.dtype == "bf16" and not args.fp8_experts:
        result["library_reference"] = library_reference(cfg, result["config"]["kept_slots"])
    if not args.no_ceilings:
        try:
            ceil = measured_ceilings()
        except Exception as e:   # context only: the line is still printed without it
            print(f"bench: measured ceilings skipped ({e})", file=sys.stderr, flush=True)
            result["measured_ceilings"] = None
        else:
            result["measured_ceilings"] = ceil
            for sub in [result] + list(result.get("other_shapes", {}).values()):
                add_measured_fracs(sub, ceil)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, inp, args.oracle_tokens, args.fp8_experts)
    print(json.dumps(result), flush=True)


def measured_ceilings(hbm_gib=4, mfma_iters=400000, reps=5):
    """The chip's practical ceilings, measured in the same run by the library's probes: one
    read of a 4 GiB buffer (moe_probe_hbm_read: 16-byte nontemporal loads, one persistent
    workgroup per CU) and a stream of independent bf16 MFMAs on random operands on every
    wavefront (moe_probe_mfma_bf16).  Context for the roofline fractions, which stay against
    the published peaks."""
    import torch
    import mixture_experts_layer_histogram_amd as M
    buf = torch.empty(hbm_gib << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    ops = torch.randn(4096, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16).cuda()

    def timed(f):
        for _ in range(2):
            f()
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        evs[0].record()
        for i in range(reps):
            f()
            evs[i + 1].record()
        torch.cuda.synchronize()
        return float(np.median([evs[i].elapsed_time(evs[i + 1]) for i in range(reps)]))

    hbm_ms = timed(lambda: M.probe_hbm_read(buf, sink))
    mfma_ms = timed(lambda: M.probe_mfma_bf16(ops, mfma_iters, sink))
    flop = float(M.probe_mfma_flop_per_iter()) * mfma_iters
    nbytes = buf.numel()
    del buf
    torch.cuda.empty_cache()
    return {"hbm_read": {"kernel": "moe_probe_hbm_read", "bytes": nbytes, "ms": hbm_ms,
                         "GBps": nbytes / (hbm_ms * 1e-3) / 1e9},
            "mfma_bf16": {"kernel": "moe_probe_mfma_bf16", "flop": flop, "ms": mfma_ms,
                          "TFLOPs": flop / (mfma_ms * 1e-3) / 1e12},
            "note": "measured in this run on this GPU; roofline fractions stay against the published peaks "
                    "(HBM 8 TB/s, dense bf16 MFMA 2.5 PFLOP/s); frac_of_measured divides by these"}


def add_measured_fracs(res, ceil):
    """frac_of_measured next to frac: the same achieved rate against the measured ceilings."""
    roof = res.get("roofline")
    if roof and roof.get("bound") == "hbm":
        roof["frac_of_measured"] = roof["achieved"] / ceil["hbm_read"]["GBps"]
    elif roof and roof.get("bound") == "mfma":
        roof["frac_of_measured"] = roof["achieved"] / ceil["mfma_bf16"]["TFLOPs"]
    g = res.get("expert_gemms")
    if g:
        t = max(g["algorithmic_flop"] / (ceil["mfma_bf16"]["TFLOPs"] * 1e12),
                g["algorithmic_bytes"] / (ceil["hbm_read"]["GBps"] * 1e9)) * 1e3
        g["frac_of_measured"] = t / g["ms"]


def library_reference(cfg, kept, reps=10):
    """The vendor library (torch.matmul -> hipBLASLt) on the dense equivalent of the up
    projection: [kept, d] x [d, n_up F] bf16, N(0, 1) data (the MFMA rate depends on the
    data through the clock, so zeros or small integers would overstate it).  A comparison
    point for the up projection's roofline figure, not part of the layer."""
    import torch
    n_up = 2 if cfg.act == "swiglu" else 1
    M, K, Nc = max(int(kept), 1), cfg.d_model, n_up * cfg.d_ff
    gen = torch.Generator(device="cuda").manual_seed(3)
    a = torch.randn((M, K), device="cuda", generator=gen).to(torch.bfloat16)
    b = torch.randn((K, Nc), device="cuda", generator=gen).to(torch.bfloat16)
    for _ in range(3):
        c = torch.matmul(a, b)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    evs[0].record()
    for i in range(reps):
        c = torch.matmul(a, b)
        evs[i + 1].record()
    torch.cuda.synchronize()
    ms = float(np.median([evs[i].elapsed_time(evs[i + 1]) for i in range(reps)]))
    del a, b, c
    flop = 2.0 * M * K * Nc
    return {"op": f"torch.matmul bf16 [{M},{K}] x [{K},{Nc}]", "ms": ms, "tflops": flop / (ms * 1e-3) / 1e12,
            "frac_of_peak": flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def measure(cfg, args, steps, warmup, fp8_experts=False, backward=False, calib_copy_mib=0):
    """Time `steps` whole-layer steps of workload `cfg` (after `warmup` untimed ones) and return
    (the JSON fields of the measurement, the host inputs)."""
    import torch
    import mixture_experts_layer_histogram_amd as M
    from workloads import make_inputs

    dev_name = "cuda:0"
    t0 = time.perf_counter()
    inp = make_inputs(cfg)
    dev = M.upload_inputs(inp, dev_name)
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t0

    if calib_copy_mib > 0:
        n = calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev_name)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    c = M.config_from(cfg)
    N, E, k, d, F, Fs = cfg.n_tokens, cfg.n_experts, cfg.top_k, cfg.d_model, cfg.d_ff, cfg.d_ff_shared
    st = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    i32, f32 = torch.int32, torch.float32
    ws = torch.empty(M.workspace_size(c), dtype=torch.uint8, device=dev_name)
    z = torch.empty((N, E), dtype=f32, device=dev_name)
    idx = torch.empty((N, k), dtype=i32, device=dev_name)
    gates = torch.empty((N, k), dtype=f32, device=dev_name)
    probsum = torch.empty(E, dtype=f32, device=dev_name) if cfg.aux_loss else None
    counts = torch.empty(E, dtype=i32, device=dev_name)
    offs = torch.empty(E + 1, dtype=i32, device=dev_name)
    R = M._lib.expert_rows(c)           # rows of the expert-ordered buffers
    perm = torch.empty(max(R, 1), dtype=i32, device=dev_name)
    slot_pos = torch.empty(N * k, dtype=i32, device=dev_name)
    drop = torch.empty(1, dtype=torch.int64, device=dev_name)
    h = torch.empty((max(R, 1), F), dtype=st, device=dev_name)
    y = torch.empty((max(R, 1), d), dtype=st, device=dev_name)
    h_sh = torch.empty((N, Fs), dtype=st, device=dev_name) if Fs else None
    y_sh = torch.empty((N, d), dtype=st, device=dev_name) if Fs else None
    out = torch.empty((N, d), dtype=st, device=dev_name)
    aux = torch.empty(1, dtype=f32, device=dev_name) if cfg.aux_loss else None
    signs = torch.empty(E, dtype=torch.int8, device=dev_name)
    fp8 = None
    if fp8_experts:
        if cfg.dtype != "bf16":
            print("--fp8-experts needs a bf16 workload", file=sys.stderr)
            sys.exit(2)
        fp8 = {}
        for n in ("w1", "w3", "w2"):
            t = dev[n]
            if t is None:
                fp8[n] = (None, None)
                continue
            q = torch.empty(t.shape, dtype=torch.uint8, device=dev_name)
            sc = torch.empty(t.shape[:-1], dtype=torch.float32, device=dev_name)
            M.quantize_fp8(t, q, sc)
            fp8[n] = (q, sc)
        torch.cuda.synchronize()
    # the bias step writes a copy, so every timed step routes with the same selection bias
    sel_next = dev["sel_bias"].clone() if dev["sel_bias"] is not None else None
    residual = dev["x"] if cfg.residual else None

    names = ["route", "permute", "expert_up", "shared", "expert_down", "combine", "aux_bias"]
    bw = None
    if backward:
        if fp8 is not None or cfg.dtype != "bf16":
            print("--backward runs on bf16 weights", file=sys.stderr)
            sys.exit(2)
        names.append("backward")
        gen = torch.Generator(device=dev_name).manual_seed(7)
        dout = (torch.randn((N, d), device=dev_name, generator=gen) * 0.1).to(st)
        bw_grads = {"dx": torch.empty((N, d), dtype=st, device=dev_name),
                    "dw_router": torch.empty((E, d), dtype=f32, device=dev_name),
                    "dlogit_bias": torch.empty(E, dtype=f32, device=dev_name),
                    "dw1": torch.empty((E, F, d), dtype=f32, device=dev_name),
                    "dw2": torch.empty((E, d, F), dtype=f32, device=dev_name)}
        if cfg.act == "swiglu":
            bw_grads["dw3"] = torch.empty((E, F, d), dtype=f32, device=dev_name)
        if cfg.ffn_bias:
            bw_grads["db1"] = torch.empty((E, F), dtype=f32, device=dev_name)
            bw_grads["db2"] = torch.empty((E, d), dtype=f32, device=dev_name)
        if Fs:
            bw_grads["dsh_w1"] = torch.empty((Fs, d), dtype=f32, device=dev_name)
            bw_grads["dsh_w3"] = torch.empty((Fs, d), dtype=f32, device=dev_name)
            bw_grads["dsh_w2"] = torch.empty((d, Fs), dtype=f32, device=dev_name)
        bw_ws = torch.empty(M.backward_workspace_size(c), dtype=torch.uint8, device=dev_name)
        # the training forward keeps the up-projection's pre-activations for the backward
        pre_act = torch.empty((2 if cfg.act == "swiglu" else 1, max(R, 1), F), dtype=st, device=dev_name)
        bw_saved = {"logits": z, "topk_idx": idx, "gates": gates, "counts": counts, "offsets": offs,
                    "perm": perm, "slot_pos": slot_pos, "y_perm": y, "pre_act": pre_act}
        bw = (dout, bw_grads, bw_ws, bw_saved)

    fuse_combine = k == 1 and fp8 is None and bw is None and cfg.dtype == "bf16"

    def step(ev=None, up=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
            if up is not None and i in (2, 3):
                up[i - 2].record()
        mark(0)
        M.route(c, dev["x"], dev["w_router"], idx, gates, logit_bias=dev["logit_bias"], sel_bias=dev["sel_bias"],
                logits=z, probsum=probsum, ws=ws)
        mark(1)
        M.permute(c, idx, None, counts, offs, perm, slot_pos, None, drop_count=drop, ws=ws)
        mark(2)
        if bw is not None:
            M.expert_up_save(c, dev["x"], perm, offs, dev["w1"], dev["w3"], h, bw[3]["pre_act"], b1=dev["b1"], ws=ws)
        elif fp8 is None:
            M.expert_up_gather(c, dev["x"], perm, offs, dev["w1"], dev["w3"], h, b1=dev["b1"], ws=ws)
        else:
            M.expert_up_fp8(c, dev["x"], perm, offs, fp8["w1"][0], fp8["w3"][0], fp8["w1"][1], fp8["w3"][1], h,
                            b1=dev["b1"], ws=ws)
        mark(3)
        if Fs:
            M.shared_ffn(c, dev["x"], dev["sh_w1"], dev["sh_w3"], dev["sh_w2"], h_sh, y_sh, ws=ws)
        mark(4)
        if fuse_combine:   # top-1: the combine runs in the down projection's epilogue
            M.expert_down_combine(c, h, offs, perm, slot_pos, gates, dev["w2"], out, b2=dev["b2"],
                                  residual=residual, shared_y=y_sh, ws=ws)
        elif fp8 is None:
            M.expert_down(c, h, offs, dev["w2"], y, b2=dev["b2"], ws=ws)
        else:
            M.expert_down_fp8(c, h, offs, fp8["w2"][0], fp8["w2"][1], y, b2=dev["b2"], ws=ws)
        mark(5)
        if not fuse_combine:
            M.combine(c, y, slot_pos, gates, out, residual=residual, shared_y=y_sh)
        mark(6)
        if cfg.aux_loss:
            M.aux_loss(c, counts, probsum, aux)
        if cfg.gamma > 0:
            M.bias_update(c, counts, cfg.gamma, sel_next, signs)
        mark(7)
        if bw is not None:
            M.backward(c, dev, dev["x"], bw[0], bw[3], bw[1], d_aux=1.0 if cfg.aux_loss else 0.0, ws=bw[2])
            mark(8)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K whole steps; the only events inside bracket the dominant kernel (the up
    # projection call), whose duration the roofline figure needs.  The per-call breakdown comes
    # from a separate, untimed pass (its events would add ~2 us per call to the step).
    K = steps
    up_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start.record()
    for i in range(K):
        step(up=up_ev[i])
    stop.record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - w0
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / K
    up_ms_timed = float(np.mean([a.elapsed_time(b) for a, b in up_ev]))
    KB = max(1, min(K, 10))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(KB)]
    for i in range(KB):
        step(evs[i])
    torch.cuda.synchronize()
    parts = {n: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(KB)]))
             for j, n in enumerate(names)}

    kept = int((slot_pos >= 0).sum().item())     # kept slots (the padded layout's padding rows excluded)
    used = int((counts > 0).sum().item())
    n_up = 2 if cfg.act == "swiglu" else 1
    up_flop = 2.0 * n_up * d * F * kept
    down_flop = 2.0 * F * d * kept
    t_up = up_ms_timed * 1e-3                    # HIP events around the up call inside the timed region
    up_tflops = up_flop / t_up / 1e12
    expert_tflops = (up_flop + down_flop) / ((parts["expert_up"] + parts["expert_down"]) * 1e-3) / 1e12
    # algorithmic bytes of the up call: each used expert's weights once (+ fp8 row scales), the
    # token rows once, b1 rows of used experts; the h rows it writes are an intermediate of the
    # layer (read back by the down projection), reported apart as overhead
    esz = 2 if cfg.dtype == "bf16" else 4
    wsz = 1 if fp8 is not None else esz
    up_bytes = (used * n_up * F * (d * wsz + (4 if fp8 is not None else 0)) + N * d * esz
                + (used * F * esz if cfg.ffn_bias else 0))
    h_bytes = kept * F * esz
    # the expert GEMMs of the layer (up + down [+ shared]) against their own roofline: routed
    # weights of used experts, shared weights, x read and out written once; FLOPs of kept rows
    sh_flop = 6.0 * d * Fs * N
    gemm_flop = up_flop + down_flop + sh_flop
    gemm_bytes = (used * (n_up + 1) * F * (d * wsz + (4 if fp8 is not None else 0)) + 3 * Fs * d * esz
                  + 2 * N * d * esz + (used * (F + d) * esz if cfg.ffn_bias else 0))
    gemm_ms = parts["expert_up"] + parts["expert_down"] + parts["shared"]
    t_roof_ms = max(gemm_flop / (PEAK_BF16_TFLOPS * 1e12), gemm_bytes / (PEAK_HBM_GBS * 1e9)) * 1e3
    expert_gemms = {"ms": gemm_ms, "up_ms": parts["expert_up"], "down_ms": parts["expert_down"],
                    "shared_ms": parts["shared"], "algorithmic_flop": gemm_flop, "algorithmic_bytes": gemm_bytes,
                    "tflops": gemm_flop / (gemm_ms * 1e-3) / 1e12, "roofline_ms": t_roof_ms,
                    "frac": t_roof_ms / gemm_ms,
                    "bound": "mfma" if gemm_flop / (PEAK_BF16_TFLOPS * 1e12) >= gemm_bytes / (PEAK_HBM_GBS * 1e9)
                    else "hbm"}
    if cfg.dtype == "bf16":
        t_mfma, t_hbm = up_flop / (PEAK_BF16_TFLOPS * 1e12), up_bytes / (PEAK_HBM_GBS * 1e9)
        if t_mfma >= t_hbm:
            roof = {"bound": "mfma", "achieved": up_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
        else:
            gbs = up_bytes / t_up / 1e9
            roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:   # fp32 storage runs on the vector ALUs
        roof = {"bound": "alu", "achieved": up_tflops, "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    bw_flop = 2.0 * (up_flop + down_flop + 2.0 * N * d * E + 6.0 * d * Fs * N)
    traffic = measured_traffic(cfg.name) if fp8 is None else None

    result = {
        "metric": METRIC,
        "value": N / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded; random weights of the named shapes)",
        "config": {"workload": cfg.name, "n_tokens": N, "d_model": d, "n_experts": E, "top_k": k, "d_ff": F,
                   "d_ff_shared": Fs, "act": cfg.act, "gate_rule": cfg.gate_rule,
                   "capacity_factor": cfg.capacity_factor, "capacity_layout": cfg.capacity_layout,
                   "capacity_priority": cfg.capacity_priority, "expert_rows": R, "kept_slots": kept,
                   "used_experts": used,
                   "expert_weights": "fp8_e4m3_row_scaled" if fp8 is not None else cfg.dtype},
        "roofline": {"kernel": "expert up-projection grouped GEMM with fused row gather and activation "
                               "(grouped_gemm_big_kernel, grouped_gemm_small_kernel, split_fixup_kernel; one "
                               f"{'moe_expert_up_fp8' if fp8 is not None else ('moe_expert_up_save' if bw is not None else 'moe_expert_up_gather')} call)",
                     **roof, "traffic": traffic, "algorithmic_bytes": up_bytes, "algorithmic_flop": up_flop,
                     "overhead_bytes_h": h_bytes},
        "expert_gemm_tflops": expert_tflops,
        "expert_gemms": expert_gemms,
        **({"backward": {"ms": parts["backward"],
                         "algorithmic_tflop": bw_flop / 1e12,
                         "tflops": bw_flop / (parts["backward"] * 1e-3) / 1e12,
                         "note": "dx, router, expert and shared-expert gradients; algorithmic FLOPs = the two "
                                 "products per forward product (input and weight gradients); the routed "
                                 "pre-activations come from the forward (moe_expert_up_save), the shared "
                                 "expert's are recomputed"}} if bw is not None else {}),
        "up_call_ms_timed": up_ms_timed,
        "breakdown_ms": parts,
        "breakdown_note": f"per-call HIP-event times from {KB} further steps after the timed region",
        "wall_s_timed": wall_s,
        "input_gen_s": gen_s,
    }

    return result, inp


def cpu_baseline(cfg, inp, n_tok, fp8=False):
    """Time the fp64 oracle (as it stands) on a bounded sample of the same workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count()
    N = cfg.n_tokens
    if n_tok is None:
        n_tok = N if N * cfg.d_model * cfg.d_ff <= 4096 * 4096 * 14336 else min(N, 256)
    n_tok = max(1, min(N, n_tok))
    sub = cfg.scaled(n_tokens=n_tok)
    sub_inp = type(inp)(cfg=sub, x=inp.x[:n_tok], w_router=inp.w_router, logit_bias=inp.logit_bias,
                        sel_bias=inp.sel_bias, w1=inp.w1, w3=inp.w3, w2=inp.w2, b1=inp.b1, b2=inp.b2,
                        sh_w1=inp.sh_w1, sh_w3=inp.sh_w3, sh_w2=inp.sh_w2)
    t0 = time.perf_counter()
    oracle.oracle_layer(sub, sub_inp, expert_weights="fp8" if fp8 else "stored")
    dt = time.perf_counter() - t0
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "seconds": dt,
            "sample": f"first {n_tok} of {N} tokens of {cfg.name}, whole layer in fp64"
                      f"{' with the fp8 round trip of the expert weights' if fp8 else ''} "
                      f"(routing, capacity and aux computed over the sample)"}


if __name__ == "__main__":
    main()
