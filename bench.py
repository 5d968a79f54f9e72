"""Benchmark of the VSA2 attention layer on one MI355X.

One step = the whole hot path on the 720p training shape (latent 44x48x104 =
219,648 tokens, B=1, 20 heads, d=128, bf16, per-sequence top64, skewed
query-cube scales): pooling, fused router, per-sequence TopK, fine-branch
forward, coarse branch + gate, coarse/gate backward and fine-branch backward,
all through the C-ABI library on device-resident inputs.

The JSON line reports effective TFLOP/s of the step (algorithmic FLOPs,
selected blocks only), per-call times, the roofline of the dominant kernel and
the CPU oracle timed on a bounded sample.
"""

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from video_dit_trainable_amd import vsa2  # noqa: E402
from video_dit_trainable_amd.configs import (WORKLOADS, compulsory_bytes, flops, gather_bytes,  # noqa: E402
                                             kernel_flops, op_bytes)
from video_dit_trainable_amd.inputs import (make_gate_inputs, make_grad_out, make_qkv,  # noqa: E402
                                            make_selection)

PEAK_BF16 = 2.5e15      # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12       # MI355X HBM3E, B/s

# kernels timed live with the library's event hooks, and their symbol names
TIMED = {"fine_fwd": (vsa2.K_FINE_FWD, "k_attn_fwd"), "bwd_dkdv": (vsa2.K_BWD_DKDV, "k_bwd_dkdv"),
         "bwd_dq": (vsa2.K_BWD_DQ, "k_bwd_dq"), "router_lse": (vsa2.K_ROUTER_LSE, "k_router (pass 1)"),
         "router_scores": (vsa2.K_ROUTER_SCORES, "k_router (pass 2)")}
# kernel sources each timed kernel is built from (hashed to tell whether stored counters are current);
# the fine kernels' traffic also depends on the work schedule their items come from
SOURCES = {"fine_fwd": ("attn_fwd.hip", "sched.hip"), "bwd_dkdv": ("attn_bwd.hip", "sched.hip"),
           "bwd_dq": ("attn_bwd.hip", "sched.hip"), "router_lse": ("router.hip",), "router_scores": ("router.hip",)}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(w, q, k, v, d_o, budget_s=20.0):
    """The oracle on a bounded sample of the same workload (head 0): router
    rows of spread-out query cubes, then fine forward + backward of query cubes
    on a seeded selection with the workload's budget, each part grown in
    batches until it has used about half of `budget_s`.  FLOPs use the GPU's
    algorithmic accounting (router pass + fine forward + backward of the
    sampled rows); the rate is in TFLOP/s."""
    from threadpoolctl import threadpool_info

    from oracle import vsa2_oracle as orc

    f64 = lambda t: t.float().cpu().double().numpy()
    # the video rows (with MMDiT text rows the oracle's backward would redo
    # every video row against the text keys on each call; the sample keeps to
    # the video part of the same work)
    qh, kh, vh, doh = (f64(t[0, 0, :w.L]) for t in (q, k, v, d_o))
    real = orc.token_valid(w.grid, w.block)
    lr = w.L // 8
    order = np.random.default_rng(0).permutation(w.nblk)
    n_router, t_router = 0, 0.0
    if w.router == "vsa":                   # the coarse scores of the whole head at once
        t0 = time.perf_counter()
        orc.coarse_scores(qh, kh, w.grid, bf16_pooled=True, block=w.block)
        t_router = time.perf_counter() - t0
        n_router = w.nblk
        fl = 2 * 2 * w.nblk * w.nblk * w.head_dim
    while w.router != "vsa" and t_router < budget_s / 2 and n_router < w.nblk:
        rows = np.sort(order[n_router:n_router + 32])
        t0 = time.perf_counter()
        orc.router_scores(qh, kh, w.grid, bf16_pooled=True, rows=rows, block=w.block)
        t_router += time.perf_counter() - t0
        n_router += len(rows)
    if w.router != "vsa":
        fl = n_router * (w.block // 8) * 2 * 2 * lr * w.head_dim
    rp, ci = make_selection(w)
    mask = orc.csr_to_mask(rp[0, 0].numpy(), ci[0, 0].numpy(), w.nblk)
    live = [int(i) for i in order if mask[i].any()]
    n_fine, pairs, t_fine = 0, 0, 0.0
    while t_fine < budget_s / 2 and n_fine < len(live):
        cubes = sorted(live[n_fine:n_fine + 16])
        sub = np.zeros_like(mask)
        sub[cubes] = mask[cubes]
        t0 = time.perf_counter()
        orc.fine_forward(qh, kh, vh, sub, rows=cubes, valid=real, block=w.block)
        orc.fine_backward(qh, kh, vh, sub, doh, valid=real, block=w.block)
        t_fine += time.perf_counter() - t0
        n_fine += len(cubes)
        pairs += int(sub.sum())
    fl += pairs * 4 * w.block * w.block * w.head_dim * 7 // 2
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    unit = "cubes" if w.block == 64 else "128-token blocks"
    note = "; video rows only, the text rows not sampled" if w.text else ""
    secs = t_router + t_fine
    return {"value": fl / secs / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "threading": f"the matrix products ran in numpy's BLAS on up to {int(threads)} threads; the oracle's "
                         "per-row and per-block loops, softmax and exponentials ran on one thread",
            "sample": f"head 0 of the same inputs: router rows of {n_router} query {unit} ({t_router:.1f} s) + "
                      f"fine fwd+bwd of {n_fine} query {unit}, {pairs} selected pairs ({t_fine:.1f} s); fp64 numpy"
                      f"{note}",
            "seconds": round(secs, 2), "cpu": cpu_model(), "host_cpus": os.cpu_count()}


def dense_attention(w, q, k, v, d_o, fwd_ms, step_ms):
    """Context for the pages' own headline (an attention speedup over a dense
    flash attention at about 220K tokens, [VSA2] §3.4 Fig. 8): the dense
    softmax attention over all L tokens that PyTorch-ROCm ships (torch SDPA,
    memory-efficient backend), on the same Q, K, V and dO, timed with torch
    events (1 warm-up, then the median of 3 forwards and of 2 forward +
    backward calls).  Not a part of this library, and not `value`."""
    if w.text or w.padded or w.batch != 1:
        return {"skipped": "timed on unpadded video-only workloads of batch 1"}
    from torch.nn.attention import SDPBackend, sdpa_kernel
    import torch.nn.functional as F

    def med(fn, reps):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    fl = 4.0 * w.L * w.L * w.head_dim * w.heads      # QK^T and PV over every pair, all heads
    out = {"what": "torch.nn.functional.scaled_dot_product_attention over all L tokens (PyTorch-ROCm, "
                   "memory-efficient backend), the same Q, K, V and dO; dense, no router",
           "dense_flops_fwd": fl}
    try:
        with sdpa_kernel([SDPBackend.EFFICIENT_ATTENTION]):
            fms = med(lambda: F.scaled_dot_product_attention(q, k, v), 3)
            out["fwd_ms"] = round(fms, 2)
            out["fwd_tflops"] = round(fl / (fms * 1e-3) / 1e12, 1)
            out["vsa2_fwd_ms"] = round(fwd_ms, 3)
            out["speedup_fwd"] = round(fms / fwd_ms, 2)
            if w.train:
                qg, kg, vg = (t.detach().clone().requires_grad_(True) for t in (q, k, v))

                def fb():
                    F.scaled_dot_product_attention(qg, kg, vg).backward(d_o)
                bms = med(fb, 2)
                del qg, kg, vg
                out["fwd_bwd_ms"] = round(bms, 2)
                out["fwd_bwd_tflops"] = round(3.5 * fl / (bms * 1e-3) / 1e12, 1)
                out["speedup_step"] = round(bms / step_ms, 2)
    except Exception as e:          # a backend this PyTorch build lacks: no context figure
        out["skipped"] = f"{type(e).__name__}: {str(e)[:200]}"
    torch.cuda.empty_cache()
    log(f"dense attention (torch SDPA): {out}")
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def describe(w):
    """The workload named by what it is, with its sizes."""
    T, Y, X = w.grid
    grid = f"latent {T}x{Y}x{X} = {w.L_real} tokens"
    if w.padded:
        Tp, Yp, Xp = w.pgrid
        grid += f" (padded to whole 4x4x4 cubes: {Tp}x{Yp}x{Xp} = {w.L} slots, pad masked)"
    what = ("full forward + backward of router, TopK, fine, coarse and gate" if w.train
            else "forward of router, TopK, fine, coarse and gate")
    skew = ", skewed query-cube scales" if w.skew else ""
    if w.text:
        skew += f", {w.text} MMDiT text tokens in the fine branch (dense video-text and text-video)"
    router = ("router pool 2x2x2" if w.router == "vsa2" else
              "VSA router baseline (coarse block scores, TopK per query block)")
    blocks = "4x4x4 cubes" if w.block == 64 else "128-token blocks of 4x4x8 (two cubes)"
    return (f"{'720p training' if w.name.startswith('train720') else w.name} shape: {grid}, B={w.batch}, "
            f"{w.heads} heads, d={w.head_dim}, {w.dtype}, {router}, {blocks}, "
            f"{'per-sequence ' if w.router == 'vsa2' else ''}top{w.topk}{skew}; {what}")


def source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for name in SOURCES[kernel] + ("common.h",):
        with open(os.path.join(ROOT, "video_dit_trainable_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when there is none or the kernel's source has changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(f"{kernel}/{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def copy_calibration(dev):
    """A plain device copy of known size (256 MiB read + 256 MiB written), for
    scaling the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    n = 64 << 20
    a = torch.randn(n, device=dev)
    b = torch.empty_like(a)
    torch.neg(a, out=b)
    torch.cuda.synchronize()
    log(f"copy calibration: torch.neg over {n * 4} bytes read and {n * 4} bytes written")


def measured_peaks(dev):
    """Peaks measured on this device, beside the vendor figures: a dense bf16
    GEMM through torch (hipBLASLt), 8192^3, and a plain 2 GiB device copy
    (bytes read + written). Medians of 10 runs each."""
    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    src = torch.empty(1 << 29, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)

    def med(fn):
        for _ in range(3):
            fn()
        ts = []
        for _ in range(10):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    gemm_ms = med(lambda: torch.mm(a, b))
    copy_ms = med(lambda: dst.copy_(src))
    out = {"bf16_gemm_tflops": round(2 * n ** 3 / (gemm_ms * 1e-3) / 1e12, 1),
           "copy_gbps": round(2 * src.numel() * 4 / (copy_ms * 1e-3) / 1e9, 1),
           "gemm": "torch.mm bf16 8192x8192x8192", "copy": "2 GiB device-to-device, read + write bytes"}
    del a, b, src, dst
    log(f"measured peaks: bf16 GEMM {out['bf16_gemm_tflops']} TFLOP/s, copy {out['copy_gbps']} GB/s")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="train720")
    ap.add_argument("--topk", type=int, default=None, help="override the workload's average KV blocks per query block")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense-attention context figure (torch SDPA over all tokens)")
    ap.add_argument("--no-sched", action="store_true",
                    help="run the fine branch one workgroup per cube instead of on the work schedule's pairs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain copy kernel of known size (for counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer shards by head "
              "across GPUs, which this library does not implement", file=sys.stderr)
        sys.exit(2)
    w = WORKLOADS[args.workload]
    if args.topk is not None:
        w = dataclasses.replace(w, name=f"{w.name}-top{args.topk}", topk=args.topk)  # no stored counters apply
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"generating inputs for {w.name} on the GPU")
    q, k, v = make_qkv(w, device=dev)
    log("Q, K, V ready")
    d_o = make_grad_out(w, device=dev)
    x, w_g = make_gate_inputs(w, device=dev, zero_gate=False)
    log("dO, X, W_g ready")
    p = vsa2.problem(w.batch, w.heads, w.head_dim, w.grid, w.dtype, block=w.block, text=w.text)
    layer = vsa2.Layer(p, w.topk, w.d_model, device=dev)
    torch.cuda.synchronize()

    st = torch.cuda.current_stream()
    names = ["pool", "route", "topk", "fine_fwd", "coarse_gate", "coarse_gate_bwd", "fine_bwd"]

    gr = layer.grads()      # allocated once, outside the timed region
    sched = None if args.no_sched else layer.sched
    # the CSC (and the KV-cube side of the schedule) feeds only the backward
    csc = (layer.col_ptr, layer.row_idx) if w.train else (None, None)
    torch.cuda.synchronize()

    def step_full(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(st)
        mark(0)
        vsa2.vsa2_pool(p, q, k, v, layer.pooled)
        mark(1)
        if w.router == "vsa":
            vsa2.vsa2_route_coarse(p, layer.pooled, layer.scores, layer.ws)
        else:
            vsa2.vsa2_route(p, layer.pooled, layer.scores, layer.ws)
        mark(2)
        if w.router == "vsa":
            vsa2.vsa2_topk_per_row(p, layer.scores, w.topk, layer.row_ptr, layer.col_idx, *csc, layer.ws,
                                   sched=sched)
        else:
            vsa2.vsa2_topk_per_seq(p, layer.scores, w.topk, layer.row_ptr, layer.col_idx, *csc, layer.ws,
                                   sched=sched)
        mark(3)
        vsa2.vsa2_sparse_attn_fwd(p, w.topk, q, k, v, layer.row_ptr, layer.col_idx, layer.o_f, layer.lse, layer.ws,
                                  sched=sched)
        mark(4)
        vsa2.vsa2_coarse_gate(p, layer.pooled, x, w.d_model, w_g, layer.o_f, layer.o, layer.saved, layer.ws)
        mark(5)
        if w.train:
            vsa2.vsa2_coarse_gate_bwd(p, layer.pooled, x, w.d_model, w_g, layer.saved, d_o, gr["dqkv_c"], gr["dx"],
                                      gr["dw_g"], layer.ws)
        mark(6)
        if w.train:
            vsa2.vsa2_sparse_attn_bwd(p, w.topk, q, k, v, layer.o_f, layer.lse, d_o, layer.row_ptr, layer.col_idx,
                                      layer.col_ptr, layer.row_idx, gr["dqkv_c"], gr["dq"], gr["dk"], gr["dv"],
                                      layer.ws, sched=sched)
        mark(7)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step_full()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    for kid, _ in TIMED.values():
        vsa2.kernel_timer_start(kid, args.steps)
    t_start.record(st)
    for s in range(args.steps):
        step_full(evs[s])
    t_stop.record(st)
    torch.cuda.synchronize()
    kern = {}
    for name, (kid, _) in TIMED.items():
        ms, n = vsa2.kernel_timer_stop(kid)
        if n:
            kern[name] = ms / n
    log("per-kernel ms: " + ", ".join(f"{n} {t:.3f}" for n, t in kern.items()))
    total_ms = t_start.elapsed_time(t_stop)
    ms_step = total_ms / args.steps
    per = {n: float(np.median([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(args.steps)]))
           for i, n in enumerate(names) if w.train or n not in ("coarse_gate_bwd", "fine_bwd")}
    log("per-call ms: " + ", ".join(f"{n} {t:.3f}" for n, t in per.items()))
    steps_ms = [evs[s][0].elapsed_time(evs[s][7]) for s in range(args.steps)]
    step_dist = {"median": round(float(np.median(steps_ms)), 3), "min": round(float(np.min(steps_ms)), 3),
                 "p90": round(float(np.percentile(steps_ms, 90)), 3)}

    # cold steps: a 512 MiB write (larger than L2 and the 256 MB Infinity Cache)
    # before each, outside its events
    flush = torch.empty(128 << 20, dtype=torch.float32, device=dev)
    cold = []
    for _ in range(3):
        flush.fill_(1.0)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
        step_full(ev)
        torch.cuda.synchronize()
        cold.append(ev[0].elapsed_time(ev[7]))
    del flush
    log(f"step ms: median {step_dist['median']}, min {step_dist['min']}, p90 {step_dist['p90']}; "
        f"cold (after a 512 MiB flush) median {float(np.median(cold)):.3f}")

    fl = flops(w)
    step_flops = fl["router"] + fl["fine_fwd"] + fl["coarse_fwd"] + fl["gate_fwd"]
    if w.train:
        step_flops += fl["fine_bwd"] + fl["coarse_bwd"] + fl["gate_bwd"]
    value = step_flops / (ms_step * 1e-3) / 1e12

    # roofline of the dominant kernel (the timed kernel with the longest average
    # launch).  Every timed kernel is a dense contraction over the selected
    # tiles (the fine kernels) or the pooled operands (the router), so it is
    # priced against the bf16 MFMA peak on its credited FLOPs.  Beside it: the
    # bytes it must move at least (every input read once, every output written
    # once), the bytes its tile gathers would move with no reuse, and the
    # committed counters' bytes, which count L2 misses to the fabric (Infinity
    # Cache hits included), not HBM alone.
    kfl, kgb, kcb = kernel_flops(w), gather_bytes(w), compulsory_bytes(w)

    def kernel_rates(n, ms):
        sec = ms * 1e-3
        return kfl[n] / sec / 1e12, kcb[n] / sec / 1e9, kgb[n] / sec / 1e9

    dom = max(kern, key=kern.get)
    tf, cgb, ggb = kernel_rates(dom, kern[dom])
    traffic = stored_traffic(dom, w.name)
    roof = {"kernel": TIMED[dom][1], "bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16 / 1e12,
            "unit": "TFLOP/s", "frac": round(tf * 1e12 / PEAK_BF16, 4), "traffic": traffic,
            "traffic_kind": "L2-miss (fabric) bytes per launch from FETCH_SIZE + WRITE_SIZE, scaled by a copy "
                            "kernel; includes Infinity Cache hits",
            "avg_launch_ms": round(kern[dom], 4), "flops_per_launch": kfl[dom],
            "compulsory_bytes": kcb[dom], "gather_bytes_no_reuse": kgb[dom],
            "traffic_over_compulsory": round(traffic / kcb[dom], 2) if traffic else None,
            "flop_per_compulsory_byte": round(kfl[dom] / kcb[dom], 1),
            "ridge_flop_per_byte": round(PEAK_BF16 / PEAK_HBM, 1),
            "l2_miss_gbps": round(traffic / (kern[dom] * 1e-3) / 1e9, 1) if traffic else None}
    kernels = {}
    for n, t in kern.items():
        tf, cgb, ggb = kernel_rates(n, t)
        tr = stored_traffic(n, w.name)
        kernels[n] = {"ms": round(t, 4), "bound": "mfma", "tflops": round(tf, 2),
                      "pct_bf16_peak": round(100 * tf * 1e12 / PEAK_BF16, 2),
                      "compulsory_gbps": round(cgb, 1), "gather_gbps_no_reuse": round(ggb, 1),
                      "l2_miss_gbps": round(tr / (t * 1e-3) / 1e9, 1) if tr else None,
                      "traffic_over_compulsory": round(tr / kcb[n], 2) if tr else None}

    ops = {n: {"ms": round(t, 4)} for n, t in per.items()}
    for n, key in (("fine_fwd", "fine_fwd"), ("fine_bwd", "fine_bwd"), ("route", "router")):
        if n not in per:        # the backward calls of a forward-only step
            continue
        ops[n]["tflops"] = round(fl[key] / (per[n] * 1e-3) / 1e12, 2)
        ops[n]["pct_bf16_peak"] = round(100 * fl[key] / (per[n] * 1e-3) / PEAK_BF16, 2)
    # the router and TopK as a fraction of HBM bandwidth, on the bytes they move
    # as implemented (every pass counted)
    ob = op_bytes(w)
    for n in ("route", "topk", "pool"):
        ops[n]["bytes"] = ob[n]
        ops[n]["gbps"] = round(ob[n] / (per[n] * 1e-3) / 1e9, 1)
        ops[n]["pct_hbm"] = round(100 * ob[n] / (per[n] * 1e-3) / PEAK_HBM, 2)

    if args.copy_calibration:
        copy_calibration(dev)
    peaks = measured_peaks(dev)
    dense = None
    if not args.no_dense:
        fwd_ms = sum(per[n] for n in ("pool", "route", "topk", "fine_fwd", "coarse_gate"))
        dense = dense_attention(w, q, k, v, d_o, fwd_ms, ms_step)

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(w, q, k, v, d_o)

    out = {
        "metric": "ms/call + effective TFLOP/s (% bf16 MFMA peak), 220K tok, 20 heads, d128, top64",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": describe(w),
                   "global_batch": w.batch, "seq_len": w.L, "heads": w.heads, "head_dim": w.head_dim,
                   "topk": w.topk, "parallelism": "single GPU",
                   "fine_work": "per-cube workgroups" if sched is None else "work-schedule pairs"},
        "step_ms": step_dist,
        "cold_ms_per_step": round(float(np.median(cold)), 3),
        "step_flops": step_flops,
        "ops": ops,
        "kernels": kernels,
        "roofline": roof,
        "measured_peaks": peaks,
        "dense_attention": dense,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
