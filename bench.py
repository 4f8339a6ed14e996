#!/usr/bin/env python3
"""Throughput of the DiT attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload wan|qwen|cosmos|sp]
                    [--no-cpu-baseline]

One step is one pass of the whole path over one batch of synthetic input.
Default workload (Wan2.2 shape, B1 H40 S75600 D128, bf16 ~ N(0,1)), laid out
as the Ring Attention Overlap of the Wan2.2 NPU page on one GPU:
  1. (nothing to restore: the prologue reads the pristine q0, k0)
  2. qk_norm_rope_out(q0, k0 -> q, k): per-head RMSNorm (eps 1e-5) + 3D
     interleaved RoPE into the tensors the attention reads,
  3. attn_fwd_ws over the local quarter of the keys   -> fp32 out_a, lse_a,
  4. attn_fwd_ws_merge over the remaining three quarters (a window of the
     same K/V), whose epilogue merges each row into (out_a, lse_a) with the
     arithmetic of attn_merge (--separate-merge: attn_fwd_ws into fp32
     out_b, lse_b, then attn_merge(out_a, lse_a, out_b, lse_b); same bits).
Steps 3+4 cover every key once, so the attention work is exactly that of
full attention: 4*B*H*Sq*Skv*D FLOP per step.  Each attention call is two
kernels, the V rewrite into the workspace and the attention kernel; both sit
inside the timed interval of the call.

`value` is that attention FLOP count divided by the whole step's time
(TFLOP/s).  Kernel durations come from HIP events recorded on the stream the
kernels are launched on (torch's current stream).  The CPU baseline times the
fp64 oracle on a bounded sample of query rows on the host cores.

Other workloads (--workload) are per-config measurements:
  qwen / cosmos: prologue (out of place), attn_fwd_ws over all keys;
  sp: attn_fwd_ws + 3 x attn_fwd_ws_merge over KV chunks of 18900 keys (Sq 18900);
      --separate-merge: 4 x attn_fwd_ws + 3 fp32 attn_merge.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s and % of bf16 MFMA peak at 1 MI355X; oracle-match"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan", choices=["wan", "qwen", "cosmos", "sp", "ulysses"],
                    help="ulysses: only the BSND<->BNSD head-slice layout kernels of one rank of a 4-way "
                         "Ulysses split at the Wan2.2 shape (reported in GB/s)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fuse-q", action="store_true",
                    help="wan workload: apply the query RMSNorm+RoPE inside the attention's Q load "
                         "(attn_fwd_ws_fused_q); the prologue kernel then normalises k only")
    ap.add_argument("--separate-merge", action="store_true",
                    help="wan workload: the remote attention call writes its own fp32 output and a separate "
                         "attn_merge kernel folds it into the local one (default: attn_fwd_ws_merge merges in "
                         "the attention epilogue)")
    ap.add_argument("--ring-streams", type=int, default=1, choices=[1, 2],
                    help="wan workload: run the local and remote attention calls on one stream in order (1) "
                         "or concurrently on two streams (2)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run plain device copies of a known size (the reference for rocprofv3's "
                         "FETCH_SIZE/WRITE_SIZE counters) and print their byte counts")
    args = ap.parse_args()
    # The merging epilogue has no fused-Q variant: --fuse-q keeps the separate merge.
    args.fuse_merge = not (args.separate_merge or args.fuse_q)
    return args


def calibrate_copy():
    """Three device-to-device copies of 1 GiB each: every copy reads and
    writes exactly 2^30 bytes, so FETCH_SIZE/WRITE_SIZE of the copy kernel
    give the counters' scale."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").random_(0, 255)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy": {"bytes_read": n, "bytes_written": n, "copies": 3}}), flush=True)


def traffic_entry(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except ValueError:
        return None
    e = data.get(kernel, {}).get(workload)
    if not e:
        return None
    src = os.path.join(ROOT, "attention_qk_norm_rope_amd", "csrc", e["source"])
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    return e["bytes_per_launch"] if digest == e["sha256"] else None


def bench_ulysses(args):
    """bsnd_to_bnsd + bnsd_to_bsnd of one rank's 10 heads (4-way split) of
    B1 S75600 H40 D128 bf16: 2 bytes read + 2 written per element each way.
    Then that rank's attention (10 heads, 75600 keys) stored back into BSND,
    once as attn_fwd_ws + bnsd_to_bsnd and once as attn_fwd_ws_bsnd."""
    import torch
    from attention_qk_norm_rope_amd import (attn_fwd_workspace_bytes, attn_fwd_ws, attn_fwd_ws_bsnd, bnsd_to_bsnd,
                                            bsnd_to_bnsd)
    B, S, H, D, P = 1, 75600, 40, 128, 4
    hs = H // P
    dev = torch.device("cuda:0")
    x = torch.randn((B, S, H, D), device=dev).bfloat16()
    o = torch.empty((B, hs, S, D), dtype=torch.bfloat16, device=dev)
    y = torch.empty_like(x)

    def step(e):
        e[0].record()
        bsnd_to_bnsd(x, 0, hs, out=o)
        e[1].record()
        bnsd_to_bsnd(o, y, 0)
        e[2].record()

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(3)]  # noqa: E731
    for _ in range(args.warmup):
        step(mk())
    evs = [mk() for _ in range(args.steps)]
    torch.cuda.synchronize()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    nbytes = B * S * hs * D * 2 * 2
    t_pre = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    t_post = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    gbs = lambda t: round(nbytes / (t * 1e-3) / 1e9, 1)  # noqa: E731

    # The rank's attention with its output returned to BSND, two ways.
    q = bsnd_to_bnsd(x, 0, hs)
    k = bsnd_to_bnsd(x, hs, hs)
    v = bsnd_to_bnsd(x, 2 * hs, hs)
    ws = torch.empty((attn_fwd_workspace_bytes(B, hs, S, D),), dtype=torch.uint8, device=dev)
    ob = torch.empty((B, hs, S, D), dtype=torch.bfloat16, device=dev)

    def two_pass():
        attn_fwd_ws(q, k, v, ws, out=ob)
        bnsd_to_bsnd(ob, y, 0)

    def fused():
        attn_fwd_ws_bsnd(q, k, v, ws, y, out_h0=0)

    att = {}
    n_att = max(1, min(args.steps, 3))
    for name, fn in (("attn_fwd_ws+bnsd_to_bsnd", two_pass), ("attn_fwd_ws_bsnd", fused)):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n_att):
            fn()
        b.record()
        torch.cuda.synchronize()
        att[name] = round(a.elapsed_time(b) / n_att, 3)
    y2 = torch.empty_like(y)
    attn_fwd_ws(q, k, v, ws, out=ob)
    bnsd_to_bsnd(ob, y2, 0)
    attn_fwd_ws_bsnd(q, k, v, ws, y, out_h0=0)
    torch.cuda.synchronize()
    same = bool(torch.equal(y[:, :, :hs], y2[:, :, :hs]))
    print(json.dumps({
        "metric": "Ulysses head-slice layout GB/s (auxiliary measurement, not the headline metric)",
        "value": gbs((t_pre + t_post) / 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "one rank of a 4-way Ulysses split, B1 S75600 H40 D128: 10 heads BSND->BNSD "
                               "and back"},
        "kernels": {"bsnd_to_bnsd": {"avg_ms": round(t_pre, 4), "bytes": nbytes, "gbs": gbs(t_pre),
                                     "frac_hbm_peak": round(nbytes / (t_pre * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
                    "bnsd_to_bsnd": {"avg_ms": round(t_post, 4), "bytes": nbytes, "gbs": gbs(t_post),
                                     "frac_hbm_peak": round(nbytes / (t_post * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}},
        "attention_to_bsnd_ms": att, "attention_to_bsnd_same_bits": same,
    }), flush=True)


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.workload == "ulysses":
        if args.gpus != 1:
            print("bench.py measures one GPU only.", file=sys.stderr)
            sys.exit(2)
        bench_ulysses(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the design notes "
              "describe how the path would shard). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from attention_qk_norm_rope_amd import (attn_fwd_ring_overlap, attn_fwd_workspace_bytes, attn_fwd_ws,
                                            attn_fwd_ws_fused_q, attn_fwd_ws_merge, attn_merge, inputs,
                                            qk_norm_rope, qk_norm_rope_out)
    from attention_qk_norm_rope_amd import binding

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    binding._load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    wl = args.workload
    cfg = {"wan": inputs.WORKLOADS["wan"], "qwen": inputs.WORKLOADS["qwen"], "cosmos": inputs.WORKLOADS["cosmos"],
           "sp": inputs.WORKLOADS["wan_sp"]}[wl]
    log(f"[bench] generating inputs for {cfg.name}")
    t0 = time.time()
    x = inputs.make_inputs(cfg)
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s")
    B, H, D, S = cfg.B, cfg.H, cfg.D, cfg.S
    Sq, Skv = cfg.Sq, cfg.Skv
    scale = cfg.scale

    q0 = to_dev(x["q"])
    k0 = to_dev(x["k"])
    v = to_dev(x["v"])
    q = torch.empty_like(q0)
    k = torch.empty_like(k0)
    kernels = {}
    # One workspace, sized for the largest KV window of the step.
    ws_keys = {"wan": S - S // 4, "qwen": Skv, "cosmos": Skv, "sp": Skv // max(cfg.chunks, 1)}[wl]
    ws = torch.empty((attn_fwd_workspace_bytes(B, H, ws_keys, D),), dtype=torch.uint8, device=dev)

    if wl in ("wan", "qwen", "cosmos"):
        cos, sin = inputs.config_rope_tables(cfg)
        cos_d = torch.from_numpy(cos).to(dev)
        sin_d = torch.from_numpy(sin).to(dev)
        w_q = torch.from_numpy(x["w_q"]).to(dev)
        w_k = torch.from_numpy(x["w_k"]).to(dev)

    if wl == "wan" and args.ring_streams == 2:
        # Local and remote calls concurrently on two streams (own workspaces);
        # the attention interval spans both calls.
        c = S // 4
        out_a = torch.empty((B, H, Sq, D), dtype=torch.float32, device=dev)
        out_b = torch.empty_like(out_a)
        lse_a = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
        lse_b = torch.empty_like(lse_a)
        ws_local = torch.empty((attn_fwd_workspace_bytes(B, H, c, D),), dtype=torch.uint8, device=dev)
        side = torch.cuda.Stream(device=dev)
        names = ["qk_norm_rope", "attn_fwd+attn_merge"]

        def step(ev):
            ev[0].record()
            qk_norm_rope_out(q0, k0, q, k, w_q, w_k, cos_d, sin_d, cfg.eps)
            ev[1].record()
            attn_fwd_ring_overlap(q, k, v, c, ws_local, ws, out_local=out_a, lse_local=lse_a, out_remote=out_b,
                                  lse_remote=lse_b, scale=scale, side_stream=side)
            ev[2].record()

        final_out, final_lse = out_a, lse_a
        n_merge = 0
    elif wl == "wan":
        c = S // 4
        out_a = torch.empty((B, H, Sq, D), dtype=torch.float32, device=dev)
        out_b = torch.empty_like(out_a)
        lse_a = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
        lse_b = torch.empty_like(lse_a)
        names = ["qk_norm_rope", "attn_fwd", "attn_fwd"] + ([] if args.fuse_merge else ["attn_merge"])

        def attn(q_, k_, v_, out, lse, merge):
            # The query prologue either ran in place on q (q_ = q) or runs in
            # the attention's Q load (q_ = q0, --fuse-q).
            if merge:
                attn_fwd_ws_merge(q_, k_, v_, ws, out, lse, scale=scale)
            elif args.fuse_q:
                attn_fwd_ws_fused_q(q_, k_, v_, ws, w_q, cos_d, sin_d, cfg.eps, out=out, lse=lse, scale=scale)
            else:
                attn_fwd_ws(q_, k_, v_, ws, out=out, lse=lse, scale=scale)

        def step(ev):
            ev[0].record()
            if args.fuse_q:
                qk_norm_rope_out(None, k0, None, k, None, w_k, cos_d, sin_d, cfg.eps)
                q_ = q0
            else:
                qk_norm_rope_out(q0, k0, q, k, w_q, w_k, cos_d, sin_d, cfg.eps)
                q_ = q
            ev[1].record()
            attn(q_, k[:, :, :c], v[:, :, :c], out_a, lse_a, False)
            ev[2].record()
            if args.fuse_merge:
                attn(q_, k[:, :, c:], v[:, :, c:], out_a, lse_a, True)
                ev[3].record()
            else:
                attn(q_, k[:, :, c:], v[:, :, c:], out_b, lse_b, False)
                ev[3].record()
                attn_merge(out_a, lse_a, out_b, lse_b)
                ev[4].record()

        final_out, final_lse = out_a, lse_a
        merge_rows = B * H * Sq
        merge_bytes = merge_rows * (D * (4 + 4 + 4) + 12)
        n_merge = 0 if args.fuse_merge else 1
    elif wl in ("qwen", "cosmos"):
        out = torch.empty((B, H, Sq, D), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
        names = ["qk_norm_rope", "attn_fwd"]

        def step(ev):
            ev[0].record()
            qk_norm_rope_out(q0, k0, q, k, w_q, w_k, cos_d, sin_d, cfg.eps)
            ev[1].record()
            attn_fwd_ws(q, k, v, ws, out=out, lse=lse, scale=scale)
            ev[2].record()

        final_out, final_lse = out, lse
        n_merge = 0
    else:  # sp: one GPU's share of 4-way sequence parallelism
        n = cfg.chunks
        cs = Skv // n
        outs = [torch.empty((B, H, Sq, D), dtype=torch.float32, device=dev) for _ in range(n)]
        lses = [torch.empty((B, H, Sq), dtype=torch.float32, device=dev) for _ in range(n)]
        names = ["attn_fwd"] * n + ([] if args.fuse_merge else ["attn_merge"] * (n - 1))

        def step(ev):
            i_ev = 0
            ev[i_ev].record()
            for i in range(n):
                kc, vc = k0[:, :, i * cs:(i + 1) * cs], v[:, :, i * cs:(i + 1) * cs]
                if args.fuse_merge and i > 0:
                    attn_fwd_ws_merge(q0, kc, vc, ws, outs[0], lses[0], scale=scale)
                else:
                    attn_fwd_ws(q0, kc, vc, ws, out=outs[i], lse=lses[i], scale=scale)
                i_ev += 1
                ev[i_ev].record()
            if not args.fuse_merge:
                for i in range(1, n):
                    attn_merge(outs[0], lses[0], outs[i], lses[i])
                    i_ev += 1
                    ev[i_ev].record()

        final_out, final_lse = outs[0], lses[0]
        merge_rows = B * H * Sq
        merge_bytes = merge_rows * (D * (4 + 4 + 4) + 12)
        n_merge = 0 if args.fuse_merge else n - 1

    n_ev = len(names) + 1
    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]  # noqa: E731

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step(mk())
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    evs = [mk() for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(evs[i])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    log(f"[bench] {ms_per_step:.3f} ms/step (wall {wall * 1e3 / args.steps:.3f} ms/step)")

    # Per-kernel durations (ms summed per step, averaged over steps).
    per_kernel = {}
    for ev in evs:
        for j, nm in enumerate(names):
            per_kernel.setdefault(nm, []).append(ev[j].elapsed_time(ev[j + 1]))
    launches = {nm: names.count(nm) for nm in set(names)}

    attn_flops = cfg.flops()
    if "attn_fwd" in per_kernel:
        attn_ms_total = sum(per_kernel["attn_fwd"]) / args.steps          # per step
        n_attn = launches["attn_fwd"]
        entry = ("attn_fwd_ws (per call: v_prep_kernel, then attn_fwd_kernel; a last round that would fill at "
                 "most half the CUs runs as a second dispatch of 4-wave workgroups)")
        if wl in ("wan", "sp") and args.fuse_merge:
            entry = ("attn_fwd_ws + attn_fwd_ws_merge (per call: v_prep_kernel, then attn_fwd_kernel; a last round "
                     "that would fill at most half the CUs runs as a second dispatch of 4-wave workgroups; the "
                     "second call merges into the first's output in its epilogue)")
    else:
        # Two streams: the interval spans both overlapped calls and the merge.
        attn_ms_total = sum(per_kernel["attn_fwd+attn_merge"]) / args.steps
        n_attn = 2
        entry = ("attn_fwd_ring_overlap: 2 attn_fwd_ws calls on two streams + attn_merge "
                 "(avg_ms = overlapped span / 2)")
    attn_launch_ms = attn_ms_total / n_attn
    attn_tflops = attn_flops / (attn_ms_total * 1e-3) / 1e12
    kernels["attn_fwd"] = {"entry": entry,
                           "launches_per_step": n_attn, "avg_ms": round(attn_launch_ms, 4),
                           "flop_per_step": attn_flops, "tflops": round(attn_tflops, 2),
                           "frac_bf16_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4)}
    if "qk_norm_rope" in per_kernel:
        pro_ms = sum(per_kernel["qk_norm_rope"]) / args.steps
        pro_bytes = (1 if args.fuse_q else 2) * (2 + 2) * B * H * S * D + 2 * S * D * 4
        kernels["qk_norm_rope"] = {"avg_ms": round(pro_ms, 4), "bytes": pro_bytes,
                                   "gbs": round(pro_bytes / (pro_ms * 1e-3) / 1e9, 1),
                                   "frac_hbm_peak": round(pro_bytes / (pro_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    if n_merge:
        mer_ms = sum(per_kernel["attn_merge"]) / args.steps / n_merge
        kernels["attn_merge"] = {"launches_per_step": n_merge, "avg_ms": round(mer_ms, 4), "bytes": merge_bytes,
                                 "gbs": round(merge_bytes / (mer_ms * 1e-3) / 1e9, 1),
                                 "frac_hbm_peak": round(merge_bytes / (mer_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}

    value = attn_flops / (ms_per_step * 1e-3) / 1e12
    flop_per_launch = attn_flops / n_attn
    roofline = {"kernel": "attn_fwd_ws call (V rewrite + attention kernel)",
                "bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                "flop_per_launch": flop_per_launch, "traffic": traffic_entry("attn_fwd", wl)}

    workload_name = {
        "wan": "Wan2.2-shaped attention step B1 H40 S75600 D128: QK RMSNorm+3D RoPE, ring-overlap "
               "attention (local 1/4 + remote 3/4 of the keys" + (", on two streams" if args.ring_streams == 2
                                                                  else "") + "), fp32 LSE merge"
               + ("; query RMSNorm+RoPE fused into the attention's Q load" if args.fuse_q else "")
               + ("; merge in the remote call's epilogue" if args.fuse_merge else ""),
        "qwen": "Qwen-Image joint attention B1 H24 S4312 D128: QK RMSNorm+RoPE, attention",
        "cosmos": "Cosmos-Predict video attention B2 H16 S12480 D128: QK RMSNorm+3D RoPE, attention",
        "sp": "Wan2.2 4-way SP share: Sq 18900 x Skv 75600 H40 D128 as 4 KV chunks"
              + (" merged in the attention epilogue" if args.fuse_merge else " + 3 fp32 merges"),
    }[wl]
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 tensors; RMSNorm weights U(0.5,1.5))",
        "config": {"workload": workload_name, "B": B, "H": H, "Sq": Sq, "Skv": Skv, "D": D,
                   "causal": False, "scale": scale},
        "roofline": roofline, "kernels": kernels,
    }

    if not args.no_cpu_baseline:
        import oracle
        from oracle import compare
        rows = inputs.sample_rows(cfg.index, B, H, Sq, per_head=64)
        log(f"[bench] cpu baseline: oracle on {rows.size} rows")
        if wl == "sp":
            q_bits, k_bits = x["q"], x["k"]
        else:
            if args.fuse_q:
                # The fused step never writes q: the attention saw the prologue
                # of q0, which qk_norm_rope reproduces bit for bit.
                q.copy_(q0)
                qk_norm_rope(q, None, w_q, None, cos_d, sin_d, cfg.eps)
                torch.cuda.synchronize()
            q_bits = q.cpu().view(torch.int16).numpy().view(np.uint16)
            k_bits = k.cpu().view(torch.int16).numpy().view(np.uint16)
        threads = oracle.default_threads()
        t0 = time.perf_counter()
        ref_o, ref_l = oracle.attn(q_bits, k_bits, x["v"], scale, False, rows=rows, nthreads=threads)
        t_cpu = time.perf_counter() - t0
        cpu_tflops = rows.size * 4.0 * Skv * D / t_cpu / 1e12
        idx = torch.from_numpy(rows).to(dev)
        got_o = final_out.reshape(-1, D).index_select(0, idx).double().cpu().numpy()
        got_l = final_lse.reshape(-1).index_select(0, idx).double().cpu().numpy()
        rep = compare.attn_report(got_o, ref_o, got_l, ref_l, bf16=final_out.dtype == torch.bfloat16)
        result["cpu_baseline"] = {
            "value": cpu_tflops, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows.size} query rows (64 per (b,h)) of the measured workload against all "
                      f"{Skv} keys, fp64 two-pass softmax, {t_cpu:.1f} s; prologue and merge not timed",
            "seconds": round(t_cpu, 2)}
        result["oracle_match"] = {k2: (round(v2, 8) if isinstance(v2, float) else v2) for k2, v2 in rep.items()}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
