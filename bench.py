#!/usr/bin/env python3
"""Throughput of the DiT attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload wan|qwen|cosmos|sp|ulysses|plain]
                    [--no-cpu-baseline] [--no-configs]

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
kernels are launched on (torch's current stream); mean, median and min are
reported, with the engine clock and socket power sampled during the timed
steps.  The CPU baseline times the fp64 oracle on this process's CPU share:
attention on 64 sampled query rows per head (extrapolated to every row), the
prologue of q and k in full (also compared element by element with the GPU
prologue) and a merge of the step's full shape.

After the default step, the line's "configs" key reports the other
workloads, each timed in the same run and compared with the oracle on its
sampled rows: Wan2.2 with q x4 (logit std ~4), the 4-way SP share, Qwen-Image
and Cosmos-Predict (--no-configs skips them).

Other workloads (--workload) are per-config measurements:
  qwen / cosmos: prologue (out of place), attn_fwd_ws over all keys;
  sp: attn_fwd_ws + 3 x attn_fwd_ws_merge over KV chunks of 18900 keys (Sq 18900);
      --separate-merge: 4 x attn_fwd_ws + 3 fp32 attn_merge.
  ulysses: the head-slice layout kernels of one rank of a 4-way Ulysses split, and
      that rank's attention stored back into BSND two ways.
  plain: attn_fwd without a workspace against attn_fwd_ws at the Wan2.2 local
      window, Qwen-Image and Cosmos-Predict shapes, and a causal call.
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
    ap.add_argument("--workload", default="wan", choices=["wan", "qwen", "cosmos", "sp", "ulysses", "plain"],
                    help="ulysses: only the BSND<->BNSD head-slice layout kernels of one rank of a 4-way "
                         "Ulysses split at the Wan2.2 shape (reported in GB/s)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="wan workload: skip the timed runs of the other workloads (Wan2.2 Q x4, the SP share, "
                         "Qwen-Image, Cosmos-Predict) that the default line reports under 'configs'")
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
    ap.add_argument("--no-split", action="store_true",
                    help="give the attention calls a workspace of the V part only, which rules out the split "
                         "launch of a partly filled last round (for comparison)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run plain device copies of a known size (the reference for rocprofv3's "
                         "FETCH_SIZE/WRITE_SIZE counters) and print their byte counts")
    args = ap.parse_args()
    # The merging epilogue has no fused-Q variant: --fuse-q keeps the separate merge.
    args.fuse_merge = not (args.separate_merge or args.fuse_q)
    return args


NO_SPLIT = False


def ws_bytes(B: int, H: int, Skv: int, D: int) -> int:
    """Workspace bytes of an attention call: the library's full size, or the
    V part alone (no split launch) under --no-split."""
    from attention_qk_norm_rope_amd import attn_fwd_workspace_bytes
    if NO_SPLIT:
        return B * H * (-(-Skv // 64) * 64 * D * 2 + D * 4)
    return attn_fwd_workspace_bytes(B, H, Skv, D)


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
    ws = torch.empty((ws_bytes(B, hs, S, D),), dtype=torch.uint8, device=dev)
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


def bench_plain(args):
    """attn_fwd without a workspace (V staged through registers inside the
    attention kernel) against attn_fwd_ws (V rewritten into the workspace
    first, V rewrite included in its time), interleaved call by call with HIP
    events, at the Wan2.2 local window, the Qwen-Image and Cosmos-Predict
    shapes and a causal call (B1 H40 S18900; half the FLOP); fp32 output.  Where both take one 8-wave launch the outputs are
    the same bits; otherwise the workspace path's split launch differs in
    the last bits of the split tiles' rows."""
    import torch
    from attention_qk_norm_rope_amd import attn_fwd, attn_fwd_launch_form, attn_fwd_workspace_bytes, attn_fwd_ws
    dev = torch.device("cuda:0")
    shapes = [("Wan2.2 local window", 1, 40, 75600, 18900, False), ("Qwen-Image", 1, 24, 4312, 4312, False),
              ("Cosmos-Predict", 2, 16, 12480, 12480, False), ("causal, B1 H40 S18900", 1, 40, 18900, 18900, True)]
    D = 128
    n_rep = max(3, args.steps)
    res = {}
    for name, B, H, Sq, Skv, causal in shapes:
        g = torch.Generator(device=dev)
        g.manual_seed(Sq)
        q = torch.randn((B, H, Sq, D), device=dev, generator=g).bfloat16()
        k = torch.randn((B, H, Skv, D), device=dev, generator=g).bfloat16()
        v = torch.randn((B, H, Skv, D), device=dev, generator=g).bfloat16()
        ws = torch.empty((attn_fwd_workspace_bytes(B, H, Skv, D),), dtype=torch.uint8, device=dev)
        o_pl = torch.empty((B, H, Sq, D), dtype=torch.float32, device=dev)
        o_ws = torch.empty_like(o_pl)
        calls = {"attn_fwd": lambda: attn_fwd(q, k, v, out=o_pl, causal=causal, return_lse=False),
                 "attn_fwd_ws": lambda: attn_fwd_ws(q, k, v, ws, out=o_ws, causal=causal, return_lse=False)}
        ts = {c: [] for c in calls}
        for _ in range(max(1, args.warmup)):
            for fn in calls.values():
                fn()
        torch.cuda.synchronize()
        for _ in range(n_rep):
            for c, fn in calls.items():
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                fn()
                b.record()
                torch.cuda.synchronize()
                ts[c].append(a.elapsed_time(b))
        flop = 4.0 * B * H * Sq * Skv * D / (2 if causal else 1)
        entry = {"B": B, "H": H, "Sq": Sq, "Skv": Skv, "D": D, "causal": causal,
                 "ws_launch_form": attn_fwd_launch_form(B, H, Sq, Skv, D, causal, workspace_bytes=ws.numel())}
        for c in calls:
            med = _stats(ts[c])["median"]
            entry[c] = {"median_ms": round(med, 4), "tflops": round(flop / (med * 1e-3) / 1e12, 2),
                        "frac_bf16_peak": round(flop / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        entry["same_bits"] = bool(torch.equal(o_pl, o_ws))
        entry["max_abs_diff"] = float((o_pl - o_ws).abs().max())
        res[name] = entry
        log(f"[bench] plain {name}: attn_fwd {entry['attn_fwd']['frac_bf16_peak']:.4f}, "
            f"attn_fwd_ws {entry['attn_fwd_ws']['frac_bf16_peak']:.4f}")
    wan = res["Wan2.2 local window"]["attn_fwd"]
    print(json.dumps({
        "metric": "attn_fwd without a workspace, TFLOP/s (auxiliary measurement, not the headline metric)",
        "value": wan["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": n_rep, "warmup": args.warmup,
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "attn_fwd (no workspace) and attn_fwd_ws, fp32 output, at the Wan2.2 local window "
                               "(B1 H40 Sq75600 Skv18900), Qwen-Image (B1 H24 S4312), Cosmos-Predict "
                               "(B2 H16 S12480) and causal B1 H40 S18900, D128"},
        "shapes": res,
    }), flush=True)


def _stats(ts) -> dict:
    """Mean, median and min of a list of durations (ms)."""
    ts = sorted(float(t) for t in ts)
    n = len(ts)
    med = ts[n // 2] if n % 2 else 0.5 * (ts[n // 2 - 1] + ts[n // 2])
    return {"mean": sum(ts) / n, "median": med, "min": ts[0]}


class ClockSampler:
    """Reads the GPU engine (GFX) clock through amdsmi on a host thread while
    the timed steps run, so the line states the clock the kernels ran at (the
    card lowers it under its power limit).  The firmware refreshes its metrics
    table a few times a second, so a reading is kept only when the table's
    firmware timestamp is new since the timed steps began: a table left over
    from before them (idle, or the warm-up) is not counted."""

    def __init__(self, period_s: float = 0.02):
        self.period = period_s
        self.samples = []
        self.error = None
        self._stop = None
        self._thread = None
        self._read = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            h = amdsmi.amdsmi_get_processor_handles()[0]

            def read():
                m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                clks = [c for c in m["current_gfxclks"] if isinstance(c, (int, float))]
                return (m.get("firmware_timestamp"), sum(clks) / len(clks), float(m["current_socket_power"]))

            self._read = read
            self._read()
        except Exception as e:  # noqa: BLE001 - the clock is reported as unavailable
            self.error = f"amdsmi unavailable: {e!r}"
            self._read = None

    def start(self):
        if self._read is None:
            return
        import threading
        self._stop = threading.Event()
        try:
            seen = {self._read()[0]}
        except Exception as e:  # noqa: BLE001
            self.error = repr(e)
            return

        def run():
            while not self._stop.is_set():
                try:
                    ts, clk, pw = self._read()
                except Exception as e:  # noqa: BLE001
                    self.error = repr(e)
                    return
                if ts not in seen:
                    seen.add(ts)
                    self.samples.append((clk, pw))
                self._stop.wait(self.period)

        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()

    def stop(self) -> dict:
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        if not self.samples:
            return {"source": "amdsmi GFX clock", "error": self.error or "no metrics update during the timed steps"}
        clk = _stats([c for c, _ in self.samples])
        pw = _stats([p for _, p in self.samples])
        return {"source": "amdsmi GPU metrics (engine clock averaged over the XCDs, socket power): the metrics-table "
                          "updates that fell inside the timed steps",
                "median_mhz": round(clk["median"]), "min_mhz": round(clk["min"]),
                "max_mhz": round(max(c for c, _ in self.samples)), "median_socket_w": round(pw["median"]),
                "updates": len(self.samples)}


def _time_calls(fn, warmup: int, reps: int, n_marks: int):
    """Run fn(events) warmup + reps times; fn records n_marks + 1 HIP events
    on the current stream.  Returns, per interval, the list of the reps'
    durations (ms)."""
    import torch
    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(n_marks + 1)]  # noqa: E731
    for _ in range(warmup):
        fn(mk())
    evs = [mk() for _ in range(reps)]
    torch.cuda.synchronize()
    for e in evs:
        fn(e)
    torch.cuda.synchronize()
    return [[e[i].elapsed_time(e[i + 1]) for e in evs] for i in range(n_marks)]


def _attn_entry(name, ms_list, flop, extra=None) -> dict:
    st = _stats(ms_list)
    r = {"entry": name, "avg_ms": round(st["mean"], 4), "median_ms": round(st["median"], 4),
         "min_ms": round(st["min"], 4), "flop": flop,
         "tflops": round(flop / (st["median"] * 1e-3) / 1e12, 2),
         "frac_bf16_peak": round(flop / (st["median"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    if extra:
        r.update(extra)
    return r


def _bw_entry(ms_list, nbytes) -> dict:
    st = _stats(ms_list)
    gbs = nbytes / (st["median"] * 1e-3) / 1e9
    return {"avg_ms": round(st["mean"], 4), "median_ms": round(st["median"], 4), "min_ms": round(st["min"], 4),
            "bytes": nbytes, "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}


def _match(final_out, final_lse, rows, ref_o, ref_l, D):
    import torch
    from oracle import compare
    idx = torch.from_numpy(rows).to(final_out.device)
    got_o = final_out.reshape(-1, D).index_select(0, idx).double().cpu().numpy()
    got_l = final_lse.reshape(-1).index_select(0, idx).double().cpu().numpy()
    rep = compare.attn_report(got_o, ref_o, got_l, ref_l, bf16=final_out.dtype == torch.bfloat16)
    rep["rows"] = int(rows.size)
    return {k: (round(v, 8) if isinstance(v, float) else v) for k, v in rep.items()}


def run_configs(args, dev, wan) -> dict:
    """Attention of the other workloads, timed in the same run (HIP events on
    the current stream; median and min over the reps) and each compared with
    the oracle on its sampled rows."""
    import numpy as np
    import torch

    import oracle
    from attention_qk_norm_rope_amd import (attn_fwd_launch_form, attn_fwd_ws, attn_fwd_ws_merge, inputs,
                                            qk_norm_rope_out)
    res = {}

    def form(B_, H_, Sq_, Skv_, D_, w):
        return attn_fwd_launch_form(B_, H_, Sq_, Skv_, D_, workspace_bytes=w.numel())
    bits = lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16)  # noqa: E731

    # Wan2.2 Q x4: the normalised q times 4 (exact in bf16) through the same
    # two calls as the default step: logit std about 4.
    cfg = wan["cfg"]
    B, H, S, D = cfg.B, cfg.H, cfg.S, cfg.D
    c = S // 4
    q4 = wan["q"] * 4
    out = torch.empty((B, H, S, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    k, v, ws = wan["k"], wan["v"], wan["ws"]

    def wan_q4(e):
        e[0].record()
        attn_fwd_ws(q4, k[:, :, :c], v[:, :, :c], ws, out=out, lse=lse, scale=cfg.scale)
        attn_fwd_ws_merge(q4, k[:, :, c:], v[:, :, c:], ws, out, lse, scale=cfg.scale)
        e[1].record()

    log("[bench] configs: wan q x4")
    (t_att,) = _time_calls(wan_q4, 2, 5, 1)
    r = _attn_entry("attn_fwd_ws + attn_fwd_ws_merge (local 1/4 + remote 3/4 of the keys)", t_att, cfg.flops(),
                    {"workload": "Wan2.2 B1 H40 S75600 D128, normalised q x4 (logit std ~4)",
                     "launch_forms": {"local": form(B, H, S, c, D, ws), "remote": form(B, H, S, S - c, D, ws)}})
    if not args.no_cpu_baseline:
        rows = inputs.sample_rows(cfg.index, B, H, S, per_head=64)
        ref_o, ref_l = oracle.attn(bits(q4), bits(k), wan["v_bits"], cfg.scale, False, rows=rows)
        r["oracle_match"] = _match(out, lse, rows, ref_o, ref_l, D)
    res["wan_q4"] = r
    del q4

    # One GPU's share of 4-way sequence parallelism: 4 KV chunks folded into
    # an fp32 (out, lse) in the attention epilogue.
    sp = inputs.WORKLOADS["wan_sp"]
    n, cs = sp.chunks, sp.Skv // sp.chunks
    qs = wan["q0"][:, :, :sp.Sq].contiguous()
    k0 = wan["k0"]
    outs = torch.empty((B, H, sp.Sq, D), dtype=torch.float32, device=dev)
    lses = torch.empty((B, H, sp.Sq), dtype=torch.float32, device=dev)

    def sp_step(e):
        e[0].record()
        for i in range(n):
            kc, vc = k0[:, :, i * cs:(i + 1) * cs], v[:, :, i * cs:(i + 1) * cs]
            if i == 0:
                attn_fwd_ws(qs, kc, vc, ws, out=outs, lse=lses, scale=sp.scale)
            else:
                attn_fwd_ws_merge(qs, kc, vc, ws, outs, lses, scale=sp.scale)
        e[1].record()

    log("[bench] configs: sp share")
    (t_att,) = _time_calls(sp_step, 2, 10, 1)
    r = _attn_entry("attn_fwd_ws + 3 x attn_fwd_ws_merge (4 KV chunks of 18900 keys, fp32 accumulator)", t_att,
                    sp.flops(), {"workload": "Wan2.2 4-way SP share: Sq 18900 x Skv 75600, H40 D128",
                                 "launch_forms": {"chunk": form(B, H, sp.Sq, cs, D, ws)}})
    if not args.no_cpu_baseline:
        rows = inputs.sample_rows(sp.index, B, H, sp.Sq, per_head=64)
        qs_bits = np.ascontiguousarray(wan["q0_bits"][:, :, :sp.Sq])
        ref_o, ref_l = oracle.attn(qs_bits, wan["k0_bits"], wan["v_bits"], sp.scale, False, rows=rows)
        r["oracle_match"] = _match(outs, lses, rows, ref_o, ref_l, D)
    res["sp"] = r
    del outs, lses

    # Qwen-Image and Cosmos-Predict: prologue, then attention over all keys.
    to_dev = wan["to_dev"]
    for name, reps in (("qwen", 50), ("cosmos", 20)):
        cf = inputs.WORKLOADS[name]
        log(f"[bench] configs: {name}")
        x = inputs.make_inputs(cf)
        cos, sin = inputs.config_rope_tables(cf)
        q0c, k0c, vc = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
        qc, kc = torch.empty_like(q0c), torch.empty_like(k0c)
        w_q, w_k = torch.from_numpy(x["w_q"]).to(dev), torch.from_numpy(x["w_k"]).to(dev)
        cos_d, sin_d = torch.from_numpy(cos).to(dev), torch.from_numpy(sin).to(dev)
        wsc = torch.empty((ws_bytes(cf.B, cf.H, cf.Skv, cf.D),), dtype=torch.uint8, device=dev)
        oc = torch.empty((cf.B, cf.H, cf.Sq, cf.D), dtype=torch.bfloat16, device=dev)
        lc = torch.empty((cf.B, cf.H, cf.Sq), dtype=torch.float32, device=dev)

        def step(e):
            e[0].record()
            qk_norm_rope_out(q0c, k0c, qc, kc, w_q, w_k, cos_d, sin_d, cf.eps)
            e[1].record()
            attn_fwd_ws(qc, kc, vc, wsc, out=oc, lse=lc, scale=cf.scale)
            e[2].record()

        t_pro, t_att = _time_calls(step, 3, reps, 2)
        pro_bytes = 2 * (2 + 2) * cf.B * cf.H * cf.S * cf.D + 2 * cf.S * cf.D * 4
        r = _attn_entry("attn_fwd_ws", t_att, cf.flops(),
                        {"workload": f"{cf.name}: RMSNorm + RoPE prologue, attention over all keys",
                         "launch_forms": {"all keys": form(cf.B, cf.H, cf.Sq, cf.Skv, cf.D, wsc)},
                         "prologue": _bw_entry(t_pro, pro_bytes)})
        if not args.no_cpu_baseline:
            rows = inputs.sample_rows(cf.index, cf.B, cf.H, cf.Sq, per_head=64)
            ref_o, ref_l = oracle.attn(bits(qc), bits(kc), x["v"], cf.scale, False, rows=rows)
            r["oracle_match"] = _match(oc, lc, rows, ref_o, ref_l, cf.D)
        res[name] = r
        del q0c, k0c, vc, qc, kc, wsc, oc, lc
    return res


def cpu_baseline(args, cfg, x, q, k, w_q, w_k, cos, sin, final_out, final_lse, ms_per_step) -> tuple:
    """The oracle as it stands on this host's CPU share: attention on the
    sampled rows (extrapolated linearly to every row, exact for non-causal
    attention where each row costs 4*Skv*D FLOP), the prologue of q and k in
    full (compared with the GPU prologue element by element) and an fp32
    out/LSE merge of the step's full shape."""
    import numpy as np
    import torch

    import oracle
    from oracle import compare
    from attention_qk_norm_rope_amd import inputs
    B, H, S, D = cfg.B, cfg.H, cfg.S, cfg.D
    Sq, Skv = cfg.Sq, cfg.Skv
    threads = oracle.default_threads()
    rows = inputs.sample_rows(cfg.index, B, H, Sq, per_head=64)
    log(f"[bench] cpu baseline: attention oracle on {rows.size} rows, {threads} threads")
    q_bits = q.cpu().view(torch.int16).numpy().view(np.uint16)
    k_bits = k.cpu().view(torch.int16).numpy().view(np.uint16)
    t0 = time.perf_counter()
    ref_o, ref_l = oracle.attn(q_bits, k_bits, x["v"], cfg.scale, False, rows=rows, nthreads=threads)
    t_att = time.perf_counter() - t0
    match = _match(final_out, final_lse, rows, ref_o, ref_l, D)
    t_att_full = t_att * (B * H * Sq) / rows.size

    # Prologue oracle over every row of q and k, one head at a time (bounded
    # host memory), compared with the GPU prologue's output.
    log("[bench] cpu baseline: prologue oracle over all of q and k")
    t_pro = 0.0
    worst = {"max_abs": 0.0, "n_above_atol": 0, "max_err_over_bound": 0.0}
    dot = na = nb = 0.0
    finite = True
    for src, got, w in ((x["q"], q_bits, x["w_q"]), (x["k"], k_bits, x["w_k"])):
        for b in range(B):
            for h in range(H):
                t0 = time.perf_counter()
                ref = oracle.qk_norm_rope(np.ascontiguousarray(src[b:b + 1, h:h + 1]), w, cos, sin, cfg.eps,
                                          nthreads=threads)
                t_pro += time.perf_counter() - t0
                g = inputs.bf16_bits_to_f64(got[b:b + 1, h:h + 1])
                rep = compare.prologue_report(g, ref)
                worst["max_abs"] = max(worst["max_abs"], rep["max_abs"])
                worst["n_above_atol"] += rep["n_above_atol"]
                worst["max_err_over_bound"] = max(worst["max_err_over_bound"], rep["max_err_over_bound"])
                dot += float(np.dot(g.ravel(), ref.ravel()))
                na += float(np.dot(g.ravel(), g.ravel()))
                nb += float(np.dot(ref.ravel(), ref.ravel()))
                finite = finite and bool(np.isfinite(g).all())
    cos_sim = dot / math.sqrt(na * nb) if na > 0 and nb > 0 else 1.0
    pro_match = {k2: round(v2, 8) if isinstance(v2, float) else v2 for k2, v2 in worst.items()}
    pro_match["cos"] = round(cos_sim, 10)
    pro_match["elements"] = int(2 * B * H * S * D)
    pro_match["ok"] = bool(finite and worst["max_err_over_bound"] <= 1.0 and cos_sim >= compare.COS_MIN)

    # Merge oracle over every row of the step's fp32 (out, lse) shape; the
    # values are the step's output on both sides (the time does not depend
    # on them).  It is timed in slices of heads.
    log("[bench] cpu baseline: merge oracle over all rows")
    t_mer = 0.0
    for b in range(B):
        for h0 in range(0, H, 8):
            o = final_out[b, h0:h0 + 8].double().cpu().numpy()
            l = final_lse[b, h0:h0 + 8].double().cpu().numpy()
            t0 = time.perf_counter()
            oracle.merge(o, l, o, l)
            t_mer += time.perf_counter() - t0
    total = t_att_full + t_pro + t_mer
    base = {
        "value": rows.size * 4.0 * Skv * D / t_att / 1e12, "unit": "TFLOP/s", "cores": threads,
        "host_cpus": os.cpu_count(), "kind": "oracle",
        "sample": (f"attention: {rows.size} query rows (64 per (b,h)) of the measured workload against all {Skv} "
                   f"keys, fp64 two-pass softmax, {t_att:.1f} s, extrapolated to all {B * H * Sq} rows; "
                   f"prologue: all of q and k in full, {t_pro:.1f} s; merge: all {B * H * Sq} rows in full "
                   f"(single-threaded), {t_mer:.1f} s"),
        "seconds": round(t_att, 2), "threads_note": "cores = the threads the oracle ran on: this process's CPU "
                                                    "share (OMP_NUM_THREADS when set, else its CPU affinity)",
        "attention_s_sampled": round(t_att, 2), "attention_s_extrapolated": round(t_att_full, 1),
        "prologue_s_full": round(t_pro, 2), "merge_s_full": round(t_mer, 2),
        "step_s_extrapolated": round(total, 1), "gpu_step_s": round(ms_per_step * 1e-3, 5),
        "oracle_over_gpu": round(total / (ms_per_step * 1e-3), 0)}
    return base, match, pro_match


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.workload in ("ulysses", "plain"):
        if args.gpus != 1:
            print("bench.py measures one GPU only.", file=sys.stderr)
            sys.exit(2)
        (bench_ulysses if args.workload == "ulysses" else bench_plain)(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the design notes "
              "describe how the path would shard). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    global NO_SPLIT
    NO_SPLIT = args.no_split
    from attention_qk_norm_rope_amd import (attn_fwd_launch_form, attn_fwd_ring_overlap, attn_fwd_workspace_bytes,
                                            attn_fwd_ws,
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
    ws = torch.empty((ws_bytes(B, H, ws_keys, D),), dtype=torch.uint8, device=dev)
    w_q = w_k = cos_d = sin_d = cos = sin = None
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
        ws_local = torch.empty((ws_bytes(B, H, c, D),), dtype=torch.uint8, device=dev)
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
        out_b = torch.empty_like(out_a) if not args.fuse_merge else None
        lse_a = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
        lse_b = torch.empty_like(lse_a)
        names = ["qk_norm_rope", "attn_fwd", "attn_fwd"] + ([] if args.fuse_merge else ["attn_merge"])

        def attn(q_, k_, v_, out, lse, merge):
            # The query prologue either ran on q (q_ = q) or runs in the
            # attention's Q load (q_ = q0, --fuse-q).
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
    clock = ClockSampler()
    torch.cuda.synchronize()
    clock.start()
    t_wall = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(evs[i])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    sclk = clock.stop()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    step_stats = _stats([ev[0].elapsed_time(ev[-1]) for ev in evs])
    log(f"[bench] {ms_per_step:.3f} ms/step (wall {wall * 1e3 / args.steps:.3f} ms/step)")

    # Per-kernel durations (ms summed per step).
    per_kernel = {}
    for ev in evs:
        acc = {}
        for j, nm in enumerate(names):
            acc[nm] = acc.get(nm, 0.0) + ev[j].elapsed_time(ev[j + 1])
        for nm, t in acc.items():
            per_kernel.setdefault(nm, []).append(t)
    launches = {nm: names.count(nm) for nm in set(names)}

    attn_flops = cfg.flops()
    if "attn_fwd" in per_kernel:
        n_attn = launches["attn_fwd"]
        entry = ("attn_fwd_ws (per call: the V rewrite kernels, then the attention launches of the form in "
                 "launch_forms: full rounds of 8-wave workgroups, and a partly filled last round as a split "
                 "launch over its key tiles or as 4-wave halves)")
        if wl in ("wan", "sp") and args.fuse_merge:
            entry = ("attn_fwd_ws + attn_fwd_ws_merge (per call: the V rewrite kernels, then the attention "
                     "launches of the form in launch_forms: full rounds of 8-wave workgroups, and a partly filled "
                     "last round as a split launch over its key tiles or as 4-wave halves; the second call merges "
                     "into the first's output in its epilogue)")
        attn_list = per_kernel["attn_fwd"]
    else:
        # Two streams: the interval spans both overlapped calls and the merge.
        n_attn = 2
        entry = ("attn_fwd_ring_overlap: 2 attn_fwd_ws calls on two streams + attn_merge "
                 "(avg_ms = overlapped span / 2)")
        attn_list = per_kernel["attn_fwd+attn_merge"]
    ast = _stats(attn_list)
    attn_tflops = attn_flops / (ast["mean"] * 1e-3) / 1e12
    kernels["attn_fwd"] = {"entry": entry, "launches_per_step": n_attn,
                           "avg_ms": round(ast["mean"] / n_attn, 4),
                           "median_ms": round(ast["median"] / n_attn, 4), "min_ms": round(ast["min"] / n_attn, 4),
                           "flop_per_step": attn_flops, "tflops": round(attn_tflops, 2),
                           "tflops_median": round(attn_flops / (ast["median"] * 1e-3) / 1e12, 2),
                           "tflops_best": round(attn_flops / (ast["min"] * 1e-3) / 1e12, 2),
                           "frac_bf16_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4)}
    kv_calls = {"wan": {"local": S // 4, "remote": S - S // 4}, "sp": {"chunk": Skv // max(cfg.chunks, 1)}}.get(
        wl, {"all keys": Skv})
    kernels["attn_fwd"]["launch_forms"] = {
        nm: attn_fwd_launch_form(B, H, Sq, n, D, workspace_bytes=ws.numel()) for nm, n in kv_calls.items()}
    if "qk_norm_rope" in per_kernel:
        pro_bytes = (1 if args.fuse_q else 2) * (2 + 2) * B * H * S * D + 2 * S * D * 4
        kernels["qk_norm_rope"] = _bw_entry(per_kernel["qk_norm_rope"], pro_bytes)
    if n_merge:
        kernels["attn_merge"] = _bw_entry([t / n_merge for t in per_kernel["attn_merge"]], merge_bytes)
        kernels["attn_merge"]["launches_per_step"] = n_merge

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
        "ms_per_step_median": round(step_stats["median"], 3), "ms_per_step_min": round(step_stats["min"], 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 tensors; RMSNorm weights U(0.5,1.5))",
        "config": {"workload": workload_name, "B": B, "H": H, "Sq": Sq, "Skv": Skv, "D": D,
                   "causal": False, "scale": scale},
        "roofline": roofline, "kernels": kernels, "sclk": sclk,
    }

    if not args.no_cpu_baseline:
        if wl == "sp" or args.fuse_q or args.ring_streams == 2 or wl != "wan":
            # The per-workload runs keep the short baseline: attention rows only.
            import oracle
            rows = inputs.sample_rows(cfg.index, B, H, Sq, per_head=64)
            log(f"[bench] cpu baseline: oracle on {rows.size} rows")
            if wl == "sp":
                q_bits, k_bits = x["q"], x["k"]
            else:
                if args.fuse_q:
                    # The fused step never writes q: the attention saw the
                    # prologue of q0, which qk_norm_rope reproduces bit for bit.
                    q.copy_(q0)
                    qk_norm_rope(q, None, w_q, None, cos_d, sin_d, cfg.eps)
                    torch.cuda.synchronize()
                q_bits = q.cpu().view(torch.int16).numpy().view(np.uint16)
                k_bits = k.cpu().view(torch.int16).numpy().view(np.uint16)
            threads = oracle.default_threads()
            t0 = time.perf_counter()
            ref_o, ref_l = oracle.attn(q_bits, k_bits, x["v"], scale, False, rows=rows, nthreads=threads)
            t_cpu = time.perf_counter() - t0
            result["cpu_baseline"] = {
                "value": rows.size * 4.0 * Skv * D / t_cpu / 1e12, "unit": "TFLOP/s", "cores": threads,
                "host_cpus": os.cpu_count(), "kind": "oracle",
                "sample": f"{rows.size} query rows (64 per (b,h)) of the measured workload against all "
                          f"{Skv} keys, fp64 two-pass softmax, {t_cpu:.1f} s",
                "seconds": round(t_cpu, 2)}
            result["oracle_match"] = _match(final_out, final_lse, rows, ref_o, ref_l, D)
        else:
            base, match, pro_match = cpu_baseline(args, cfg, x, q, k, w_q, w_k, cos, sin, final_out, final_lse,
                                                  ms_per_step)
            result["cpu_baseline"] = base
            result["oracle_match"] = match
            result["prologue_oracle_match"] = pro_match

    if wl == "wan" and not args.no_configs and args.ring_streams == 1 and not args.fuse_q:
        wan = {"cfg": cfg, "q": q, "k": k, "v": v, "ws": ws, "q0": q0, "k0": k0, "to_dev": to_dev,
               "v_bits": x["v"], "q0_bits": x["q"], "k0_bits": x["k"]}
        del x
        result["configs"] = run_configs(args, dev, wan)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
