#!/usr/bin/env python3
"""Benchmark of the DiT long-sequence attention hot path on one MI355X.

Headline (the JSON line's value): attention forward with LSE on the FLUX.1 1024^2
sequence, B=1, N=4608 (4096 image + 512 text tokens), 24 heads of 128, bf16 inputs
with logits of standard deviation about 3, non-causal; one step = one attn_fwd_lse
call over the whole sequence; value = 4*N*N*H*D flops / step time, in TFLOP/s.

Legs timed in the same run and reported under "legs":
  wan5b       attention at N=27280 (Wan2.2-TI2V-5B video tokens), 24 x 128
  wan5b_cross Wan2.2 cross-attention: 27280 video queries x 512 text keys, 24 x 128
  flux_ring4  one GPU's FLUX Ring-4 share: Ulysses-4 permute of the Q shards, then
              Q[1152] x 4 KV chunks of 1152 through attn_fwd_lse (f32 partials), then the
              LSE merge; each kernel's time and rate; and the same share with the rounds
              folded in by attn_fwd_lse_accumulate (no partials, no merge)
  wan14b_u8   one GPU's Wan2.1-14B Ulysses-8 share: N=75600, 5 heads, 8 KV chunks of 9450
              + merge, and accumulated
  permute_wan14b  the Ulysses-8 permutes at Wan2.1-14B 720p: seq->head [8,1,9450,40,128] ->
              [8,1,75600,5,128], its inverse head->seq, and the fused QKV seq->head
              [8,1,9450,3,40,128] -> [8,3,1,75600,5,128], and that pass with QK-RMSNorm +
              RoPE fused in (qkv_norm_rope_permute)

Inputs are seeded synthetic tensors (no dataset, no weights) already resident in
HBM when a timed region starts.  Times come from HIP events recorded on the stream
the kernels are launched on.  "roofline" describes the headline kernel;
"cpu_baseline" times the fp64 CPU oracle over the whole headline workload on the host's
cores, with each workload's oracle wall time beside it (c4 and c5 extrapolated from one
head, or a block of its rows).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6    # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk/CU
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
PMC_SUMMARY = os.path.join(PROFILES, "attn_fwd_flux_N4608_H24_D128_pmc.txt")
_CSRC = os.path.join(ROOT, "diffusion_transformer_long_amd", "csrc")
_BUILD = os.path.join(ROOT, "diffusion_transformer_long_amd", "build.py")   # the compile flags
# the sources of each kernel family: a counter summary taken on other sources is stale
KERNEL_SRCS = {
    "attn_fwd": [os.path.join(_CSRC, f) for f in ("attn_fwd.hip", "common.h", "streamk.h", "tile_layout.h")] + [_BUILD],
    "merge": [os.path.join(_CSRC, f) for f in ("merge.hip", "common.h", "fastdiv.h")] + [_BUILD],
    "permute": [os.path.join(_CSRC, f) for f in ("permute.hip", "runmap.h", "common.h", "fastdiv.h")] + [_BUILD],
    "norm_rope": [os.path.join(_CSRC, f) for f in ("norm_rope.hip", "common.h", "fastdiv.h")] + [_BUILD],
}
ATTN_SRCS = KERNEL_SRCS["attn_fwd"]


def source_sha256(family="attn_fwd"):
    """Hash of one kernel family's sources and build flags."""
    h = hashlib.sha256()
    for f in KERNEL_SRCS[family]:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def attn_source_sha256():
    return source_sha256("attn_fwd")


def counter_records():
    """Per-kernel counter figures from the committed rocprofv3 summaries (lines 'json: {...}'
    in profiles/*_pmc.txt), keyed by (leg, entry); records taken on other kernel sources than
    the current ones are left out."""
    import glob
    out = {}
    shas = {f: source_sha256(f) for f in KERNEL_SRCS}
    for path in sorted(glob.glob(os.path.join(PROFILES, "*_pmc.txt"))):
        for line in open(path):
            if not line.startswith("json: "):
                continue
            rec = json.loads(line[6:])
            if shas.get(rec.get("family")) != rec.get("source_sha256"):
                continue
            key = (rec["leg"], rec["entry"])
            cur = out.setdefault(key, {"summary": "profiles/" + os.path.basename(path)})
            cur.update({k: v for k, v in rec.items() if k not in ("leg", "entry", "family", "source_sha256")})
    return out


def attach_counters(legs, recs):
    """Adds each leg's counter figures under legs[leg]["counters"][entry]."""
    for (leg, entry), rec in recs.items():
        if leg in legs:
            legs[leg].setdefault("counters", {})[entry] = rec


def err(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--legs", default="wan5b,wan5b_cross,flux_ring4,wan14b_u8,permute_wan14b",
                    help="comma list of extra legs (or 'none'); 'copy' adds a plain copy kernel "
                         "used to calibrate HBM counters")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-headline", action="store_true",
                    help="skip the headline workload (for profiling one leg at a time); the JSON "
                         "line then carries the legs only, with value null")
    ap.add_argument("--cpu-c5-rows", type=int, default=4096,
                    help="rows of one Wan2.1-14B share head the oracle times (extrapolated)")
    ap.add_argument("--print-source-hash", action="store_true",
                    help="print the attention kernel source hash and exit")
    return ap.parse_args()


class Timer:
    """HIP-event timing of work enqueued on one stream."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def time(self, fn, reps, warmup=0):
        torch = self.torch
        for _ in range(warmup):
            fn()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(self.stream)
        for _ in range(reps):
            fn()
        b.record(self.stream)
        b.synchronize()
        return a.elapsed_time(b) / reps  # ms per call

    def time_batches(self, fn, batches, per_batch, warmup=0):
        """(median, min) in ms per call over `batches` batches of `per_batch` back-to-back
        calls, each batch between one pair of events (a pair around every single call
        would add the events' own ~2 us to kernels of 10-15 us)."""
        t = sorted(self.time(fn, per_batch, warmup if i == 0 else 0) for i in range(batches))
        return t[len(t) // 2], t[0]


def pmc_traffic():
    """HBM bytes per launch of the headline kernel from the committed rocprofv3 counter
    summary, or None when the summary is missing or was taken on another kernel source."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    text = open(PMC_SUMMARY).read()
    sha = attn_source_sha256()
    m = re.search(r"^source_sha256:\s*(\w+)", text, re.M)
    t = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m or not t or m.group(1) != sha:
        return None
    return float(t.group(1))


def prewarm(torch, dev, seconds=1.0, step=None, step_seconds=0.5):
    """Untimed work that brings the GPU out of its idle clocks before anything is timed: bf16
    GEMMs, then (if given) the timed step's own kernel, so that the timed steps start at the
    clock the workload itself settles at.  Measured on one box: 20 FLUX steps right after 2 s
    idle took 304 us each, 200 steps 248 us, and 20 steps after this pre-warm 243 us.  Not
    part of any step."""
    a = torch.randn((8192, 8192), device=dev, dtype=torch.bfloat16)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            a = torch.matmul(a, a).clamp_(-1.0, 1.0)
        torch.cuda.synchronize()
    del a
    if step is not None:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < step_seconds:
            for _ in range(10):
                step()
            torch.cuda.synchronize()


def _oracle_timed(fn):
    t0 = time.perf_counter()
    fn()
    return time.perf_counter() - t0


def cpu_baseline(w, c5_rows):
    """The fp64 CPU oracle as it stands, timed on this host's cores: the whole headline
    workload (every query row against every key), and beside it each workload's oracle
    wall time (whole where it takes seconds; from one whole head, or a block of rows of
    one head, extrapolated by flops where the whole would take minutes)."""
    import numpy as np
    import oracle
    import synthetic
    q, k, v = synthetic.workload_qkv(w)
    dt = _oracle_timed(lambda: oracle.attn(q, k, v))
    per_config = {}
    per_config[w.name] = {"oracle_s": round(dt, 3), "rows": "all %d" % (w.B * w.H * w.Nq),
                          "tflops": round(w.flops / dt / 1e12, 5), "extrapolated": False}
    err("[bench] oracle %s: %.2f s (whole)" % (w.name, dt))
    tr = synthetic.TINY_RING
    tq, tk, tv = synthetic.workload_qkv(tr)
    t1 = _oracle_timed(lambda: oracle.attn(tq, tk, tv))
    per_config[tr.name] = {"oracle_s": round(t1, 4), "rows": "all %d" % (tr.B * tr.H * tr.Nq),
                           "tflops": round(tr.flops / t1 / 1e12, 5), "extrapolated": False}
    r4 = synthetic.FLUX_RING4
    q4 = q[:, r4.q_row0:r4.q_row0 + r4.Nq].contiguous()
    t3 = _oracle_timed(lambda: oracle.attn(q4, k, v))
    per_config[r4.name] = {"oracle_s": round(t3, 3), "rows": "all %d (rank 0's Q block)" % (r4.B * r4.H * r4.Nq),
                           "tflops": round(r4.flops / t3 / 1e12, 5), "extrapolated": False}
    del q, k, v, q4
    for wl, nrows in ((synthetic.WAN5B, None), (synthetic.WAN14B_U8, c5_rows)):
        a, b, c = synthetic.workload_qkv(wl)
        a, b, c = (t.double().numpy() for t in (a, b, c))
        n = wl.Nq if nrows is None else min(nrows, wl.Nq)
        rows = np.stack([np.zeros(n, np.int64), np.zeros(n, np.int64), np.arange(n, dtype=np.int64)], axis=1)
        t = _oracle_timed(lambda: oracle.attn_rows(a, b, c, rows))
        scale = (wl.B * wl.H * wl.Nq) / n
        per_config[wl.name] = {
            "oracle_s": round(t * scale, 1), "extrapolated": True,
            "measured": "%s of head 0 (each against all %d keys) in %.2f s, x%.1f by flops"
                        % ("all %d rows" % n if n == wl.Nq else "rows 0..%d" % (n - 1), wl.Nkv, t, scale),
            "tflops": round(wl.flops / scale / t / 1e12, 5)}
        err("[bench] oracle %s: %s" % (wl.name, per_config[wl.name]))
        del a, b, c
    return {"value": w.flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": "the whole %s workload: all %d query rows against all %d keys, fp64, %.2f s"
                      % (w.name, w.B * w.H * w.Nq, w.Nkv, dt),
            "cpu_model": _cpu_model(), "per_config": per_config}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.print_source_hash:
        print(attn_source_sha256())
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE=%d)." % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import diffusion_transformer_long_amd as dtl
    import synthetic

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    timer = Timer(torch, stream)
    legs_req = [] if args.legs == "none" else [x for x in args.legs.split(",") if x]

    # ---------------------------------------------------------------- headline
    w = synthetic.FLUX
    value = ms_per_step = roofline = None
    if not args.no_headline:
        err("[bench] headline %s: generating inputs" % w.name)
        q, k, v = (t.to(dev) for t in synthetic.workload_qkv(w))
        o = torch.empty((w.B, w.Nq, w.H, w.D), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)

        def step():
            dtl.attn_fwd_lse(q, k, v, o=o, lse=lse)

        prewarm(torch, dev, step=step)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(args.steps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_per_step = wall * 1e3 / args.steps
        kernel_ms = ev0.elapsed_time(ev1) / args.steps
        value = w.flops / (ms_per_step * 1e-3) / 1e12
        achieved = w.flops / (kernel_ms * 1e-3) / 1e12
        err("[bench] headline: %.3f ms/step (wall), %.3f ms/launch (events), %.1f TFLOP/s"
            % (ms_per_step, kernel_ms, achieved))

        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                    "traffic": pmc_traffic(),
                    "kernel": "attn_fwd_kernel<128,bf16> on %s" % w.name,
                    "flops_per_launch": w.flops,
                    "algorithmic_bytes_per_launch": 2 * (3 + 1) * w.B * w.Nq * w.H * w.D + 4 * w.B * w.H * w.Nq}
        del q, k, v, o, lse

    legs = {}

    # ---------------------------------------------------------------- wan5b
    if "wan5b" in legs_req:
        w5 = synthetic.WAN5B
        err("[bench] leg wan5b: generating inputs")
        q, k, v = (t.to(dev) for t in synthetic.workload_qkv(w5))
        o = torch.empty((w5.B, w5.Nq, w5.H, w5.D), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((w5.B, w5.H, w5.Nq), dtype=torch.float32, device=dev)
        ms = timer.time(lambda: dtl.attn_fwd_lse(q, k, v, o=o, lse=lse), reps=max(3, args.steps // 4),
                        warmup=2)
        tf = w5.flops / (ms * 1e-3) / 1e12
        med, mn = timer.time_batches(lambda: dtl.attn_fwd_lse(q, k, v, o=o, lse=lse), 5, 1)
        legs["wan5b"] = {"workload": w5.name, "attn_ms": round(ms, 4), "attn_tflops": round(tf, 2),
                         "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                         "attn_median_ms": round(med, 4), "attn_min_ms": round(mn, 4)}
        err("[bench] wan5b: %.3f ms, %.1f TFLOP/s" % (ms, tf))
        del q, k, v, o, lse

    # ---------------------------------------------------------------- wan5b cross-attention
    if "wan5b_cross" in legs_req:
        wc = synthetic.WAN5B_CROSS
        err("[bench] leg wan5b_cross: generating inputs")
        q, k, v = (t.to(dev) for t in synthetic.workload_qkv(wc))
        o = torch.empty((wc.B, wc.Nq, wc.H, wc.D), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((wc.B, wc.H, wc.Nq), dtype=torch.float32, device=dev)
        ms = timer.time(lambda: dtl.attn_fwd_lse(q, k, v, o=o, lse=lse), reps=20, warmup=3)
        med, mn = timer.time_batches(lambda: dtl.attn_fwd_lse(q, k, v, o=o, lse=lse), 7, 5)
        tf = wc.flops / (ms * 1e-3) / 1e12
        nbytes = 2 * wc.B * (2 * wc.Nq + 2 * wc.Nkv) * wc.H * wc.D + 4 * wc.B * wc.H * wc.Nq
        legs["wan5b_cross"] = {"workload": wc.name, "attn_ms": round(ms, 4), "attn_tflops": round(tf, 2),
                               "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                               "algorithmic_bytes": nbytes, "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                               "attn_median_ms": round(med, 4), "attn_min_ms": round(mn, 4)}
        err("[bench] wan5b_cross: %s" % legs["wan5b_cross"])
        del q, k, v, o, lse

    # ---------------------------------------------------------------- flux ring-4 share
    if "flux_ring4" in legs_req:
        w3 = synthetic.FLUX_RING4
        err("[bench] leg flux_ring4")
        qf, k, v = (t.to(dev) for t in synthetic.workload_qkv(synthetic.FLUX))
        shards = qf.reshape(1, 4, w3.Nq, w3.H, w3.D).transpose(0, 1).contiguous()
        q = qf[:, :w3.Nq].contiguous()
        C = w3.chunk_len
        # rotate buffer sets so each rep of the bandwidth kernels misses the 256 MB MALL
        nrot = 10
        perm_out = [torch.empty((4, 1, w3.Nkv, w3.H // 4, w3.D), dtype=torch.bfloat16, device=dev) for _ in range(nrot)]
        perm_in = [shards.clone() for _ in range(nrot)]
        parts = [torch.empty((w3.chunks, 1, w3.Nq, w3.H, w3.D), dtype=torch.float32, device=dev) for _ in range(nrot)]
        lparts = [torch.empty((w3.chunks, 1, w3.H, w3.Nq), dtype=torch.float32, device=dev) for _ in range(nrot)]
        o = torch.empty((1, w3.Nq, w3.H, w3.D), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((1, w3.H, w3.Nq), dtype=torch.float32, device=dev)
        for i in range(nrot):
            dtl.attn_fwd_lse_kv_chunks(q, k, v, w3.chunks, parts[i], lparts[i])
        ctr = [0]

        def rot():
            ctr[0] = (ctr[0] + 1) % nrot
            return ctr[0]

        reps = 3 * nrot
        ms_perm = timer.time(lambda: dtl.seq_to_head_permute(perm_in[rot()], 4, out=perm_out[ctr[0]]), reps, warmup=nrot)
        ms_chunk = timer.time(lambda: dtl.attn_fwd_lse(q, k[:, :C], v[:, :C], o=parts[0][0], lse=lparts[0][0]),
                              reps=20, warmup=3)
        ms_merge = timer.time(lambda: dtl.attn_merge_lse(parts[rot()], lparts[ctr[0]], o=o, lse=lse), reps, warmup=nrot)
        perm_med, perm_min = timer.time_batches(
            lambda: dtl.seq_to_head_permute(perm_in[rot()], 4, out=perm_out[ctr[0]]), 7, nrot, warmup=nrot)
        merge_med, merge_min = timer.time_batches(
            lambda: dtl.attn_merge_lse(parts[rot()], lparts[ctr[0]], o=o, lse=lse), 7, nrot, warmup=nrot)

        def share_step():   # ring_attention's default: here the one-launch partials (a round's
            # 216 tiles leave workgroup slots idle), then the merge
            dtl.seq_to_head_permute(perm_in[0], 4, out=perm_out[0])
            dtl.ring_attention(q, k, v, w3.chunks, o_parts=parts[0], lse_parts=lparts[0], o=o, lse=lse)
        ms_step = timer.time(share_step, reps=10, warmup=2)

        def share_step_rounds():   # one attn_fwd_lse call per round, then the merge
            dtl.seq_to_head_permute(perm_in[0], 4, out=perm_out[0])
            dtl.ring_attention(q, k, v, w3.chunks, o_parts=parts[0], lse_parts=lparts[0], o=o, lse=lse,
                               one_launch=False)
        ms_step_rounds = timer.time(share_step_rounds, reps=10, warmup=2)

        def share_step_one():   # the partials of all rounds from one launch, then the merge
            dtl.seq_to_head_permute(perm_in[0], 4, out=perm_out[0])
            dtl.ring_attention(q, k, v, w3.chunks, o_parts=parts[0], lse_parts=lparts[0], o=o, lse=lse,
                               one_launch=True)
        ms_step_one = timer.time(share_step_one, reps=10, warmup=2)
        ms_chunks_one = timer.time(lambda: dtl.attn_fwd_lse_kv_chunks(q, k, v, w3.chunks, parts[0], lparts[0]),
                                   reps=20, warmup=3)
        o_acc = parts[1][0]

        def share_step_acc():
            dtl.seq_to_head_permute(perm_in[0], 4, out=perm_out[0])
            dtl.ring_attention(q, k, v, w3.chunks, accumulate=True, o_acc=o_acc, o=o, lse=lse)
        ms_step_acc = timer.time(share_step_acc, reps=10, warmup=2)
        # the default step captured once in a HIP graph and replayed (launch overhead only
        # differs; tests/test_gpu_graph.py checks that replays equal the eager step)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            share_step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            share_step()
        torch.cuda.synchronize()
        ms_step_graph = timer.time(lambda: graph.replay(), reps=10, warmup=2)
        del graph
        ms_acc = timer.time(lambda: dtl.attn_fwd_lse_accumulate(q, k[:, C:2 * C], v[:, C:2 * C], o_acc, lse),
                            reps=20, warmup=3)
        perm_bytes = 2 * shards.numel() * 2
        merge_bytes = (w3.chunks * w3.Nq * w3.H * (w3.D + 1) * 4) + w3.Nq * w3.H * (w3.D * 2 + 4)
        chunk_flops = 4.0 * w3.Nq * C * w3.H * w3.D
        legs["flux_ring4"] = {
            "workload": w3.name, "step_ms": round(ms_step, 4),
            "step_tflops": round(w3.flops / (ms_step * 1e-3) / 1e12, 2),
            "step_accumulate_ms": round(ms_step_acc, 4),
            "step_accumulate_tflops": round(w3.flops / (ms_step_acc * 1e-3) / 1e12, 2),
            "step_graph_ms": round(ms_step_graph, 4),
            "step_one_launch_ms": round(ms_step_one, 4),
            "step_one_launch_tflops": round(w3.flops / (ms_step_one * 1e-3) / 1e12, 2),
            "step_per_round_ms": round(ms_step_rounds, 4),
            "step_per_round_tflops": round(w3.flops / (ms_step_rounds * 1e-3) / 1e12, 2),
            "all_chunks_one_launch_ms": round(ms_chunks_one, 4),
            "all_chunks_one_launch_tflops": round(w3.flops / (ms_chunks_one * 1e-3) / 1e12, 2),
            "accumulate_chunk_ms": round(ms_acc, 4),
            "permute_ms": round(ms_perm, 4), "permute_gbs": round(perm_bytes / (ms_perm * 1e-3) / 1e9, 1),
            "permute_bytes": perm_bytes,
            "chunk_attn_ms": round(ms_chunk, 4), "chunk_attn_tflops": round(chunk_flops / (ms_chunk * 1e-3) / 1e12, 2),
            "merge_ms": round(ms_merge, 4), "merge_gbs": round(merge_bytes / (ms_merge * 1e-3) / 1e9, 1),
            "merge_bytes": merge_bytes, "rotation_buffers": nrot,
            "permute_median_ms": round(perm_med, 4), "permute_min_ms": round(perm_min, 4),
            "merge_median_ms": round(merge_med, 4), "merge_min_ms": round(merge_min, 4)}
        err("[bench] flux_ring4: %s" % legs["flux_ring4"])
        del qf, k, v, shards, q, perm_out, perm_in, parts, lparts, o, lse

    # ---------------------------------------------------------------- wan14b u8 share
    if "wan14b_u8" in legs_req:
        w5 = synthetic.WAN14B_U8
        err("[bench] leg wan14b_u8: generating inputs")
        q, k, v = (t.to(dev) for t in synthetic.workload_qkv(w5))
        C = w5.chunk_len
        parts = torch.empty((w5.chunks, 1, w5.Nq, w5.H, w5.D), dtype=torch.float32, device=dev)
        lparts = torch.empty((w5.chunks, 1, w5.H, w5.Nq), dtype=torch.float32, device=dev)
        o = torch.empty((1, w5.Nq, w5.H, w5.D), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((1, w5.H, w5.Nq), dtype=torch.float32, device=dev)
        dtl.attn_fwd_lse_kv_chunks(q, k, v, w5.chunks, parts, lparts)
        ms_chunk = timer.time(lambda: dtl.attn_fwd_lse(q, k[:, :C], v[:, :C], o=parts[0], lse=lparts[0]),
                              reps=4, warmup=1)
        ms_merge = timer.time(lambda: dtl.attn_merge_lse(parts, lparts, o=o, lse=lse), reps=10, warmup=2)
        merge_med, merge_min = timer.time_batches(lambda: dtl.attn_merge_lse(parts, lparts, o=o, lse=lse), 5, 2)
        ms_step = timer.time(lambda: dtl.ring_attention(q, k, v, w5.chunks, o_parts=parts, lse_parts=lparts,
                                                         o=o, lse=lse), reps=2, warmup=1)
        o_acc = parts[0]
        ms_step_acc = timer.time(lambda: dtl.ring_attention(q, k, v, w5.chunks, accumulate=True, o_acc=o_acc,
                                                             o=o, lse=lse), reps=2, warmup=1)
        ms_acc = timer.time(lambda: dtl.attn_fwd_lse_accumulate(q, k[:, C:2 * C], v[:, C:2 * C], o_acc, lse),
                            reps=4, warmup=1)
        merge_bytes = (w5.chunks * w5.Nq * w5.H * (w5.D + 1) * 4) + w5.Nq * w5.H * (w5.D * 2 + 4)
        chunk_flops = 4.0 * w5.Nq * C * w5.H * w5.D
        legs["wan14b_u8"] = {
            "workload": w5.name, "step_ms": round(ms_step, 3),
            "step_tflops": round(w5.flops / (ms_step * 1e-3) / 1e12, 2),
            "step_accumulate_ms": round(ms_step_acc, 3),
            "step_accumulate_tflops": round(w5.flops / (ms_step_acc * 1e-3) / 1e12, 2),
            "accumulate_chunk_ms": round(ms_acc, 4),
            "chunk_attn_ms": round(ms_chunk, 4), "chunk_attn_tflops": round(chunk_flops / (ms_chunk * 1e-3) / 1e12, 2),
            "merge_ms": round(ms_merge, 4), "merge_gbs": round(merge_bytes / (ms_merge * 1e-3) / 1e9, 1),
            "merge_bytes": merge_bytes, "merge_frac_of_hbm": round(merge_bytes / (ms_merge * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "merge_median_ms": round(merge_med, 4), "merge_min_ms": round(merge_min, 4)}
        err("[bench] wan14b_u8: %s" % legs["wan14b_u8"])
        del q, k, v, parts, lparts, o, lse

    # ---------------------------------------------------------------- permutes at Wan-14B U8
    if "permute_wan14b" in legs_req:
        p, Ns, H, D = 8, 9450, 40, 128
        err("[bench] leg permute_wan14b")
        res = {}

        def one(name, fn, x, out, shape):
            ms = timer.time(lambda: fn(x, p, out=out), reps=10, warmup=2)
            med, mn = timer.time_batches(lambda: fn(x, p, out=out), 5, 2)
            nbytes = 2 * x.numel() * x.element_size()
            res[name] = {"shape": shape, "ms": round(ms, 4), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                         "bytes": nbytes, "frac_of_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         "median_ms": round(med, 4), "min_ms": round(mn, 4)}
            err("[bench]   %s: %s" % (name, res[name]))

        x = torch.empty((p, 1, Ns, H, D), dtype=torch.bfloat16, device=dev).normal_()
        y = torch.empty((p, 1, Ns * p, H // p, D), dtype=torch.bfloat16, device=dev)
        one("seq_to_head", dtl.seq_to_head_permute, x, y, "[8,1,9450,40,128]->[8,1,75600,5,128] bf16")
        one("head_to_seq", dtl.head_to_seq_permute, y, x, "[8,1,75600,5,128]->[8,1,9450,40,128] bf16")
        del x, y
        x = torch.empty((p, 1, Ns, 3, H, D), dtype=torch.bfloat16, device=dev).normal_()
        y = torch.empty((p, 3, 1, Ns * p, H // p, D), dtype=torch.bfloat16, device=dev)
        one("qkv_seq_to_head", dtl.qkv_seq_to_head_permute, x, y, "[8,1,9450,3,40,128]->[8,3,1,75600,5,128] bf16")
        # the same pass with QK-RMSNorm and rotary embedding fused in (tables: seeded angles)
        g = torch.Generator(device="cpu").manual_seed(9)
        gq = (0.5 + torch.rand(H * D, generator=g)).to(dev)
        gk = (0.5 + torch.rand(H * D, generator=g)).to(dev)
        ang = (torch.rand((Ns * p, D // 2), generator=g) * 12.0 - 6.0).to(dev)
        cs, sn = torch.cos(ang), torch.sin(ang)
        one("qkv_norm_rope", lambda a, p_, out: dtl.qkv_norm_rope_permute(a, gq, gk, cs, sn, p_, out=out),
            x, y, "[8,1,9450,3,40,128]->[8,3,1,75600,5,128] bf16, QK-RMSNorm + RoPE fused")
        del x, y, gq, gk, ang, cs, sn
        legs["permute_wan14b"] = res

    # ---------------------------------------------------------------- copy (counter calibration)
    if "copy" in legs_req:
        nb = 1 << 30
        a = torch.empty(nb // 4, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        ms = timer.time(lambda: b.copy_(a), reps=5, warmup=2)
        legs["copy"] = {"bytes_read": nb, "bytes_written": nb, "ms": round(ms, 4),
                        "gbs": round(2 * nb / (ms * 1e-3) / 1e9, 1)}
        del a, b

    cpu = None
    if not args.no_cpu_baseline and not args.no_headline:
        err("[bench] cpu baseline (oracle on host cores)")
        cpu = cpu_baseline(w, args.cpu_c5_rows)
        err("[bench] cpu baseline: %s" % cpu)

    recs = counter_records()
    attach_counters(legs, recs)
    if roofline is not None and ("headline", "attn") in recs:
        roofline["counters"] = recs[("headline", "attn")]

    line = {
        "metric": "attention TFLOP/s + % bf16 MFMA peak at N=4608 and N=27280, 1 GPU",
        "value": None if value is None else round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": None if ms_per_step is None else round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "seq_len": w.Nq, "heads": w.H, "head_dim": w.D,
                   "k_scale": w.k_scale, "causal": False, "o_dtype": "bf16", "lse_dtype": "f32",
                   "parallelism": "none (one GPU's full sequence)"},
        "frac_of_peak": None if value is None else round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "legs": legs,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
