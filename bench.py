"""Benchmark of the hot path on one MI355X.

The timed step is the DECODE step of the Qwen-3-8B-like single layer (B=16, H=4096,
32 Q / 8 KV heads, d=128, bf16 KV in 16-token pages, MLP scorer 4096->512->8) on a
context of 32767 prompt positions compressed to ~25% (tau at the 75th percentile of
the prompt's scores, computed on the device; the most recent 128 positions kept): one
kvp_decode_step call, which scores the 16 new tokens with the MLP (its split-K first layer,
then the rest inside the step), applies the delayed step and runs GQA attention over the
kept entries only.  The same steps as separate calls (kvp_score_step_delayed, then
kvp_decode_attn) are timed beside it.
The prompt is compressed once before timing (kvp_score -> kvp_threshold -> kvp_select ->
kvp_compact); those calls are timed one by one in the "prefill" record.  Every input is
resident in HBM before the timed region; the decode positions T-1, T, ... are appended
on the device, step after step.

    value        kept token-heads attended per second of decode-step time: the token-heads
                 each timed step's attention reads, summed over the K timed steps, over
                 their total time (one HIP event pair on the launch stream around the K
                 steps, queued back to back)
    ms_per_step  that time / K
    roofline     decode attention (its stream kernel + merge kernel): algorithmic bytes per
                 call / mean call duration, from K calls back to back on the cache the timed
                 steps left, one HIP event pair around them on the launch stream (an event
                 recorded between two kernels idles the GPU for microseconds, so no event
                 sits inside a timed loop)

Records of the same run, each on its own seeded synthetic inputs:
    prefill         the compression calls of the headline workload, one by one
    keep_scaling    decode step and cache-flushed attention at keep 1.0 / 0.5 / 0.25
    dms_delayed     8192-token prompt + 1024 delayed-eviction decode steps, eager and graph
    long_70b_layer  decode steps at keep 0.5 / 0.25 (and 1.0) on the 70B-like layer
    beacon_mixed    decode steps over the bf16 + int8 pools, and the demoting compaction
    beacon_int4     the same with the demoted tokens as int4 codes
    beacon_fp8      the same with the demoted tokens as fp8 E4M3 codes
    copy_ceiling    a plain 1 GiB device copy and a 1 GiB read (torch kernels)

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME[,NAME...]] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
METRIC = "kept-KV decode attention tokens/s + achieved HBM GB/s (% of peak), 1 GPU"
RECORDS = ("headline", "prefill", "keep_scaling", "dms_delayed", "long_70b_layer",
           "beacon_mixed", "beacon_int4", "beacon_fp8", "copy_ceiling")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def pmc_traffic(key):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs
    (scaled by the plain-copy calibration), or None once any source file of the kernel
    differs from the one that was profiled."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    try:
        rec = json.load(open(path))[key]
        h = hashlib.sha256()
        for f in rec["sources"]:  # every source file the kernel is built from
            h.update(open(os.path.join(ROOT, f), "rb").read())
    except (OSError, KeyError, ValueError):
        return None
    if h.hexdigest()[:16] != rec["source_sha256_16"]:
        return None
    return rec["hbm_bytes_per_launch"]


def dtype_name(dt) -> str:
    import torch
    return {torch.bfloat16: "bf16", torch.float32: "f32"}[dt]


def new_event():
    import torch
    return torch.cuda.Event(enable_timing=True)


def gbs(nbytes, ms):
    return nbytes / (ms * 1e-3) / 1e9


def code_bytes(lp_bits) -> float:
    """Bytes per low-precision code: int4 two per byte, int8 and fp8 one."""
    return 0.5 if lp_bits == 4 else 1.0


# ------------------------------------------------------------------------------ inputs

class Context:
    """Seeded synthetic inputs of one workload (a prompt of T - 1 positions plus the
    decode token's draws) and a pruned cache sized for the prompt and `extra` decode
    steps."""

    def __init__(self, wl, dev, extra: int = 64):
        import torch

        import kvp_workloads as W
        import sparse_decode_attention_kvzap_amd as K
        from sparse_decode_attention_kvzap_amd.pipeline import PrunedKVCache

        self.wl, self.K, self.W = wl, K, W
        self.T0 = wl.T - 1
        t0 = time.perf_counter()
        self.hidden = W.hidden_states(wl, self.T0, dev)
        self.kd, self.vd = W.kv_dense(wl, self.T0, dev)
        self.sw = W.scorer_weights(wl, dev)
        self.h_new, self.k_new, self.v_new, self.q = W.step_inputs(wl, 0, dev)
        if wl.scorer == "mlp":
            self.scorer = K.Scorer(K.KVP_SCORER_MLP, self.sw.W1, self.sw.b1, self.sw.W2, self.sw.b2)
        else:
            self.scorer = K.Scorer(K.KVP_SCORER_LINEAR, self.sw.W1, self.sw.b1)
        self.cache = PrunedKVCache(wl.B, wl.Hkv, wl.Hq, wl.d, wl.T + extra, wl.kv_dtype,
                                   self.scorer, wl.R, 0.0, device=dev, max_prompt=self.T0,
                                   demote=wl.int8_demote, lp_bits=wl.lp_bits)
        torch.cuda.synchronize()
        log(f"[bench] {wl.name}: inputs generated in {time.perf_counter() - t0:.1f}s")

    def compress(self, q_keep, stream):
        """Score the prompt, set tau (the q_keep quantile on the device; -inf keeps all),
        select, compact, and point the next decode position at T - 1."""
        c = self.cache
        c.score(self.hidden, stream=stream)
        if q_keep is None:
            c.set_tau(float("-inf"), stream)
            c.tau = c.tau_dev
        else:
            c.calibrate(q_keep, self.T0, stream)
        c.select(self.T0, stream)
        c.compact(self.kd, self.vd, stream)
        c.set_position(self.T0, stream)

    def advance(self, stream):
        self.cache.advance(self.h_new, self.k_new, self.v_new, stream=stream)

    def step(self, stream):
        """One decode step: kvp_decode_step (the delayed step folded into the attention)
        for a bf16 cache without a low-precision pool, else the separate calls."""
        self.cache.step(self.h_new, self.k_new, self.v_new, self.q, stream=stream)

    def attend(self, stream):
        self.cache.attend(self.q, stream)

    def read_split(self):
        """(full-precision token-heads, low-precision token-heads) the next attention
        reads: pool + non-empty ring slots, and the low-precision pool."""
        c = self.cache
        main = int(c.kv.length.sum()) + int((c.ring.pos >= 0).sum())
        lp = int(c.kv.length8.sum()) if self.wl.int8_demote else 0
        return main, lp

    def attn_bytes(self, main, lp) -> float:
        """Algorithmic bytes of one decode attention: K and V of every full-precision
        token-head, codes plus two fp32 scales of every low-precision one, one block-table
        entry per 16 tokens, the queries read and the fp32 outputs written."""
        wl = self.wl
        elt = 2 if dtype_name(wl.kv_dtype) == "bf16" else 4
        return (main * 2 * wl.d * elt + lp * 2 * (wl.d * code_bytes(wl.lp_bits) + 4)
                + (main + lp) / 16 * 4 + wl.B * wl.Hq * wl.d * (elt + 4))


# ------------------------------------------------------------------------------ decode

def decode_run(ctx, q_keep, steps, warmup, stream, graph=False):
    """Compress, then `warmup` + `steps` decode steps back to back, timed by one pair of
    events around the `steps` (an event recorded between kernels costs the GPU several
    microseconds of idle time, so none sits inside the timed steps).  The token-heads each
    step's attention reads come from an identical untimed pass (same inputs, same device
    state sequence).  The decode attention alone is then timed the same way: `steps` calls
    back to back on the cache the steps left."""
    import numpy as np
    import torch

    n = warmup + steps
    ctx.compress(q_keep, stream)
    split = []
    for _ in range(n):
        ctx.advance(stream)
        stream.synchronize()
        split.append(ctx.read_split())
    tau = float(ctx.cache.tau_dev.item())

    def timed_steps(fused):
        ctx.compress(q_keep, stream)
        for _ in range(warmup):
            if fused:
                ctx.step(stream)
            else:
                ctx.advance(stream)
                ctx.attend(stream)
        start, end = new_event(), new_event()
        stream.synchronize()
        start.record(stream)
        for _ in range(steps):
            if fused:
                ctx.step(stream)
            else:
                ctx.advance(stream)
                ctx.attend(stream)
        end.record(stream)
        torch.cuda.synchronize()
        assert ctx.cache.check(stream) == 0, "pool overflow"
        return start.elapsed_time(end)

    # the same steps as separate calls (delayed step, then attention), then as the fused
    # call, which the headline times
    separate_ms = timed_steps(False)
    total_ms = timed_steps(True)
    # the attention alone, back to back on the cache as the last step left it
    last = ctx.read_split()
    for _ in range(2):
        ctx.attend(stream)
    e0, e1 = new_event(), new_event()
    e0.record(stream)
    for _ in range(steps):
        ctx.attend(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    attn_ms = e0.elapsed_time(e1) / steps
    nbytes = ctx.attn_bytes(*last)
    timed = split[warmup:]
    th = [m + lp for m, lp in timed]
    r = {
        "keep_quantile": q_keep, "tau": tau,
        "token_heads_per_step": float(np.mean(th)),
        "low_precision_token_heads_per_step": float(np.mean([lp for _, lp in timed])),
        "total_token_heads": ctx.wl.B * ctx.wl.Hkv * ctx.wl.T,
        "ms_per_step": total_ms / steps,
        "separate_calls_ms_per_step": separate_ms / steps,
        "fused_step": bool(ctx.cache.fused_step),
        "token_heads_per_s": float(np.sum(th)) / (total_ms * 1e-3),
        "attn": {"ms": attn_ms, "launches": steps, "bytes_per_call": nbytes,
                 "token_heads": sum(last), "gbs": gbs(nbytes, attn_ms),
                 "frac_of_peak": gbs(nbytes, attn_ms) / PEAK_HBM_GBS,
                 "token_heads_per_s": sum(last) / (attn_ms * 1e-3),
                 "timing": "calls back to back on the cache after the timed steps, one "
                           "event pair around them"},
    }
    if graph:
        # the same decode step captured once and replayed: every per-step value lives in
        # device memory, so a replay needs no host work
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            ctx.step(side)
        torch.cuda.synchronize()
        ctx.compress(q_keep, stream)
        with torch.cuda.stream(stream):
            for _ in range(warmup):
                g.replay()
            e0, e1 = new_event(), new_event()
            e0.record(stream)
            for _ in range(steps):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        assert ctx.cache.check(stream) == 0, "pool overflow"
        r["graph_ms_per_step"] = e0.elapsed_time(e1) / steps
        del g
        # eight consecutive decode steps captured as one graph: the GPU's idle time before
        # each replay (the same for any graph here) is paid once per eight steps
        G = 8
        reps = max(1, min(steps, 48) // G)
        g8 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g8, stream=side):
            for _ in range(G):
                ctx.step(side)
        torch.cuda.synchronize()
        ctx.compress(q_keep, stream)
        with torch.cuda.stream(stream):
            g8.replay()
            e0, e1 = new_event(), new_event()
            e0.record(stream)
            for _ in range(reps):
                g8.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        assert ctx.cache.check(stream) == 0, "pool overflow"
        r["graph8_ms_per_step"] = e0.elapsed_time(e1) / (reps * G)
        del g8
    return r


def flushed_attn_ms(ctx, stream, reps=8, stats=False):
    """Median decode-attention time on the cache as it stands, each call right after a
    1 GiB READ that evicts the 256 MB MALL (a write flush would leave dirty lines draining
    into the timed call); the flush and the call are queued back to back.  With stats:
    {"median_ms", "min_ms", "reps"}."""
    import numpy as np
    import torch

    flush = torch.ones(1 << 28, dtype=torch.int32, device=stream.device)
    acc = torch.zeros(1, dtype=torch.int64, device=stream.device)
    out = []
    with torch.cuda.stream(stream):
        for r in range(reps + 2):
            acc.add_(flush.sum())
            e0, e1 = new_event(), new_event()
            e0.record(stream)
            ctx.attend(stream)
            e1.record(stream)
            torch.cuda.synchronize()
            if r >= 2:
                out.append(e0.elapsed_time(e1))
    if stats:
        return {"median_ms": float(np.median(out)), "min_ms": float(np.min(out)), "reps": reps}
    return float(np.median(out))


# ------------------------------------------------------------------------------ records

def record_prefill(ctx, stream, reps=5):
    """The compression calls of one workload, each timed with events (median of reps),
    then the prefill attention under the same selection.  Before each repetition a 1 GiB
    READ (outside the timed calls) lets the previous repetition's compaction writes drain
    and evicts the 256 MB MALL, so the scorer does not start inside that write-back."""
    import numpy as np
    import torch

    wl, c = ctx.wl, ctx.cache
    names = ["score", "threshold", "select", "compact"]
    times = {n: [] for n in names}
    q_keep = wl.keep_quantiles[0]
    flush = torch.ones(1 << 28, dtype=torch.int32, device=stream.device)
    acc = torch.zeros(1, dtype=torch.int64, device=stream.device)
    for r in range(reps + 1):
        with torch.cuda.stream(stream):
            acc.add_(flush.sum())
        ev = [new_event() for _ in range(5)]
        ev[0].record(stream)
        c.score(ctx.hidden, stream=stream)
        ev[1].record(stream)
        c.calibrate(q_keep, ctx.T0, stream)
        ev[2].record(stream)
        c.select(ctx.T0, stream)
        ev[3].record(stream)
        c.compact(ctx.kd, ctx.vd, stream)
        ev[4].record(stream)
        torch.cuda.synchronize()
        if r >= 1:
            for i, n in enumerate(names):
                times[n].append(ev[i].elapsed_time(ev[i + 1]))
    del flush, acc
    ms = {n: float(np.median(v)) for n, v in times.items()}
    kept = int(c.kept_count.sum())
    B, Hkv, d, H, T0 = wl.B, wl.Hkv, wl.d, wl.H, ctx.T0
    elt = 2 if dtype_name(wl.kv_dtype) == "bf16" else 4
    ntok = B * T0
    if wl.scorer == "mlp":
        flops = 2.0 * ntok * H * wl.inner + 2.0 * ntok * wl.inner * Hkv
    else:
        flops = 2.0 * ntok * H * Hkv
    score_bytes = ntok * H * elt + ntok * Hkv * 4
    select_bytes = ntok * Hkv * 4 + B * Hkv * T0 * 4 + B * Hkv * ((T0 + 31) // 32) * 4
    compact_bytes = kept * 2 * d * elt * 2 + kept * 4
    if wl.int8_demote:  # demoted tokens: read in full, written as codes + one scale per row
        demoted = B * Hkv * T0 - kept
        compact_bytes += demoted * (2 * d * elt + 2 * (d * code_bytes(wl.lp_bits) + 4) + 4)
    tflops = flops / (ms["score"] * 1e-3) / 1e12
    tk = ("compact_quant" if wl.lp_bits == 8 else None) if wl.int8_demote else "compact_copy"
    out = {
        "workload": wl.name, "kept_token_heads": kept,
        "score": {"ms": ms["score"], "kind": wl.scorer, "flop": flops, "tflops": tflops,
                  "frac_of_bf16_peak": tflops / PEAK_BF16_TFLOPS if wl.scorer == "mlp" else None,
                  "gbs": gbs(score_bytes, ms["score"]),
                  "traffic": pmc_traffic("score_mlp_bf16") if wl.scorer == "mlp" else None},
        "threshold": {"ms": ms["threshold"], "note": "exact radix select on the device"},
        "select": {"ms": ms["select"], "gbs": gbs(select_bytes, ms["select"])},
        "compact": {"ms": ms["compact"], "bytes": compact_bytes,
                    "gbs": gbs(compact_bytes, ms["compact"]),
                    "frac_of_peak": gbs(compact_bytes, ms["compact"]) / PEAK_HBM_GBS,
                    # counters were taken for the copy kernel, and for the int8 quantizing kernel
                    "traffic": pmc_traffic(tk) if tk else None, "traffic_kernel": tk},
    }
    if not wl.int8_demote and dtype_name(wl.kv_dtype) == "bf16":
        out["prefill_attn"] = measure_prefill_attn(ctx, stream)
    return out


def measure_prefill_attn(ctx, stream, reps=3) -> dict:
    """kvp_prefill_attn over the prompt under the current selection: every prompt
    position attends to the kept keys before it plus the last `window` positions.
    Useful work = 4 d flop per (query row, visible key) pair (QK^T and PV)."""
    import torch

    wl, c, T0 = ctx.wl, ctx.cache, ctx.T0
    dev = stream.device
    c.select(T0, stream)
    qp = ctx.W.prompt_queries(wl, T0, dev)
    out = torch.empty((wl.B, wl.Hq, T0, wl.d), dtype=torch.float32, device=dev)
    R = c.window
    keep = (c.scores[:, :, :T0] >= c.tau_dev).reshape(c.P, T0)
    ck = torch.cumsum(keep.to(torch.int32), dim=1)
    i = torch.arange(T0, device=dev)
    before = torch.where(i >= R, ck[:, (i - R).clamp(min=0)], torch.zeros_like(ck))
    vis = before.double().sum().item() + c.P * float(torch.clamp(i + 1, max=R).double().sum())
    pairs = vis * wl.g
    flops = pairs * 4 * wl.d
    causal = c.P * wl.g * T0 * (T0 + 1) / 2
    c.prefill_attention(qp, ctx.kd, ctx.vd, out, stream)
    e0, e1 = new_event(), new_event()
    e0.record(stream)
    for _ in range(reps):
        c.prefill_attention(qp, ctx.kd, ctx.vd, out, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del qp, out, keep, ck
    torch.cuda.empty_cache()
    tflops = flops / (ms * 1e-3) / 1e12
    return {"ms": ms, "tflops": tflops, "frac_of_bf16_peak": tflops / PEAK_BF16_TFLOPS,
            "traffic": pmc_traffic("prefill_attn"), "useful_flop": flops,
            "visible_pairs": pairs, "visible_fraction": pairs / causal,
            "note": "q/k/v bf16, out fp32; useful = 4 d flop per visible (row, key) pair"}


def record_keep_scaling(ctx, stream, keeps=(1.0, 0.5, 0.25)):
    """Decode step back to back and cache-flushed attention after compressing the same
    prompt at several keep ratios (keep 1.0: tau = -inf)."""
    rows = []
    for keep in keeps:
        r = decode_run(ctx, None if keep >= 1.0 else 1.0 - keep, 8, 3, stream)
        iso = flushed_attn_ms(ctx, stream)
        rows.append({"keep": keep, "tau": r["tau"], "token_heads_per_step": r["token_heads_per_step"],
                     "attn_bytes": r["attn"]["bytes_per_call"],
                     "decode_step_ms": r["ms_per_step"], "attn_ms": r["attn"]["ms"],
                     "attn_flushed_ms": iso,
                     "attn_flushed_gbs": gbs(r["attn"]["bytes_per_call"], iso)})
    base = rows[0]
    for e in rows:
        e["bytes_ratio_vs_keep1"] = e["attn_bytes"] / base["attn_bytes"]
        e["decode_step_ratio_vs_keep1"] = e["decode_step_ms"] / base["decode_step_ms"]
        e["attn_flushed_ratio_vs_keep1"] = e["attn_flushed_ms"] / base["attn_flushed_ms"]
    log("[bench] keep scaling " + ctx.wl.name + ": " + "; ".join(
        f"keep {e['keep']}: step {e['decode_step_ms'] * 1e3:.1f} us "
        f"(x{e['decode_step_ratio_vs_keep1']:.2f}), flushed attn {e['attn_flushed_ms'] * 1e3:.1f} us "
        f"(x{e['attn_flushed_ratio_vs_keep1']:.2f}), bytes x{e['bytes_ratio_vs_keep1']:.2f}"
        for e in rows))
    return {"workload": ctx.wl.name, "rows": rows}


def record_long(dev, stream, steps, warmup):
    """70B-like layer: decode steps at keep 0.5 and 0.25, and at keep 1.0 for the
    scaling check."""
    import kvp_workloads as W
    wl = W.BY_NAME["long_70b_layer"]
    ctx = Context(wl, dev, extra=warmup + steps + 16)
    out = {"workload": wl.name, "batch": wl.B, "context": wl.T, "q_heads": wl.Hq,
           "kv_heads": wl.Hkv, "scorer": wl.scorer, "dtype": dtype_name(wl.kv_dtype)}
    for q_keep in list(wl.keep_quantiles) + [None]:
        keep = 1.0 if q_keep is None else round(1.0 - q_keep, 3)
        r = decode_run(ctx, q_keep, steps, warmup, stream)
        r["attn_flushed_ms"] = flushed_attn_ms(ctx, stream)
        out[f"keep_{keep}"] = r
        log(f"[bench] {wl.name} keep {keep}: step {r['ms_per_step'] * 1e3:.1f} us, attention "
            f"{r['attn']['ms'] * 1e3:.1f} us = {r['attn']['gbs']:.0f} GB/s "
            f"({100 * r['attn']['frac_of_peak']:.1f}% of peak)")
    del ctx
    return out


def record_beacon(dev, stream, steps, warmup, name="beacon_mixed"):
    """Beacon-style mixed precision: decode steps over the bf16 and low-precision pools
    (int8 codes; int4 for beacon_int4, fp8 E4M3 for beacon_fp8), and the demoting
    compaction."""
    import torch

    import kvp_workloads as W
    wl = W.BY_NAME[name]
    ctx = Context(wl, dev, extra=warmup + steps + 16)
    r = decode_run(ctx, wl.keep_quantiles[0], steps, warmup, stream)
    r["attn_flushed_ms"] = flushed_attn_ms(ctx, stream)
    pre = record_prefill(ctx, stream, reps=3)
    out = {"workload": wl.name, "lp_bits": wl.lp_bits, "dtype": dtype_name(wl.kv_dtype),
           "decode": r, "compact_demote": pre["compact"], "score": pre["score"]}
    log(f"[bench] {wl.name}: step {r['ms_per_step'] * 1e3:.1f} us, attention "
        f"{r['attn']['ms'] * 1e3:.1f} us = {r['attn']['gbs']:.0f} GB/s; demoting compaction "
        f"{pre['compact']['ms']:.3f} ms = {pre['compact']['gbs']:.0f} GB/s")
    del ctx
    torch.cuda.empty_cache()
    return out


def record_copy_ceiling(dev, stream):
    """What plain torch kernels reach on this GPU: a 1 GiB device-to-device copy
    (read + write bytes) and a 1 GiB read (fp32 sum reduction)."""
    import numpy as np
    import torch

    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    acc = torch.zeros(1, dtype=torch.float32, device=dev)
    cp, rd = [], []
    with torch.cuda.stream(stream):
        for r in range(8):
            e0, e1, e2 = new_event(), new_event(), new_event()
            e0.record(stream)
            dst.copy_(src)
            e1.record(stream)
            acc.add_(src.sum())
            e2.record(stream)
            torch.cuda.synchronize()
            if r >= 2:
                cp.append(e0.elapsed_time(e1))
                rd.append(e1.elapsed_time(e2))
    nb = src.numel() * 4
    copy_gbs = gbs(2 * nb, float(np.median(cp)))
    read_gbs = gbs(nb, float(np.median(rd)))
    del src, dst
    torch.cuda.empty_cache()
    return {"copy_gbs": copy_gbs, "read_gbs": read_gbs,
            "copy_frac_of_peak": copy_gbs / PEAK_HBM_GBS, "read_frac_of_peak": read_gbs / PEAK_HBM_GBS,
            "note": "torch copy_ of 1 GiB (2 GiB moved) and torch sum over 1 GiB, medians of 6; "
                    "the sum is torch's reduction kernel, which does not reach the read "
                    "bandwidth, so only the copy serves as a ceiling"}


def dms_loop(dev, stream):
    """The delayed-eviction decode loop: compress the prompt (tau = 0, recent window w),
    then wl.steps decode steps (score the new token -> delayed step -> attention),
    eagerly and as one captured HIP graph replayed per step.  Eager steps take each
    step's inputs where they lie (views of the pre-generated per-step arrays); the
    captured graph reads fixed buffers, refilled before each replay (four small copies
    per step, counted in its time)."""
    import numpy as np
    import torch

    import kvp_workloads as W
    import sparse_decode_attention_kvzap_amd as K
    from sparse_decode_attention_kvzap_amd.pipeline import PrunedKVCache

    wl = W.BY_NAME["dms_delayed"]
    B, Hkv, Hq, d, P0, S = wl.B, wl.Hkv, wl.Hq, wl.d, wl.prompt, wl.steps
    log(f"[bench] {wl.name}: B={B} Hq={Hq} Hkv={Hkv} d={d} prompt={P0} steps={S} w={wl.w}")
    hidden = W.hidden_states(wl, P0, dev)
    kd, vd = W.kv_dense(wl, P0, dev)
    sw = W.scorer_weights(wl, dev)
    steps_in = [W.step_inputs(wl, i, dev) for i in range(S)]
    H_all, K_all, V_all, Q_all = (torch.stack([x[j] for x in steps_in]) for j in range(4))
    del steps_in
    scorer = K.Scorer(K.KVP_SCORER_LINEAR, sw.W1, sw.b1)
    cache = PrunedKVCache(B, Hkv, Hq, d, P0 + S, wl.kv_dtype, scorer, wl.w, wl.fixed_tau,
                          device=dev, max_prompt=P0)
    hb, kb, vb, qb = (torch.empty_like(X[0]) for X in (H_all, K_all, V_all, Q_all))
    elt = 2

    def prefill():
        cache.set_tau(wl.fixed_tau, stream)
        cache.prefill(hidden, kd, vd, stream)
        cache.set_position(P0, stream)
        cache.tau = cache.tau_dev  # the steps read tau from the device copy

    def feed(i):
        with torch.cuda.stream(stream):
            hb.copy_(H_all[i])
            kb.copy_(K_all[i])
            vb.copy_(V_all[i])
            qb.copy_(Q_all[i])

    # 1. token-heads each step's attention reads (untimed)
    prefill()
    visible = []
    for i in range(S):
        cache.advance(H_all[i], K_all[i], V_all[i], stream=stream)
        visible.append(cache.visible_token_heads())
    assert cache.check(stream) == 0

    def timed_loop(fused):
        prefill()
        torch.cuda.synchronize()
        e0, e1 = new_event(), new_event()
        e0.record(stream)
        for i in range(S):
            if fused:
                cache.step(H_all[i], K_all[i], V_all[i], Q_all[i], stream=stream)
            else:
                cache.advance(H_all[i], K_all[i], V_all[i], stream=stream)
                cache.attend(Q_all[i], stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    # 2. eager loops, timed: the separate calls (delayed step, then attention), and the
    #    fused decode step
    separate_ms = timed_loop(False)
    out_separate = cache.out.clone()
    eager_ms = timed_loop(True)
    out_fused = cache.out.clone()
    # the same eager steps reading fixed buffers refilled before each step (the four
    # copies the one-step graph below also makes), for a like-for-like comparison
    prefill()
    torch.cuda.synchronize()
    e0, e1 = new_event(), new_event()
    e0.record(stream)
    for i in range(S):
        feed(i)
        cache.step(hb, kb, vb, qb, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    eager_refill_ms = e0.elapsed_time(e1)
    assert torch.equal(cache.out, out_fused)
    fused_vs_separate = float((out_fused - out_separate).abs().max())

    # 3. the same loop with the step captured once and replayed
    prefill()
    feed(0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        cache.step(hb, kb, vb, qb, stream=side)
    torch.cuda.synchronize()
    prefill()
    torch.cuda.synchronize()
    e0, e1 = new_event(), new_event()
    e0.record(stream)
    with torch.cuda.stream(stream):
        for i in range(S):
            feed(i)
            graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    graph_ms = e0.elapsed_time(e1)
    assert cache.check(stream) == 0
    same = bool(torch.equal(cache.out, out_fused))
    del graph
    # 4. eight consecutive steps captured as one graph, each reading its slot of fixed
    #    buffers that hold eight steps' inputs (refilled by four copies before each
    #    replay, counted in its time): the GPU's idle time before a replay is paid once
    #    per eight steps
    G = 8
    bufs = [torch.empty((G,) + tuple(X.shape[1:]), dtype=X.dtype, device=dev)
            for X in (H_all, K_all, V_all, Q_all)]
    prefill()
    torch.cuda.synchronize()
    graph8 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph8, stream=side):
        for k in range(G):
            cache.step(*(b[k] for b in bufs), stream=side)
    torch.cuda.synchronize()
    prefill()
    torch.cuda.synchronize()
    e0, e1 = new_event(), new_event()
    e0.record(stream)
    with torch.cuda.stream(stream):
        for r8 in range(S // G):
            for b, X in zip(bufs, (H_all, K_all, V_all, Q_all)):
                b.copy_(X[r8 * G:(r8 + 1) * G])
            graph8.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    graph8_ms = e0.elapsed_time(e1) * S / (G * (S // G))
    assert cache.check(stream) == 0
    same8 = bool(torch.equal(cache.out, out_fused)) if S % G == 0 else None
    del graph8, bufs
    # 5. one graph per window of eight steps, each step reading its inputs where they lie
    #    (no refills): all windows captured before timing, then replayed in order
    graphs = []
    prefill()
    torch.cuda.synchronize()
    for r8 in range(S // G):
        gw = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gw, stream=side):
            for k in range(G):
                i = r8 * G + k
                cache.step(H_all[i], K_all[i], V_all[i], Q_all[i], stream=side)
        graphs.append(gw)
    torch.cuda.synchronize()
    prefill()
    torch.cuda.synchronize()
    e0, e1 = new_event(), new_event()
    e0.record(stream)
    with torch.cuda.stream(stream):
        for gw in graphs:
            gw.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    graph8_inplace_ms = e0.elapsed_time(e1) * S / (G * (S // G))
    assert cache.check(stream) == 0
    same8_inplace = bool(torch.equal(cache.out, out_fused)) if S % G == 0 else None
    del graphs
    # the decode attention alone, back to back on the cache the loop left (the last step's
    # token-heads)
    for _ in range(2):
        cache.attend(Q_all[S - 1], stream)
    e0, e1 = new_event(), new_event()
    e0.record(stream)
    for _ in range(20):
        cache.attend(Q_all[S - 1], stream)
    e1.record(stream)
    torch.cuda.synchronize()
    attn_ms = e0.elapsed_time(e1) / 20
    last_bytes = visible[-1] * (2 * d * elt + 4 / 16) + B * Hq * d * (elt + 4)
    achieved = gbs(last_bytes, attn_ms)
    th = float(np.sum(visible))
    r = {"workload": wl.name, "batch": B, "prompt": P0, "decode_steps": S, "delay_window": wl.w,
         "tau": wl.fixed_tau, "dtype": dtype_name(wl.kv_dtype),
         "eager_ms_per_step": eager_ms / S, "separate_calls_ms_per_step": separate_ms / S,
         "eager_refill_ms_per_step": eager_refill_ms / S,
         "graph_ms_per_step": graph_ms / S, "graph8_ms_per_step": graph8_ms / S,
         "graph8_inplace_ms_per_step": graph8_inplace_ms / S,
         "graph8_inplace_output_equals_eager": same8_inplace,
         "token_heads_per_s_eager": th / (eager_ms * 1e-3),
         "token_heads_per_s_graph": th / (graph_ms * 1e-3),
         "token_heads_per_s_graph8": th / (graph8_ms * 1e-3),
         "fused_vs_separate_max_abs": fused_vs_separate,
         "graph_output_equals_eager": same, "graph8_output_equals_eager": same8,
         "attn": {"ms": attn_ms, "bytes_per_call": last_bytes, "token_heads": visible[-1],
                  "gbs": achieved, "frac_of_peak": achieved / PEAK_HBM_GBS,
                  "token_heads_per_s": visible[-1] / (attn_ms * 1e-3),
                  "timing": "kvp_decode_attn back to back on the cache after the last step"},
         "token_heads_first_step": visible[0], "token_heads_last_step": visible[-1],
         "note": "each eager step: kvp_decode_step (the linear scorer and the delayed step "
                 "folded into the attention's stream and merge kernels) on that step's inputs "
                 "in place; separate_calls = kvp_score_step_delayed then kvp_decode_attn; the "
                 "graph holds the decode step and reads fixed buffers, refilled before each "
                 "replay (4 small copies per step, in its time); graph8 holds eight steps, "
                 "their inputs refilled by 4 copies per replay; graph8_inplace: one graph per "
                 "window of eight steps reading the inputs in place, captured before timing"}
    log(f"[bench] dms loop: eager {eager_ms / S * 1e3:.1f} us/step (separate calls "
        f"{separate_ms / S * 1e3:.1f}; with the graph's input refills "
        f"{eager_refill_ms / S * 1e3:.1f}), graph {graph_ms / S * 1e3:.1f} us/step, eight steps per "
        f"graph {graph8_ms / S * 1e3:.1f} us/step (output equals eager: {same8}), one graph per "
        f"eight-step window on the inputs in place {graph8_inplace_ms / S * 1e3:.1f} us/step "
        f"(equal: {same8_inplace}); attention "
        f"{attn_ms * 1e3:.1f} us at {achieved:.0f} GB/s on the last cache; token-heads "
        f"{visible[0]} -> {visible[-1]}; fused vs separate max diff {fused_vs_separate:.2e}")
    return r


# ------------------------------------------------------------------------------ CPU

def blas_threads():
    """Threads of the BLAS numpy calls into (None if threadpoolctl cannot tell)."""
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else None
    except Exception:
        return None


def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(ctx, rows):
    """The oracle as it stands, on a bounded sample of the headline workload: for `rows`
    batch rows (all KV heads) the MLP scores of every position, tau by the oracle's own
    quantile over the sample's prompt scores, the keep mask and the decode attention over
    the kept positions, timed on this host's cores."""
    import numpy as np
    import torch

    import oracle

    wl = ctx.wl

    def host(t):
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return oracle.bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
        return t.numpy().astype(np.float64)

    log(f"[bench] cpu baseline: oracle on {rows} batch row(s)")
    x = host(ctx.hidden[:rows])
    xn = host(ctx.h_new[:rows])
    Kd, Vd = host(ctx.kd[:rows]), host(ctx.vd[:rows])
    kn, vn, qq = host(ctx.k_new[:rows]), host(ctx.v_new[:rows]), host(ctx.q[:rows])
    sw = ctx.sw
    W1, b1 = host(sw.W1), host(sw.b1)
    W2 = host(sw.W2) if sw.W2 is not None else None
    b2 = host(sw.b2) if sw.b2 is not None else None
    t0 = time.perf_counter()
    xa = np.concatenate([x, xn], axis=1)
    if wl.scorer == "mlp":
        s = oracle.score_mlp(xa, W1, b1, W2, b2)
    else:
        s = oracle.score_linear(xa, W1, b1)
    tau = oracle.threshold_quantile(s[..., :ctx.T0], wl.keep_quantiles[0])
    vis = oracle.keep_mask(s, tau, wl.R)
    Ka = np.concatenate([Kd, kn[:, :, None]], axis=2)
    Va = np.concatenate([Vd, vn[:, :, None]], axis=2)
    out = oracle.decode_attention(qq, Ka, Va, vis, oracle.sm_scale(wl.d))
    dt = time.perf_counter() - t0
    kept = int(vis.sum())
    assert np.isfinite(out).all()
    return {"value": kept / dt, "unit": "kept token-heads/s",
            "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "threads": int(os.environ.get("OMP_NUM_THREADS", "0")) or None,
            "blas_threads": blas_threads(), "host": host_cpu_model(),
            "sample": f"{rows} of {wl.B} batch rows, all {wl.Hkv} KV heads, context {wl.T}: "
                      f"MLP scores of every position, tau = oracle.threshold_quantile of the "
                      f"sample's prompt scores at q {wl.keep_quantiles[0]}, keep mask, decode "
                      f"attention over the {kept} kept token-heads; {dt:.2f}s"}


# ------------------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default="all",
                    help="comma-separated records to run: " + ",".join(RECORDS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=16, help="batch rows in the CPU sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (the reference "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); this path has no "
              "cross-GPU work to measure", file=sys.stderr)
        sys.exit(2)
    only = RECORDS if args.only == "all" else tuple(args.only.split(","))
    bad = [r for r in only if r not in RECORDS]
    if bad:
        ap.error(f"unknown record(s) {bad}; choose from {RECORDS}")

    import torch

    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.int32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": src.numel() * 4, "launches": 5}))
        return

    import kvp_workloads as W
    import sparse_decode_attention_kvzap_amd as K

    torch.cuda.set_device(0)
    dev = "cuda:0"
    K.load()
    stream = torch.cuda.current_stream()
    wl = W.BY_NAME["qwen3_8b_layer"]
    records = {}
    line = None
    extra = args.warmup + args.steps + 64

    if any(r in only for r in ("headline", "prefill", "keep_scaling")):
        ctx = Context(wl, dev, extra=extra)
        if "headline" in only:
            log(f"[bench] headline {wl.name}: B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} d={wl.d} T={wl.T} "
                f"scorer={wl.scorer} keep quantile {wl.keep_quantiles[0]}")
            r = decode_run(ctx, wl.keep_quantiles[0], args.steps, args.warmup, stream, graph=True)
            a = r["attn"]
            # the same call timed one at a time after a 1 GiB read flush, 30 repetitions
            fl = flushed_attn_ms(ctx, stream, reps=30, stats=True)
            fl_bytes = ctx.attn_bytes(*ctx.read_split())
            fl["gbs_median"] = gbs(fl_bytes, fl["median_ms"])
            fl["frac_of_peak_median"] = fl["gbs_median"] / PEAK_HBM_GBS
            fl["bytes_per_call"] = fl_bytes
            a["flushed"] = fl
            log(f"[bench] decode step {r['ms_per_step'] * 1e3:.1f} us (separate calls "
                f"{r['separate_calls_ms_per_step'] * 1e3:.1f} us, graph replay "
                f"{r['graph_ms_per_step'] * 1e3:.1f} us, eight steps per graph "
                f"{r['graph8_ms_per_step'] * 1e3:.1f} us); attention {a['ms'] * 1e3:.1f} us = "
                f"{a['gbs']:.0f} GB/s ({100 * a['frac_of_peak']:.1f}% of peak), after a flush "
                f"{fl['median_ms'] * 1e3:.1f} us median / {fl['min_ms'] * 1e3:.1f} us min of 30; "
                f"{r['token_heads_per_step']:.0f} token-heads per step")
            cpu = None if args.no_cpu else cpu_baseline(ctx, args.cpu_rows)
            line = {
                "metric": METRIC,
                "value": r["token_heads_per_s"],
                "unit": "kept token-heads/s",
                "n_gpus": 1,
                "steps": args.steps,
                "warmup": args.warmup,
                "ms_per_step": r["ms_per_step"],
                "higher_is_better": True,
                "scaling": "weak",
                "vs_baseline": None,
                "dtype": dtype_name(wl.kv_dtype),
                "data": "synthetic (seeded N(0,1) hidden states, K, V, queries; random-init "
                        "MLP scorer)",
                "config": {"workload": wl.name, "batch": wl.B, "hidden": wl.H, "q_heads": wl.Hq,
                           "kv_heads": wl.Hkv, "head_dim": wl.d, "context": wl.T,
                           "scorer": f"mlp {wl.H}->{wl.inner}->{wl.Hkv}",
                           "keep_quantile": wl.keep_quantiles[0], "tau": r["tau"],
                           "recent": wl.R, "page": 16,
                           "token_heads_per_step": r["token_heads_per_step"],
                           "total_token_heads": r["total_token_heads"],
                           "step": "kvp_decode_step (MLP split-K first layer, then scoring finish, "
                                   "delayed step and attention in the attention's two kernels)"},
                "roofline": {"kernel": "kvp_decode_attn (decode_attn_kernel + decode_attn_merge_kernel)",
                             "bound": "hbm", "achieved": a["gbs"], "peak": PEAK_HBM_GBS,
                             "unit": "GB/s", "frac": a["frac_of_peak"],
                             "traffic": pmc_traffic("decode_attn"),
                             "traffic_unit": "HBM bytes/launch",
                             "per_launch_work": a["bytes_per_call"],
                             "per_launch_work_unit": "bytes", "launch_ms": a["ms"],
                             "launches_timed": a["launches"]},
                "cpu_baseline": cpu,
                "decode_step": {"ms": r["ms_per_step"], "graph_replay_ms": r["graph_ms_per_step"],
                                "graph8_replay_ms": r["graph8_ms_per_step"],
                                "separate_calls_ms": r["separate_calls_ms_per_step"],
                                "steps_per_s": 1e3 / r["ms_per_step"],
                                "sequence_steps_per_s": wl.B * 1e3 / r["ms_per_step"]},
                "decode_attn": a,
            }
        if "prefill" in only:
            records["prefill"] = record_prefill(ctx, stream)
            p = records["prefill"]
            log(f"[bench] prefill: score {p['score']['ms']:.3f} ms ({p['score']['tflops']:.0f} "
                f"TFLOP/s), threshold {p['threshold']['ms']:.3f}, select {p['select']['ms']:.3f}, "
                f"compact {p['compact']['ms']:.3f} ms ({p['compact']['gbs']:.0f} GB/s)")
        if "keep_scaling" in only:
            records["keep_scaling"] = record_keep_scaling(ctx, stream)
        del ctx
        torch.cuda.empty_cache()
    if "dms_delayed" in only:
        records["dms_delayed"] = dms_loop(dev, stream)
        torch.cuda.empty_cache()
    if "long_70b_layer" in only:
        records["long_70b_layer"] = record_long(dev, stream, args.steps, args.warmup)
        torch.cuda.empty_cache()
    for name in ("beacon_mixed", "beacon_int4", "beacon_fp8"):
        if name in only:
            records[name] = record_beacon(dev, stream, args.steps, args.warmup, name)
            torch.cuda.empty_cache()
    if "copy_ceiling" in only:
        records["copy_ceiling"] = record_copy_ceiling(dev, stream)
        log(f"[bench] copy ceiling: copy {records['copy_ceiling']['copy_gbs']:.0f} GB/s, read "
            f"{records['copy_ceiling']['read_gbs']:.0f} GB/s")

    if line is None:  # a run without the headline prints its records alone
        print(json.dumps({"records": records}), flush=True)
        return
    cc = records.get("copy_ceiling")
    if cc:
        line["roofline"]["frac_of_measured_copy"] = line["roofline"]["achieved"] / cc["copy_gbs"]
    line["records"] = records
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
