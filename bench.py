"""Benchmark of the hot path on one MI355X.

A step is one pass of every hot-path call over one batch of synthetic input, in the
configuration the headline metric is quoted on (Qwen-3-8B-like single layer: B=16,
H=4096, 32 Q / 8 KV heads, d=128, T=32768 including the decode token, bf16 KV in
16-token pages, MLP scorer 4096->512->8, tau at the 75th percentile (25% kept),
recent 128 kept):
    prefill compression:  kvp_score (MLP over 16 x 32767 hidden states)
                          -> kvp_threshold (tau = 75th percentile, on the device)
                          -> kvp_select -> kvp_compact (pool + 128-slot ring)
    decode step:          kvp_score_step_delayed (the new tokens scored inside the
                          delayed step) -> kvp_decode_attn
Inputs are resident in HBM before timing.  `value` is kept-KV decode-attention
token-heads per second of whole step time; the per-call breakdown, the decode-only
rate and an isolated (cache-flushed) decode-attention rate are reported beside it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
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


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def pmc_traffic(key):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs
    (scaled by the plain-copy calibration), or None once the kernel's source differs
    from the one that was profiled."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "pmc_traffic_qwen3_8b_layer.json")
    try:
        rec = json.load(open(path))[key]
        src = open(os.path.join(ROOT, rec["source"]), "rb").read()
    except (OSError, KeyError, ValueError):
        return None
    if hashlib.sha256(src).hexdigest()[:16] != rec["source_sha256_16"]:
        return None
    return rec["hbm_bytes_per_launch"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_8b_layer")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=16, help="batch rows in the CPU sample")
    ap.add_argument("--no-scaling", action="store_true",
                    help="skip the keep-ratio sweep (profiling runs of the headline workload)")
    ap.add_argument("--no-prefill-attn", action="store_true",
                    help="skip the prefill-attention-under-eviction measurement")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (the reference "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        src = torch.ones(1 << 28, dtype=torch.int32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": src.numel() * 4, "launches": 5}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); this path has no "
              "cross-GPU work to measure", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import kvp_workloads as W
    import sparse_decode_attention_kvzap_amd as K
    from sparse_decode_attention_kvzap_amd.pipeline import PrunedKVCache

    torch.cuda.set_device(0)
    dev = "cuda:0"
    K.load()
    wl = W.BY_NAME[args.workload]
    if wl.steps:
        return dms_loop(args, wl, dev)
    T = wl.T
    T0 = T - 1  # prompt positions 0..T-2, the decode token is position T-1
    B, Hkv, Hq, d, H = wl.B, wl.Hkv, wl.Hq, wl.d, wl.H
    log(f"[bench] workload {wl.name}: B={B} H={H} Hq={Hq} Hkv={Hkv} d={d} T={T} "
        f"scorer={wl.scorer}")

    t0 = time.perf_counter()
    hidden = W.hidden_states(wl, T0, dev)
    kd, vd = W.kv_dense(wl, T0, dev)
    sw = W.scorer_weights(wl, dev)
    h_new, k_new, v_new, q = W.step_inputs(wl, 0, dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs generated in {time.perf_counter() - t0:.1f}s")

    if wl.scorer == "mlp":
        scorer = K.Scorer(K.KVP_SCORER_MLP, sw.W1, sw.b1, sw.W2, sw.b2)
    else:
        scorer = K.Scorer(K.KVP_SCORER_LINEAR, sw.W1, sw.b1)
    q_keep = wl.keep_quantiles[0]
    cache = PrunedKVCache(B, Hkv, Hq, d, T, wl.kv_dtype, scorer, wl.R, 0.0, device=dev,
                          max_prompt=T0, demote=wl.int8_demote, lp_bits=wl.lp_bits)
    # tau is calibrated on the device inside every step (kvp_threshold: the exact
    # q-quantile of the prompt's scores); its value is logged once here
    cache.score(hidden)
    cache.calibrate(q_keep, T0)
    tau = float(cache.tau_dev.item())
    log(f"[bench] tau = {tau:.6f} (quantile {q_keep}, computed on the device)")

    calls = ["score_prefill", "threshold", "select", "compact", "score_step", "decode_attn"]
    pos_start = torch.tensor([T0, 0], dtype=torch.int32, device=dev)

    def one_step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        cache.score(hidden)
        mark(1)
        cache.calibrate(q_keep, T0)
        mark(2)
        cache.select(T0)
        mark(3)
        cache.compact(kd, vd)
        cache.pos_dev.copy_(pos_start)  # the decode token's position, T0
        mark(4)
        K.kvp_score_step_delayed(scorer, h_new, cache.kv, cache.ring, k_new, v_new, cache.tau_dev,
                                 cache.pos_dev, cache.s_new, cache.ws_score)
        mark(5)
        cache.attend(q)
        mark(6)

    for i in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    st = cache.check()
    assert st == 0, f"capacity error {st}"
    visible = cache.visible_token_heads()
    kept_prefill = int(cache.kept_count.sum())  # before the keep sweep below re-selects
    lp_visible = int(cache.kv.length8.sum()) if wl.int8_demote else 0
    kv_bytes_attn = attn_bytes(cache, wl, B, Hq, d)
    total_th = B * Hkv * T
    log(f"[bench] warmup done; visible token-heads {visible} of {total_th} "
        f"({visible / total_th:.3f})")

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
           for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for s in range(args.steps):
        one_step(evs[s])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    per_call = {c: float(np.mean([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(args.steps)]))
                for i, c in enumerate(calls)}
    log(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step (wall {wall:.3f}s); "
        + ", ".join(f"{c} {v:.3f}" for c, v in per_call.items()))

    # isolated decode attention; before each repetition the 256 MB MALL is flushed by
    # READING 1 GiB (a write flush would leave dirty lines draining into the timed run).
    # The flush runs on the same stream right before the timed call, with no host sync
    # in between: an idle GPU takes several microseconds to start the next kernel.
    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)  # 1 GiB
    fsum = torch.zeros(1, dtype=torch.int64, device=dev)
    iso = []
    for r in range(12):
        fsum.add_(flush.sum())
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        cache.attend(q)
        e1.record()
        torch.cuda.synchronize()
        if r >= 2:
            iso.append(e0.elapsed_time(e1))
    attn_iso_ms = float(np.median(iso))
    del flush
    # the prefill scoring call back to back (no other kernels between calls)
    iso = []
    for r in range(5):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        cache.score(hidden)
        e1.record()
        torch.cuda.synchronize()
        if r >= 1:
            iso.append(e0.elapsed_time(e1))
    score_iso_ms = float(np.median(iso))

    # The decode step alone, back to back on the compressed context (positions T0, T0 + 1,
    # ... appended on the device): eagerly, and captured once as a HIP graph and replayed
    # (every per-step value lives in device memory, so the replays need no host work).
    def decode_only():
        K.kvp_score_step_delayed(scorer, h_new, cache.kv, cache.ring, k_new, v_new,
                                 cache.tau_dev, cache.pos_dev, cache.s_new, cache.ws_score)
        cache.attend(q)

    def time_steps(fn, n=8):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    cache.select(T0)
    cache.compact(kd, vd)
    cache.pos_dev.copy_(pos_start)
    decode_eager_ms = time_steps(decode_only)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        decode_only()
    torch.cuda.synchronize()
    cache.select(T0)
    cache.compact(kd, vd)
    cache.pos_dev.copy_(pos_start)
    decode_graph_ms = time_steps(graph.replay)
    assert cache.check() == 0
    del graph
    log(f"[bench] decode step back to back: eager {decode_eager_ms * 1e3:.1f} us, "
        f"graph replay {decode_graph_ms * 1e3:.1f} us")

    # End-to-end scaling with kept tokens: the decode step (score the new tokens ->
    # delayed step -> attention) right after compressing the same context at several
    # keep ratios (keep 1.0: tau = -inf keeps every token), and the attention alone after
    # a read flush.  Compression is redone untimed before every repetition.
    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    keep_scaling = []
    for keep in (() if args.no_scaling else (1.0, 0.5, 0.25)):
        if keep >= 1.0:
            tau_k = float("-inf")
        else:
            cache.calibrate(1.0 - keep, T0)
            tau_k = float(cache.tau_dev.item())
        cache.tau = tau_k
        dec, att = [], []
        for r in range(6):
            cache.select(T0)
            cache.compact(kd, vd)
            cache.tau_dev.fill_(tau_k)
            cache.pos_dev.copy_(pos_start)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            ev[0].record()
            K.kvp_score_step_delayed(scorer, h_new, cache.kv, cache.ring, k_new, v_new,
                                     cache.tau_dev, cache.pos_dev, cache.s_new, cache.ws_score)
            ev[1].record()
            cache.attend(q)
            ev[2].record()
            fsum.add_(flush.sum())
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            cache.attend(q)
            e1.record()
            torch.cuda.synchronize()
            if r >= 1:
                dec.append(ev[0].elapsed_time(ev[2]))
                att.append(e0.elapsed_time(e1))
        vis_k = cache.visible_token_heads()
        bytes_k = attn_bytes(cache, wl, B, Hq, d)
        # steady state: decode steps back to back (positions T0, T0 + 1, ... appended on the
        # device, as in a decode loop), timed after three untimed steps let the compaction's
        # write-back drain
        cache.select(T0)
        cache.compact(kd, vd)
        cache.tau_dev.fill_(tau_k)
        cache.pos_dev.copy_(pos_start)

        def dstep():
            K.kvp_score_step_delayed(scorer, h_new, cache.kv, cache.ring, k_new, v_new,
                                     cache.tau_dev, cache.pos_dev, cache.s_new, cache.ws_score)
            cache.attend(q)
        for _ in range(3):
            dstep()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(8):
            dstep()
        e1.record()
        torch.cuda.synchronize()
        assert cache.check() == 0
        keep_scaling.append({"keep": keep, "tau": tau_k if keep < 1.0 else None,
                             "visible_token_heads": vis_k,
                             "attn_bytes": bytes_k,
                             "decode_step_ms": float(np.median(dec)),
                             "decode_step_steady_ms": e0.elapsed_time(e1) / 8,
                             "attn_isolated_ms": float(np.median(att))})
    del flush
    cache.calibrate(q_keep, T0)
    base = keep_scaling[0] if keep_scaling else None
    for e in keep_scaling:
        e["bytes_ratio_vs_keep1"] = e["attn_bytes"] / base["attn_bytes"]
        e["decode_step_ratio_vs_keep1"] = e["decode_step_ms"] / base["decode_step_ms"]
        e["decode_step_steady_ratio_vs_keep1"] = e["decode_step_steady_ms"] / base["decode_step_steady_ms"]
        e["attn_ratio_vs_keep1"] = e["attn_isolated_ms"] / base["attn_isolated_ms"]
        e["attn_gbs"] = e["attn_bytes"] / (e["attn_isolated_ms"] * 1e-3) / 1e9
    log("[bench] keep scaling: " + "; ".join(
        f"keep {e['keep']}: decode {e['decode_step_ms']:.3f} ms (x{e['decode_step_ratio_vs_keep1']:.2f}), "
        f"steady {e['decode_step_steady_ms']:.3f} ms (x{e['decode_step_steady_ratio_vs_keep1']:.2f}), "
        f"attn {e['attn_isolated_ms']:.3f} ms (x{e['attn_ratio_vs_keep1']:.2f}), bytes x{e['bytes_ratio_vs_keep1']:.2f}"
        for e in keep_scaling))

    prefill_attn = None
    if not args.no_prefill_attn and wl.kv_dtype == torch.bfloat16 and not wl.int8_demote:
        prefill_attn = measure_prefill_attn(K, W, wl, cache, kd, vd, T0, dev)
        log(f"[bench] prefill attention under eviction (keep {1 - q_keep:.2f}, window {wl.R}): "
            f"{prefill_attn['ms']:.2f} ms, {prefill_attn['tflops']:.0f} TFLOP/s useful "
            f"({100 * prefill_attn['frac_of_bf16_peak']:.1f}% of the bf16 dense peak), "
            f"visible keys {prefill_attn['visible_fraction']:.3f} of causal")

    # algorithmic work per call
    elt = 2 if wl.kv_dtype == torch.bfloat16 else 4
    ntok = B * T0
    if wl.scorer == "mlp":
        score_flops = 2.0 * ntok * H * wl.inner + 2.0 * ntok * wl.inner * Hkv
    else:
        score_flops = 2.0 * ntok * H * Hkv
    score_bytes = ntok * H * elt + ntok * Hkv * 4
    select_bytes = ntok * Hkv * 4 + B * Hkv * T0 * 4 + B * Hkv * ((T0 + 31) // 32) * 4 * 2
    compact_bytes = kept_prefill * 2 * d * elt * 2 + kept_prefill * 4
    if wl.int8_demote:  # demoted tokens: read in full, written as codes + one scale per row
        demoted = B * Hkv * T0 - kept_prefill
        compact_bytes += demoted * (2 * d * elt + 2 * (d * wl.lp_bits // 8 + 4) + 4)
    gbs = lambda b, ms: b / (ms * 1e-3) / 1e9  # noqa: E731
    kernels = {
        "score_prefill": {"ms": per_call["score_prefill"],
                          "tflops": score_flops / (per_call["score_prefill"] * 1e-3) / 1e12,
                          "gbs": gbs(score_bytes, per_call["score_prefill"]),
                          "traffic": pmc_traffic("score_mlp_bf16") if wl.scorer == "mlp" else None},
        "score_prefill_back_to_back": {"ms": score_iso_ms,
                                       "tflops": score_flops / (score_iso_ms * 1e-3) / 1e12},
        "threshold": {"ms": per_call["threshold"], "gbs": gbs(ntok * Hkv * 4 * 3, per_call["threshold"]),
                      "note": "exact radix select on the device, three passes over the scores"},
        "select": {"ms": per_call["select"], "gbs": gbs(select_bytes, per_call["select"])},
        "compact": {"ms": per_call["compact"], "gbs": gbs(compact_bytes, per_call["compact"]),
                    "traffic": pmc_traffic("compact_copy")},
        "score_step": {"ms": per_call["score_step"],
                       "note": "kvp_score_step_delayed: the new tokens' scores computed inside the "
                               "delayed step (linear: one kernel; MLP: split-K first layer, then "
                               "the step with the MLP finish)"},
        "decode_attn": {"ms": per_call["decode_attn"], "gbs": gbs(kv_bytes_attn, per_call["decode_attn"]),
                        "token_heads_per_s": visible / (per_call["decode_attn"] * 1e-3)},
        "prefill_attn": prefill_attn,
        "decode_attn_isolated": {"ms": attn_iso_ms, "gbs": gbs(kv_bytes_attn, attn_iso_ms),
                                 "frac_of_peak": gbs(kv_bytes_attn, attn_iso_ms) / PEAK_HBM_GBS,
                                 "token_heads_per_s": visible / (attn_iso_ms * 1e-3),
                                 "traffic": pmc_traffic("decode_attn"),
                                 "note": "main + merge kernel, after a 1 GiB read flush"},
    }
    decode_ms = per_call["score_step"] + per_call["decode_attn"]
    dominant = max(("score_prefill", "select", "compact", "decode_attn"), key=lambda c: per_call[c])
    if dominant == "score_prefill" and wl.scorer == "mlp":
        achieved = score_flops / (per_call[dominant] * 1e-3) / 1e12
        roofline = {"kernel": "kvp_score (MLP: score_mlp_bf16 + score_mlp_finish)",
                    "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                    "traffic": pmc_traffic("score_mlp_bf16"), "traffic_unit": "HBM bytes/launch",
                    "per_launch_work": score_flops, "per_launch_work_unit": "flop"}
    else:
        b = {"score_prefill": score_bytes, "select": select_bytes, "compact": compact_bytes,
             "decode_attn": kv_bytes_attn}[dominant]
        achieved = gbs(b, per_call[dominant])
        roofline = {"kernel": dominant, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                    "traffic": pmc_traffic({"decode_attn": "decode_attn", "compact": "compact_copy"}.get(dominant, dominant)),
                    "traffic_unit": "HBM bytes/launch", "per_launch_work": b,
                    "per_launch_work_unit": "bytes"}

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(wl, hidden, kd, vd, q, h_new, k_new, v_new, sw, tau, T0, args.cpu_rows)

    line = {
        "metric": "kept-KV decode attention tokens/s + achieved HBM GB/s (% of peak), 1 GPU",
        "value": visible / (ms_per_step * 1e-3),
        "unit": "kept token-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "hidden": H, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": d, "context": T, "scorer": wl.scorer, "keep_quantile": q_keep,
                   "recent": wl.R, "page": 16, "visible_token_heads": visible,
                   "low_precision_pool": ({"bits": wl.lp_bits, "token_heads": lp_visible}
                                          if wl.int8_demote else None),
                   "total_token_heads": total_th},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "decode_step": {"ms": decode_ms, "token_heads_per_s": visible / (decode_ms * 1e-3),
                        "back_to_back_eager_ms": decode_eager_ms,
                        "back_to_back_graph_ms": decode_graph_ms,
                        "note": "ms: right after compaction, inside the step; back_to_back: the "
                                "decode step repeated on the compressed context, eagerly and "
                                "as one captured graph replayed"},
        "kernels": kernels,
        "keep_scaling": keep_scaling,
    }
    print(json.dumps(line), flush=True)


def measure_prefill_attn(K, W, wl, cache, kd, vd, T0, dev, reps=3) -> dict:
    """kvp_prefill_attn over the prompt under the headline selection: every prompt
    position attends to the kept keys before it plus the last `window` positions.
    Useful work = 4 d flop per (query row, visible key) pair (QK^T and PV)."""
    import torch
    cache.select(T0)
    qp = W.prompt_queries(wl, T0, dev)
    out = torch.empty((wl.B, wl.Hq, T0, wl.d), dtype=torch.float32, device=dev)
    R = cache.window
    keep = (cache.scores[:, :, :T0] >= cache.tau_dev).reshape(cache.P, T0)
    ck = torch.cumsum(keep.to(torch.int32), dim=1)
    i = torch.arange(T0, device=dev)
    before = torch.where(i >= R, ck[:, (i - R).clamp(min=0)], torch.zeros_like(ck))
    vis = before.double().sum().item() + cache.P * float(torch.clamp(i + 1, max=R).double().sum())
    pairs = vis * (wl.Hq // wl.Hkv)
    flops = pairs * 4 * wl.d
    causal = cache.P * (wl.Hq // wl.Hkv) * T0 * (T0 + 1) / 2
    stream = torch.cuda.current_stream()
    cache.prefill_attention(qp, kd, vd, out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        cache.prefill_attention(qp, kd, vd, out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del qp, out, keep, ck
    torch.cuda.empty_cache()
    tflops = flops / (ms * 1e-3) / 1e12
    return {"ms": ms, "tflops": tflops, "frac_of_bf16_peak": tflops / PEAK_BF16_TFLOPS,
            "traffic": pmc_traffic("prefill_attn"), "traffic_unit": "HBM bytes/launch",
            "useful_flop": flops, "visible_pairs": pairs, "visible_fraction": pairs / causal,
            "note": "kvp_prefill_attn (prefill_attn_kernel<128>), q/k/v bf16, out fp32; "
                    "useful = 4 d flop per visible (row, key) pair"}


def attn_bytes(cache, wl, B, Hq, d) -> int:
    """Algorithmic bytes of one decode attention over the cache as it stands: K and V of
    every visible bf16/fp32 token-head, codes plus two fp32 scales of every token-head in
    the low-precision pool, the queries read and the fp32 outputs written."""
    import torch

    elt = 2 if wl.kv_dtype == torch.bfloat16 else 4
    lp = int(cache.kv.length8.sum()) if wl.int8_demote else 0
    main = cache.visible_token_heads() - lp
    return main * 2 * d * elt + lp * 2 * (d * wl.lp_bits // 8 + 4) + B * Hq * d * (elt + 4)


def dms_loop(args, wl, dev):
    """The delayed-eviction decode loop: compress the prompt (tau = 0, recent window w),
    then run wl.steps decode steps (score the new token -> delayed step -> attention),
    eagerly and as one captured HIP graph replayed per step.  The graph is possible
    because every per-step value (threshold, position) lives in device memory; inputs go
    through fixed buffers that are refilled before each replay."""
    import numpy as np
    import torch

    import kvp_workloads as W
    import sparse_decode_attention_kvzap_amd as K
    from sparse_decode_attention_kvzap_amd.pipeline import PrunedKVCache

    B, Hkv, Hq, d, P0, S = wl.B, wl.Hkv, wl.Hq, wl.d, wl.prompt, wl.steps
    log(f"[bench] workload {wl.name}: B={B} Hq={Hq} Hkv={Hkv} d={d} prompt={P0} steps={S} "
        f"w={wl.w} scorer={wl.scorer} tau={wl.fixed_tau}")
    t0 = time.perf_counter()
    hidden = W.hidden_states(wl, P0, dev)
    kd, vd = W.kv_dense(wl, P0, dev)
    sw = W.scorer_weights(wl, dev)
    steps_in = [W.step_inputs(wl, i, dev) for i in range(S)]
    H_all = torch.stack([x[0] for x in steps_in])
    K_all = torch.stack([x[1] for x in steps_in])
    V_all = torch.stack([x[2] for x in steps_in])
    Q_all = torch.stack([x[3] for x in steps_in])
    del steps_in
    torch.cuda.synchronize()
    log(f"[bench] inputs generated in {time.perf_counter() - t0:.1f}s")
    scorer = K.Scorer(K.KVP_SCORER_LINEAR, sw.W1, sw.b1) if wl.scorer == "linear" else \
        K.Scorer(K.KVP_SCORER_MLP, sw.W1, sw.b1, sw.W2, sw.b2)
    cache = PrunedKVCache(B, Hkv, Hq, d, P0 + S, wl.kv_dtype, scorer, wl.w, wl.fixed_tau,
                          device=dev, max_prompt=P0)
    hb, kb, vb, qb = (torch.empty_like(X[0]) for X in (H_all, K_all, V_all, Q_all))

    def prefill():
        cache.set_tau(wl.fixed_tau)
        cache.prefill(hidden, kd, vd)
        cache.set_position(P0)
        cache.tau = cache.tau_dev  # the steps read tau from the device copy

    def feed(i):
        hb.copy_(H_all[i])
        kb.copy_(K_all[i])
        vb.copy_(V_all[i])
        qb.copy_(Q_all[i])

    # 1. visible token-heads per step and per-call attention time (eager, untimed loop)
    prefill()
    visible, attn_ms = [], []
    for i in range(S):
        feed(i)
        cache.advance(hb, kb, vb)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        cache.attend(qb)
        e1.record()
        torch.cuda.synchronize()
        attn_ms.append(e0.elapsed_time(e1))
        visible.append(cache.visible_token_heads())
    assert cache.check() == 0
    out_eager = cache.out.clone()

    # 2. eager loop, timed
    prefill()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(S):
        feed(i)
        cache.step(hb, kb, vb, qb)
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1)
    assert torch.equal(cache.out, out_eager)

    # 3. the same loop with the step captured once and replayed
    prefill()
    feed(0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        cache.set_position(P0)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            cache.step(hb, kb, vb, qb)
    torch.cuda.synchronize()
    prefill()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(S):
        feed(i)
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_ms = e0.elapsed_time(e1)
    assert cache.check() == 0
    same = bool(torch.equal(cache.out, out_eager))
    # replays alone (inputs left in place; the same work per step)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    prefill()
    torch.cuda.synchronize()
    e0.record()
    for i in range(S):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    replay_ms = e0.elapsed_time(e1)

    elt = 2 if wl.kv_dtype == torch.bfloat16 else 4
    th = float(np.sum(visible))
    attn_bytes = th * 2 * d * elt
    attn_total_ms = float(np.sum(attn_ms))
    achieved = attn_bytes / (attn_total_ms * 1e-3) / 1e9
    line = {
        "metric": "kept-KV decode attention tokens/s + achieved HBM GB/s (% of peak), 1 GPU",
        "value": th / (graph_ms * 1e-3),
        "unit": "kept token-heads/s",
        "n_gpus": 1,
        "steps": S,
        "warmup": 0,
        "ms_per_step": graph_ms / S,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "hidden": wl.H, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": d, "prompt": P0, "decode_steps": S, "delay_window": wl.w,
                   "tau": wl.fixed_tau, "scorer": wl.scorer, "page": 16},
        "roofline": {"kernel": "kvp_decode_attn (main + merge)", "bound": "hbm",
                     "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": None,
                     "per_launch_work": attn_bytes / S, "per_launch_work_unit": "bytes (mean)"},
        "cpu_baseline": None,
        "dms_loop": {"eager_ms_per_step": eager_ms / S, "graph_ms_per_step": graph_ms / S,
                     "graph_replay_only_ms_per_step": replay_ms / S,
                     "attn_ms_per_step": attn_total_ms / S,
                     "visible_token_heads_first": visible[0], "visible_token_heads_last": visible[-1],
                     "graph_output_equals_eager": same,
                     "note": "each step: refill the 4 input buffers, then score the new token + "
                             "delayed step (one kernel, kvp_score_step_delayed, for the linear "
                             "scorer) and attention (main + merge); the graph holds the last two"},
    }
    log(f"[bench] dms loop: eager {eager_ms / S * 1e3:.1f} us/step, graph {graph_ms / S * 1e3:.1f} "
        f"us/step (replay only {replay_ms / S * 1e3:.1f}), attention {attn_total_ms / S * 1e3:.1f} "
        f"us/step at {achieved:.0f} GB/s; visible {visible[0]} -> {visible[-1]}")
    print(json.dumps(line), flush=True)


def cpu_baseline(wl, hidden, kd, vd, q, h_new, k_new, v_new, sw, tau, T0, rows):
    """The oracle as it stands, on a bounded sample: the whole path for `rows` batch
    rows (all KV heads), timed on this host's cores."""
    import numpy as np
    import torch

    import oracle

    def host(t):
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return oracle.bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
        return t.numpy().astype(np.float64)

    log(f"[bench] cpu baseline: oracle on {rows} batch row(s)")
    x = host(hidden[:rows])
    xn = host(h_new[:rows])
    Kd = host(kd[:rows])
    Vd = host(vd[:rows])
    kn = host(k_new[:rows])
    vn = host(v_new[:rows])
    qq = host(q[:rows])
    W1, b1 = host(sw.W1), host(sw.b1)
    W2 = host(sw.W2) if sw.W2 is not None else None
    b2 = host(sw.b2) if sw.b2 is not None else None
    t0 = time.perf_counter()
    xa = np.concatenate([x, xn], axis=1)
    if wl.scorer == "mlp":
        s = oracle.score_mlp(xa, W1, b1, W2, b2)
    else:
        s = oracle.score_linear(xa, W1, b1)
    vis = oracle.keep_mask(s, tau, wl.R)
    Ka = np.concatenate([Kd, kn[:, :, None]], axis=2)
    Va = np.concatenate([Vd, vn[:, :, None]], axis=2)
    if wl.int8_demote:  # every token stays visible; the evicted ones as low-precision codes
        out = oracle.beacon_decode_attention(qq, Ka, Va, vis, oracle.sm_scale(wl.d), bits=wl.lp_bits)
        vis = np.ones_like(vis)
    else:
        out = oracle.decode_attention(qq, Ka, Va, vis, oracle.sm_scale(wl.d))
    dt = time.perf_counter() - t0
    kept = int(vis.sum())
    assert np.isfinite(out).all()
    return {"value": kept / dt, "unit": "kept token-heads/s",
            "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "threads": int(os.environ.get("OMP_NUM_THREADS", "0")) or None,
            "sample": f"whole path (score, threshold, mask, compact, attend) for {rows} of "
                      f"{wl.B} batch rows, all {wl.Hkv} KV heads; {dt:.2f}s"}


if __name__ == "__main__":
    main()
