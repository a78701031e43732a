"""End-to-end parity of the whole hot path on every workload, against the CPU oracle.

Each test runs the pipeline through the C ABI (score -> select -> compact for the
prompt, then delayed steps and decode attention) and compares with the oracle:
scores within an absolute bound, visible sets exactly outside the band of scores within
1e-4 of tau (reported), attention within the parity tolerances (max-abs 2e-3 for bf16
KV) with the GPU's own decisions taken inside the band.  Reduced shapes are checked on every pair; the full
workload sizes (the configuration bench.py times) are checked on sampled pairs and
query heads, with tau taken from oracle scores.
"""
import math

import numpy as np
import pytest
import torch

import kvp_workloads as W
import oracle
from kvp_testlib import (BAND, check_attention, f64, np_bits, read_pool8, unpack_bits,
                         visible_positions)

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCORE_ATOL = 2.5e-5


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_decode_attention_kvzap_amd as K
    K.load()
    return K


def make_scorer(K, wl, sw):
    if wl.scorer == "mlp":
        return K.Scorer(K.KVP_SCORER_MLP, sw.W1, sw.b1, sw.W2, sw.b2)
    return K.Scorer(K.KVP_SCORER_LINEAR, sw.W1, sw.b1)


def oracle_scores(wl, sw, x_bits_rows, chunk=2048):
    """Oracle scores [rows, Hkv, T] for hidden rows given as a torch tensor [rows, T, H]."""
    W1 = f64(sw.W1)
    b1 = f64(sw.b1) if sw.b1 is not None else None
    out = []
    for r in range(x_bits_rows.shape[0]):
        parts = []
        for t0 in range(0, x_bits_rows.shape[1], chunk):
            x = f64(x_bits_rows[r:r + 1, t0:t0 + chunk])
            if wl.scorer == "mlp":
                parts.append(oracle.score_mlp(x, W1, b1, f64(sw.W2), f64(sw.b2)))
            else:
                parts.append(oracle.score_linear(x, W1, b1))
        out.append(np.concatenate(parts, axis=-1)[0])
    return np.stack(out)


def run_kvzap(K, wl, T, rows_check, tau=None, q_keep=None, demote=False, B=None):
    bits = wl.lp_bits
    """Prefill T-1 tokens, one decode step; compare sampled batch rows with the oracle."""
    from sparse_decode_attention_kvzap_amd.pipeline import PrunedKVCache
    B = B or wl.B
    wl = wl.scaled(B=B, T=T)
    T0 = T - 1
    x = W.hidden_states(wl, T, DEV)
    kd, vd = W.kv_dense(wl, T, DEV)
    q = W.queries(wl, DEV)
    sw = W.scorer_weights(wl, DEV)
    s64 = oracle_scores(wl, sw, x[rows_check])  # [rows, Hkv, T]
    if tau is None:
        tau = float(oracle.threshold_quantile(s64, q_keep))
    tau = np.float32(tau)
    cache = PrunedKVCache(B, wl.Hkv, wl.Hq, wl.d, T, wl.kv_dtype, make_scorer(K, wl, sw), wl.R,
                          float(tau), demote=demote, device=DEV, max_prompt=T0, lp_bits=bits)
    cache.prefill(x[:, :T0].contiguous(), kd[:, :, :T0].contiguous(), vd[:, :, :T0].contiguous())
    g_prefill_scores = cache.scores[rows_check].clone()
    out = cache.step(x[:, T0:].contiguous(), kd[:, :, T0].contiguous(), vd[:, :, T0].contiguous(),
                     q, T0)
    assert cache.check() == 0
    # scores (prompt from the prefill call, decode token from the step call)
    gs = np.concatenate([g_prefill_scores.cpu().double().numpy(),
                         cache.s_new[rows_check].cpu().double().numpy()], axis=-1)
    assert np.abs(gs - s64).max() < SCORE_ATOL, np.abs(gs - s64).max()
    keep = oracle.keep_mask(s64, tau, wl.R)  # [rows, Hkv, T] visible set at length T
    band = np.abs(s64 - np.float64(tau)) < BAND
    kd64, vd64, q64 = f64(kd[rows_check]), f64(vd[rows_check]), f64(q[rows_check])
    vis_gpu = np.zeros_like(keep)
    nband = int(band.sum())
    for ri, b in enumerate(rows_check):
        for h in range(wl.Hkv):
            p = b * wl.Hkv + h
            pos = visible_positions(cache.kv, cache.ring, p) if not demote else \
                np.sort(np.concatenate([_pool_ring_positions(cache, p)]))
            vis_gpu[ri, h, pos] = True
            assert len(np.unique(pos)) == len(pos)
    ok = ~band
    assert np.array_equal(vis_gpu[ok], keep[ok]), "visible set differs outside the band"
    vis_ref = np.where(band, vis_gpu, keep)
    if demote:
        ref = oracle.beacon_decode_attention(q64, kd64, vd64, vis_ref, oracle.sm_scale(wl.d),
                                             bits=bits)
        for ri, b in enumerate(rows_check):
            for h in range(wl.Hkv):
                p = b * wl.Hkv + h
                allpos = np.sort(np.concatenate([_pool_ring_positions(cache, p),
                                                 read_pool8(cache.kv, p)[0]]))
                assert np.array_equal(allpos, np.arange(T))
    else:
        ref = oracle.decode_attention(q64, kd64, vd64, vis_ref, oracle.sm_scale(wl.d))
    err = check_attention(out[rows_check], ref, wl.kv_dtype)
    return dict(tau=float(tau), band=nband, kept=float(keep.mean()), err=float(err),
                visible=cache.visible_token_heads())


def _pool_ring_positions(cache, p):
    from kvp_testlib import read_pool, read_ring
    return np.concatenate([read_pool(cache.kv, p)[0], read_ring(cache.ring, p)[0]])


# ------------------------------------------------------------------ tiny (full size)


def test_tiny_workload_end_to_end(K):
    r = run_kvzap(K, W.TINY, W.TINY.T, [0], q_keep=0.5)
    assert 0.45 < r["kept"] < 0.7


# ------------------------------------------------------------------ Qwen-3-8B-like


def test_qwen3_8b_layer_reduced_all_pairs(K):
    wl = W.QWEN3_8B_LAYER
    r = run_kvzap(K, wl, 3000, list(range(2)), q_keep=0.75, B=2)
    assert 0.2 < r["kept"] < 0.35


@pytest.mark.slow
def test_qwen3_8b_layer_full_size_sampled(K):
    """The benchmarked configuration (B=16, T=32768, MLP scorer, 25% kept): one batch
    row (8 pairs, 32 query heads) compared in full, tau from that row's oracle scores."""
    wl = W.QWEN3_8B_LAYER
    r = run_kvzap(K, wl, wl.T, [5], q_keep=0.75)
    assert 0.22 < r["kept"] < 0.3
    print(r)


# ------------------------------------------------------------------ 70B-like, outliers


@pytest.mark.parametrize("q_keep", [0.5, 0.75])
def test_long_70b_layer_reduced(K, q_keep):
    wl = W.LONG_70B_LAYER.scaled(H=1024)
    r = run_kvzap(K, wl, 6000, [0, 1], q_keep=q_keep, B=2)
    assert abs(r["kept"] - (1 - q_keep)) < 0.05


@pytest.mark.slow
@pytest.mark.parametrize("q_keep,row", [(0.5, 2), (0.75, 1)])
def test_long_70b_layer_full_size_sampled(K, q_keep, row):
    """B=4, H=8192, 64/8 heads, T=131072, outliers x8, keep 0.5 and 0.25: one batch row
    (8 pairs, 64 query heads) in full, tau from that row's oracle scores."""
    wl = W.LONG_70B_LAYER
    print(f"long_70b_layer full size q_keep={q_keep} row={row}", flush=True)
    r = run_kvzap(K, wl, wl.T, [row], q_keep=q_keep)
    assert abs(r["kept"] - (1 - q_keep)) < 0.03
    print(r)


# ------------------------------------------------------------------ BeaconKV


def test_beacon_reduced_all_pairs(K):
    wl = W.BEACON_MIXED
    r = run_kvzap(K, wl, 2500, [0, 1], q_keep=0.9, demote=True, B=2)
    assert 0.1 < r["kept"] < 0.2


@pytest.mark.slow
def test_beacon_full_size_sampled(K):
    """c2 shape with top-10% + recent 128 in bf16 and everything else int8: one batch
    row's 8 pairs; the oracle quantizes every demoted row itself."""
    wl = W.BEACON_MIXED
    r = run_kvzap(K, wl, wl.T, [11], q_keep=0.9, demote=True)
    print(r)


def test_beacon_int4_reduced_all_pairs(K):
    wl = W.BEACON_INT4
    r = run_kvzap(K, wl, 2500, [0, 1], q_keep=0.9, demote=True, B=2)
    assert 0.1 < r["kept"] < 0.2


@pytest.mark.slow
def test_beacon_int4_full_size_sampled(K):
    """The same shape and inputs with the demoted tokens in an int4 pool: one batch
    row's 8 pairs against the oracle's int4 round trips."""
    wl = W.BEACON_INT4
    r = run_kvzap(K, wl, wl.T, [5], q_keep=0.9, demote=True)
    print(r)


def test_beacon_fp8_reduced_all_pairs(K):
    wl = W.BEACON_FP8
    r = run_kvzap(K, wl, 2500, [0, 1], q_keep=0.9, demote=True, B=2)
    assert 0.1 < r["kept"] < 0.2


@pytest.mark.slow
def test_beacon_fp8_full_size_sampled(K):
    """The beacon shape and inputs with the demoted tokens as fp8 E4M3 codes: one batch
    row's 8 pairs against the oracle's E4M3 round trips."""
    wl = W.BEACON_FP8
    r = run_kvzap(K, wl, wl.T, [3], q_keep=0.9, demote=True)
    print(r)


# ------------------------------------------------------------------ DMS delayed eviction


def run_dms(K, wl, prompt, steps, rows_check, check_every=1, attn_steps=()):
    from sparse_decode_attention_kvzap_amd.pipeline import PrunedKVCache
    B = wl.B
    T = prompt + steps
    sw = W.scorer_weights(wl, DEV)
    x = W.hidden_states(wl, prompt, DEV)
    kd, vd = W.kv_dense(wl, prompt, DEV)
    scorer = make_scorer(K, wl, sw)
    cache = PrunedKVCache(B, wl.Hkv, wl.Hq, wl.d, T, wl.kv_dtype, scorer, wl.w, 0.0,
                          device=DEV, max_prompt=prompt)
    cache.prefill(x, kd, vd)
    # oracle flags for the checked rows: prompt scores, then each step's new score
    s_rows = [oracle_scores(wl, sw, x[rows_check])]
    k_rows, v_rows = [f64(kd[rows_check])], [f64(vd[rows_check])]
    nband = 0
    for i in range(steps):
        p = prompt + i
        h, k, v, q = W.step_inputs(wl, i, DEV)
        out = cache.step(h, k, v, q, p)
        s_rows.append(oracle_scores(wl, sw, h[rows_check]))
        k_rows.append(f64(k[rows_check])[:, :, None])
        v_rows.append(f64(v[rows_check])[:, :, None])
        if i % check_every and i not in attn_steps and i != steps - 1:
            continue
        s64 = np.concatenate(s_rows, axis=-1)  # [rows, Hkv, p+1]
        band = np.abs(s64) < BAND
        nband += int(band.sum())
        want = oracle.dms_visible(oracle.dms_evict_flags(s64), p, wl.w)
        got = np.zeros_like(want)
        for ri, b in enumerate(rows_check):
            for hh in range(wl.Hkv):
                got[ri, hh, visible_positions(cache.kv, cache.ring, b * wl.Hkv + hh)] = True
        assert np.array_equal(got[~band], want[~band]), f"step {i}"
        if i in attn_steps or i == steps - 1:
            kall = np.concatenate(k_rows, axis=2)
            vall = np.concatenate(v_rows, axis=2)
            ref = oracle.decode_attention(f64(q[rows_check]), kall, vall, np.where(band, got, want),
                                          oracle.sm_scale(wl.d))
            check_attention(out[rows_check], ref, wl.kv_dtype)
    assert cache.check() == 0
    return nband


def test_dms_reduced_every_step(K):
    wl = W.DMS_DELAYED.scaled(B=3, H=1024)
    run_dms(K, wl, prompt=700, steps=300, rows_check=[0, 1, 2], check_every=1,
            attn_steps=(0, 1, 255, 256, 257, 299))


@pytest.mark.slow
def test_dms_full_size_sampled(K):
    """B=64, 8192-token prompt + 1024 steps, w=256: batch rows 0 and 37 checked at the
    sampled steps (visible sets vs the stateless oracle; attention at a subset)."""
    wl = W.DMS_DELAYED
    run_dms(K, wl, prompt=wl.prompt, steps=wl.steps, rows_check=[0, 37], check_every=64,
            attn_steps=(0, 1, 255, 256, 257, 511, 1023))
