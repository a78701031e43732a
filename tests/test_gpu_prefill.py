"""Parity of prefill attention under eviction (kvp_prefill_attn, through the C ABI)
against the oracle's masked causal attention: position i sees key j iff j <= i and
(keep_j or i - j < W).

Shapes cover every supported head ratio (g = 1, 2, 4, 8), both head dims, ragged T
(tails of the 64-key tiles and of the 128 / g position blocks), W = 0 (rows that see
nothing), W > T (plain causal attention), nothing or everything kept, keep bits set
past T, outlier keys (peaked softmax), the selection written by kvp_select for the
KVzap and DMS rules, V values beyond fp16's range, and the full qwen3-8B-like layer
shape on sampled rows.  Tolerance: max-abs 2e-3 (bf16 K/V).
"""
import numpy as np
import pytest
import torch

import kvp_workloads as W
import oracle
from kvp_testlib import check_attention, f64, np_bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_decode_attention_kvzap_amd as K
    K.load()
    return K


def pack_bits(keep: np.ndarray, tail: bool = False) -> torch.Tensor:
    """bool [P, T] -> keep_bits [P, ceil(T/32)] (int32 storage of u32 words)."""
    P, T = keep.shape
    nw = (T + 31) // 32
    full = np.zeros((P, nw * 32), bool)
    full[:, :T] = keep
    if tail:
        full[:, T:] = True  # bits past T must be ignored
    w = np.zeros((P, nw), np.uint32)
    for bit in range(32):
        w |= full[:, bit::32].astype(np.uint32) << np.uint32(bit)
    return torch.from_numpy(w.view(np.int32)).to(DEV)


def kept_list(keep: np.ndarray) -> torch.Tensor:
    P, T = keep.shape
    idx = np.zeros((P, T), np.int32)
    for p in range(P):
        k, e = oracle.partition_indices(keep[p])
        idx[p] = np.concatenate([k, e])
    return torch.from_numpy(idx).to(DEV)


def inputs(B, Hq, Hkv, T, d, seed, outliers=0.0):
    q = W.normal((B, Hq, T, d), torch.bfloat16, seed, DEV)
    k = W.normal((B, Hkv, T, d), torch.bfloat16, seed + 1, DEV)
    v = W.normal((B, Hkv, T, d), torch.bfloat16, seed + 2, DEV)
    if outliers > 0:
        g = torch.Generator().manual_seed(seed + 3)
        n = max(1, int(outliers * T))
        for b in range(B):
            pos = torch.randperm(T, generator=g)[:n].to(DEV)
            k[b][:, pos] *= 8
            v[b][:, pos] *= 8
    return q, k, v


def run(K, q, k, v, bits, idx, window):
    B, Hq, T, d = q.shape
    out = torch.full((B, Hq, T, d), float("nan"), device=DEV)
    K.kvp_prefill_attn(q, k, v, bits, idx, window, K.sm_scale(d), out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("B,Hq,Hkv,T,d,window,keepfrac,outl", [
    (1, 8, 2, 1000, 128, 128, 0.3, 0.0),   # g 4, several position blocks and key tiles
    (2, 8, 8, 517, 128, 64, 0.25, 0.0),    # g 1, ragged
    (1, 16, 2, 300, 64, 16, 0.5, 0.0),     # g 8, d 64
    (2, 4, 2, 777, 64, 128, 0.1, 0.0),     # g 2
    (1, 32, 2, 700, 128, 64, 0.3, 0.0),    # g 16: 16-position blocks, one head per column tile
    (2, 16, 1, 301, 64, 128, 0.5, 0.0),    # g 16, d 64, ragged
    (1, 4, 1, 1, 128, 128, 0.5, 0.0),      # a one-token prompt
    (1, 8, 2, 200, 128, 0, 0.2, 0.0),      # W 0: rows with no kept key before them are 0
    (1, 8, 2, 450, 128, 1000, 0.0, 0.0),   # W > T: plain causal attention
    (1, 8, 2, 333, 128, 1, 1.0, 0.0),      # everything kept
    (1, 8, 2, 1300, 128, 128, 0.25, 0.01),  # outlier keys x8: peaked softmax
    (1, 32, 8, 2100, 128, 128, 0.25, 0.0),  # the layer's head layout
])
def test_prefill_attn(K, B, Hq, Hkv, T, d, window, keepfrac, outl):
    P = B * Hkv
    rng = np.random.default_rng(7 * T + d + window)
    keep = rng.random((P, T)) < keepfrac
    q, k, v = inputs(B, Hq, Hkv, T, d, 100 + T, outl)
    bits, idx = pack_bits(keep, tail=True), kept_list(keep)
    out = run(K, q, k, v, bits, idx, window)
    ref = oracle.prefill_attention(f64(q), f64(k), f64(v), keep.reshape(B, Hkv, T), window,
                                   oracle.sm_scale(d))
    err = check_attention(out, ref, torch.bfloat16)
    print(f"prefill B{B} Hq{Hq} Hkv{Hkv} T{T} d{d} W{window}: max-abs error {err:.2e}")
    # deterministic
    out2 = run(K, q, k, v, bits, idx, window)
    assert torch.equal(out, out2)


@pytest.mark.parametrize("d", [128, 64])
def test_prefill_attn_large_values(K, d):
    """A pair whose V holds magnitudes at and beyond 2^16 (past the fp16 range, so a
    product in fp16 would overflow): its outputs stay finite and within 2e-3 + 2^-14
    max|v| of the oracle (the error of P's ~16 significant bits scales with |v|); the
    other pair keeps the plain 2e-3 bar."""
    B, Hq, Hkv, T, window = 1, 8, 2, 900, 128
    rng = np.random.default_rng(31 + d)
    keep = rng.random((B * Hkv, T)) < 0.3
    q, k, v = inputs(B, Hq, Hkv, T, d, 4242 + d)
    big = torch.tensor([70000.0, -131072.0, 65536.0, 3.0e5], dtype=torch.bfloat16, device=DEV)
    pos = torch.tensor([5, 300, 301, 811], device=DEV)
    v[0, 1, pos, 7] = big
    bits, idx = pack_bits(keep), kept_list(keep)
    out = run(K, q, k, v, bits, idx, window)
    assert torch.isfinite(out).all()
    ref = oracle.prefill_attention(f64(q), f64(k), f64(v), keep.reshape(B, Hkv, T), window,
                                   oracle.sm_scale(d))
    g = Hq // Hkv
    err = np.abs(out.double().cpu().numpy() - ref)
    assert err[:, :g].max() <= 2e-3, err[:, :g].max()
    vmax = float(v[0, 1].abs().max())
    assert vmax >= 65536
    assert err[:, g:].max() <= 2e-3 + 2.0 ** -14 * vmax, err[:, g:].max()


@pytest.mark.parametrize("rule", ["kvzap", "dms"])
def test_prefill_attn_after_select(K, rule):
    """The selection comes from kvp_select: KVzap (tau = 0.75 quantile, R = 128, window
    = R) and DMS (tau = 0 on a biased scorer, delay w = 64, window = w)."""
    B, Hq, Hkv, T, d = 2, 16, 4, 1200, 128
    bias = W.DMS_BIAS if rule == "dms" else 0.0
    scores = W.normal((B, Hkv, T), torch.float32, 501, DEV) + bias
    s64 = f64(scores)
    if rule == "kvzap":
        tau, R = float(oracle.threshold_quantile(np_bits(scores), 0.75)), 128
        keep = s64 >= tau
    else:
        tau, R = 0.0, 64
        keep = ~oracle.dms_evict_flags(s64)
    P = B * Hkv
    bits = torch.zeros((P, (T + 31) // 32), dtype=torch.int32, device=DEV)
    idx = torch.zeros((P, T), dtype=torch.int32, device=DEV)
    cnt = torch.zeros((P,), dtype=torch.int32, device=DEV)
    ws = torch.empty(max(1, K.kvp_select_workspace_size(B, Hkv, T) // 4), dtype=torch.int32,
                     device=DEV)
    K.kvp_select(scores, T, tau, R, bits, idx, cnt, ws)
    q, k, v = inputs(B, Hq, Hkv, T, d, 601)
    out = run(K, q, k, v, bits, idx, R)
    ref = oracle.prefill_attention(f64(q), f64(k), f64(v), keep, R, oracle.sm_scale(d))
    check_attention(out, ref, torch.bfloat16)


def test_prefill_attn_layer_shape_sampled(K):
    """qwen3-8B-like layer (B 16, 32 query / 8 KV heads, d 128, T 32768), keep 0.25 at
    the scores' 0.75 quantile, R = 128: sampled output rows against the oracle, one
    row at a time (first, last, block and band edges, random)."""
    wl = W.QWEN3_8B_LAYER
    B, Hq, Hkv, T, d, R = wl.B, wl.Hq, wl.Hkv, wl.T, wl.d, W.RECENT
    scores = W.normal((B, Hkv, T), torch.float32, 701, DEV)
    tau = float(np.float32(torch.quantile(scores.double().flatten(), 0.75).item()))
    P = B * Hkv
    bits = torch.zeros((P, (T + 31) // 32), dtype=torch.int32, device=DEV)
    idx = torch.zeros((P, T), dtype=torch.int32, device=DEV)
    cnt = torch.zeros((P,), dtype=torch.int32, device=DEV)
    ws = torch.empty(max(1, K.kvp_select_workspace_size(B, Hkv, T) // 4), dtype=torch.int32,
                     device=DEV)
    K.kvp_select(scores, T, tau, R, bits, idx, cnt, ws)
    q = W.prompt_queries(wl, T, DEV)
    k, v = W.kv_dense(wl, T, DEV)
    out = run(K, q, k, v, bits, idx, R)
    assert not torch.isnan(out).any()
    rng = np.random.default_rng(5)
    rows = [(0, 0, 0), (B - 1, Hq - 1, T - 1), (3, 5, 127), (3, 5, 128), (7, 13, 31), (7, 13, 32),
            (9, 2, 191), (9, 2, 192), (11, 30, T - 33)]
    rows += [(int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(T))) for _ in range(15)]
    scale = oracle.sm_scale(d)
    g = Hq // Hkv
    worst = 0.0
    for b, hq, i in rows:
        h = hq // g
        s_row = f64(scores[b, h, : i + 1])
        vis = oracle.prefill_visible(s_row >= tau, R)[i]
        sel = np.flatnonzero(vis)
        kr = f64(k[b, h, : i + 1])[sel]
        vr = f64(v[b, h, : i + 1])[sel]
        ref = oracle.attend_one(f64(q[b, hq, i]), kr, vr, scale)
        err = float(np.abs(out[b, hq, i].double().cpu().numpy() - ref).max())
        worst = max(worst, err)
        assert err <= 2e-3, (b, hq, i, err)
    print(f"layer shape: {len(rows)} sampled rows, max-abs error {worst:.2e}")
