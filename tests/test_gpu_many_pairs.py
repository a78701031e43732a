"""Decode attention and the fused decode step on caches with more (batch, KV head) pairs
than the split's page prefix fits in a work-group's LDS (~20000 pairs, ~10000 with a
low-precision pool), through the C ABI: the prefix is then built by a plan kernel in
the workspace and read from there.  Parity with the oracle within max-abs 2e-3 (bf16 KV),
reruns bit-identical, and the fused step against the separate calls.
"""
import numpy as np
import pytest
import torch

import oracle
from kvp_testlib import check_attention, f64, read_pool, read_ring
from test_gpu_kernels import build_cache, rerun_identical, seeded, upload_selection

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_decode_attention_kvzap_amd as K
    K.load()
    return K


@pytest.mark.parametrize("B,Hq,Hkv,T,d,ring_w,demote", [
    (2600, 8, 8, 40, 64, 0, False),      # 20800 pairs, bf16 pool only
    (1300, 16, 8, 40, 64, 16, True),     # 10400 pairs with an int8 pool and a ring
])
def test_decode_attn_many_pairs(K, B, Hq, Hkv, T, d, ring_w, demote):
    P = B * Hkv
    print(f"many pairs: P={P} Hq={Hq} T={T} d={d} ring={ring_w} demote={demote}", flush=True)
    g = torch.Generator().manual_seed(P)
    keep = (torch.rand((P, T), generator=g) < 0.4).numpy()
    keep[:, T - (ring_w or 8):] = True
    keep[5, :] = False  # one pair with nothing visible: zeros
    if ring_w:
        keep[5, T - ring_w:] = True
    k, v, kv, ring = build_cache(K, B, Hkv, T, d, torch.bfloat16, keep, ring_w, seed=81,
                                 demote=demote)
    q = seeded((B, Hq, d), 84, torch.bfloat16)
    out = torch.full((B, Hq, d), float("nan"), device=DEV)
    ws = K.decode_attn_workspace(B, Hq, kv)
    K.kvp_decode_attn(q, kv, ring, K.sm_scale(d), out, ws)
    torch.cuda.synchronize()
    if demote:
        ref = oracle.beacon_decode_attention(f64(q), f64(k), f64(v), keep.reshape(B, Hkv, T),
                                             oracle.sm_scale(d), bits=8)
    else:
        ref = oracle.decode_attention(f64(q), f64(k), f64(v), keep.reshape(B, Hkv, T),
                                      oracle.sm_scale(d))
    err = check_attention(out, ref, torch.bfloat16)
    print(f"many pairs: max-abs error {err:.2e}")
    rerun_identical(K, q, kv, ring, d, out, ws)


def test_fused_step_many_pairs(K):
    """kvp_decode_step with given scores on 20800 pairs against kvp_step_delayed_dev then
    kvp_decode_attn: outputs within fp32 rounding, rings, lengths and counters identical,
    and the pools of sampled pairs identical row for row, over a few steps that turn ring
    slots over."""
    B, Hkv, g, d, w, T0, steps, tau = 2600, 8, 1, 64, 16, 40, 4, 0.0
    P, Hq = B * Hkv, Hkv * g
    total = T0 + steps
    k_all = seeded((B, Hkv, total, d), 311, torch.bfloat16)
    v_all = seeded((B, Hkv, total, d), 312, torch.bfloat16)
    s_all = seeded((B, Hkv, total), 313) - 0.3
    q_all = seeded((steps, B, Hq, d), 315, torch.bfloat16)
    keep0 = oracle.keep_mask(f64(s_all[..., :T0]).reshape(P, T0), tau, w)
    idx, cnt = upload_selection(keep0)
    maxpp = total // 16 + 2
    caches = []
    for _ in range(2):
        kv = K.PagedKV.allocate(P, d, P * maxpp, maxpp, torch.bfloat16, DEV, poison=True)
        ring = K.Ring.allocate(P, w, d, torch.bfloat16, DEV, poison=True)
        K.kvp_compact(k_all[:, :, :T0].contiguous(), v_all[:, :, :T0].contiguous(), idx, cnt, kv,
                      torch.empty(K.kvp_compact_workspace_size(B, Hkv) // 4, dtype=torch.int32,
                                  device=DEV),
                      ring=ring, scores=s_all[..., :T0].contiguous())
        taud = torch.full((1,), tau, dtype=torch.float32, device=DEV)
        pos = torch.tensor([T0, 0], dtype=torch.int32, device=DEV)
        caches.append((kv, ring, taud, pos))
    (kvF, ringF, tauF, posF), (kvS, ringS, tauS, posS) = caches
    ws_f = K.decode_step_workspace(None, B, Hq, kvF)
    ws_a = K.decode_attn_workspace(B, Hq, kvS)
    outF = torch.empty((B, Hq, d), device=DEV)
    outS = torch.empty((B, Hq, d), device=DEV)
    sample = [0, 1, 777, 5000, 12345, P - 1]
    for i in range(steps):
        p = T0 + i
        k_new = k_all[:, :, p].contiguous()
        v_new = v_all[:, :, p].contiguous()
        s_in = s_all[:, :, p].contiguous()
        q = q_all[i]
        outF.fill_(float("nan"))
        K.kvp_decode_step(None, None, kvF, ringF, k_new, v_new, tauF, posF, q, K.sm_scale(d), outF,
                          ws_f, s_in=s_in)
        K.kvp_step_delayed(kvS, ringS, k_new, v_new, s_in, tauS, posS)
        K.kvp_decode_attn(q, kvS, ringS, K.sm_scale(d), outS, ws_a)
        torch.cuda.synchronize()
        assert int(posF[0]) == p + 1 and int(posF[1]) == 0
        assert torch.equal(kvF.length, kvS.length), i
        for n, t in ringF.tensors.items():
            iv = {1: torch.int8, 2: torch.int16, 4: torch.int32}[t.element_size()]
            assert torch.equal(t.view(iv), ringS.tensors[n].view(iv)), ("ring", n, i)
        for pr in sample:
            for a, b in zip(read_pool(kvF, pr), read_pool(kvS, pr)):
                assert np.array_equal(a, b), ("pool", pr, i)
        assert not torch.isnan(outF).any()
        assert (outF - outS).abs().max().item() <= 1e-4, i
    assert K.kvp_check(kvF) == 0 and K.kvp_check(kvS) == 0
    for pr in sample:
        assert len(read_ring(ringF, pr)[0]) == min(w, total)
