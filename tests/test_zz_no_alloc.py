"""kvp_decode_attn_noalloc (fixed per-GPU scratch, no workspace argument) against
kvp_decode_attn (caller's workspace) through the C ABI.

Both run the same kernels, so the outputs must agree bit for bit; each is also held to
the oracle at the bf16-KV / fp32-KV tolerances.  Two calls in a row, the second on a
smaller cache, so the second runs over the scratch the first one left behind.
"""
import numpy as np
import pytest
import torch

import oracle
from kvp_testlib import check_attention, f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_decode_attention_kvzap_amd as K
    K.load()
    return K


def seeded(shape, seed, dtype=torch.float32):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV).to(dtype)


def make_case(K, B, Hq, Hkv, T, d, dtype, ring_w, keepfrac, seed, bits=0):
    """A compacted paged cache (+ ring, + optional low-precision pool) and a query."""
    P = B * Hkv
    g = torch.Generator().manual_seed(seed)
    keep = (torch.rand((P, T), generator=g) < keepfrac).numpy()
    if ring_w:
        keep[:, T - ring_w:] = True
    k = seeded((B, Hkv, T, d), seed, dtype)
    v = seeded((B, Hkv, T, d), seed + 1, dtype)
    s = seeded((B, Hkv, T), seed + 2)
    idx = np.zeros((P, T), np.int32)
    cnt = np.zeros(P, np.int32)
    for p in range(P):
        kk, ee = oracle.partition_indices(keep[p])
        idx[p] = np.concatenate([kk, ee])
        cnt[p] = len(kk)
    idx_d, cnt_d = torch.from_numpy(idx).to(DEV), torch.from_numpy(cnt).to(DEV)
    maxpp = T // 16 + 2
    kw = dict(num_pages8=P * maxpp, max_pages8_per_pair=maxpp, lp_bits=bits) if bits else {}
    kv = K.PagedKV.allocate(P, d, P * maxpp, maxpp, dtype, DEV, poison=True, **kw)
    ring = K.Ring.allocate(P, ring_w, d, dtype, DEV, poison=True) if ring_w else None
    ws = torch.empty(K.kvp_compact_workspace_size(B, Hkv) // 4, dtype=torch.int32, device=DEV)
    K.kvp_compact(k, v, idx_d, cnt_d, kv, ws, ring=ring, scores=s,
                  mode=K.KVP_COMPACT_DEMOTE_INT8 if bits else K.KVP_COMPACT_EVICT)
    q = seeded((B, Hq, d), seed + 3, dtype)
    if bits:
        ref = oracle.beacon_decode_attention(f64(q), f64(k), f64(v), keep.reshape(B, Hkv, T),
                                             oracle.sm_scale(d), bits=bits)
    else:
        ref = oracle.decode_attention(f64(q), f64(k), f64(v), keep.reshape(B, Hkv, T),
                                      oracle.sm_scale(d))
    return q, kv, ring, ref


def run_both(K, q, kv, ring, d):
    B, Hq, _ = q.shape
    out_ws = torch.full((B, Hq, d), float("nan"), device=DEV)
    ws = K.decode_attn_workspace(B, Hq, kv)
    K.kvp_decode_attn(q, kv, ring, K.sm_scale(d), out_ws, ws)
    out_na = torch.full((B, Hq, d), float("nan"), device=DEV)
    K.kvp_decode_attn_noalloc(q, kv, ring, K.sm_scale(d), out_na)
    torch.cuda.synchronize()
    assert K.kvp_check(kv) == 0
    return out_ws, out_na


@pytest.mark.parametrize("first,second", [
    # (B, Hq, Hkv, T, d, dtype, ring_w, keepfrac, seed, bits)
    ((4, 32, 8, 3000, 128, torch.bfloat16, 128, 0.3, 11, 0),
     (1, 8, 2, 500, 128, torch.bfloat16, 128, 0.5, 12, 0)),
    ((2, 16, 2, 2500, 128, torch.bfloat16, 128, 0.15, 21, 4),
     (1, 4, 2, 700, 64, torch.float32, 64, 0.4, 22, 0)),
])
def test_noalloc_matches_workspace_entry_point(K, first, second):
    for case in (first, second):
        B, Hq, Hkv, T, d, dtype, ring_w, keepfrac, seed, bits = case
        print(f"noalloc case B={B} Hq={Hq} Hkv={Hkv} T={T} d={d} {dtype} ring={ring_w} "
              f"bits={bits}", flush=True)
        q, kv, ring, ref = make_case(K, B, Hq, Hkv, T, d, dtype, ring_w, keepfrac, seed, bits)
        out_ws, out_na = run_both(K, q, kv, ring, d)
        assert torch.equal(out_ws, out_na)
        check_attention(out_na, ref, dtype)


def test_noalloc_rejects_oversize(K):
    """A launch whose workspace would exceed the fixed scratch is refused on the host
    (KVP_E_WORKSPACE) before anything is enqueued."""
    B, Hkv, g, d = 125, 16, 16, 128
    P = B * Hkv
    need = K.kvp_decode_attn_workspace_size(B, Hkv * g, P, d)
    assert need > K.KVP_NOALLOC_SCRATCH_BYTES
    kv = K.PagedKV.allocate(P, d, 16, 1, torch.bfloat16, DEV, poison=False)
    q = torch.zeros((B, Hkv * g, d), dtype=torch.bfloat16, device=DEV)
    out = torch.zeros((B, Hkv * g, d), device=DEV)
    with pytest.raises(K.KvpError) as e:
        K.kvp_decode_attn_noalloc(q, kv, None, K.sm_scale(d), out)
    assert e.value.status == 3
