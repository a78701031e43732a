"""kvp_decode_step (the delayed step folded into the decode attention) against the two
separate calls it replaces, through the C ABI.

Two caches are compacted from the same prompt and driven side by side: one by
kvp_decode_step, the other by the delayed step (kvp_score_step_delayed, or
kvp_step_delayed_dev with given scores) followed by kvp_decode_attn.  After every step the
caches must hold the same logical content bit for bit (rings, counters, each pair's pool
rows; physical page ids may differ), the stored scores must be identical, and the outputs
must agree to fp32 rounding (the fused attention groups the tokens differently: the token
leaving the ring is read from its ring slot, the new token from its own page).  The
outputs are also held to the oracle over the visible set within max-abs 2e-3.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from kvp_testlib import check_attention, f64, read_pool, read_ring, visible_positions

pytestmark = pytest.mark.gpu
DEV = "cuda"
FUSED_VS_SEPARATE_ATOL = 1e-4  # same token set and values, another summation order


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_decode_attention_kvzap_amd as K
    K.load()
    return K


def seeded(shape, seed, dtype=torch.float32, scale=1.0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV) * scale).to(dtype)


def upload_selection(keep: np.ndarray):
    P, T = keep.shape
    idx = np.zeros((P, T), np.int32)
    cnt = np.zeros(P, np.int32)
    for p in range(P):
        k, e = oracle.partition_indices(keep[p])
        idx[p] = np.concatenate([k, e])
        cnt[p] = len(k)
    return torch.from_numpy(idx).to(DEV), torch.from_numpy(cnt).to(DEV)


def same_cache(kvA, ringA, kvB, ringB):
    for n, t in ringA.tensors.items():
        iv = {1: torch.int8, 2: torch.int16, 4: torch.int32}[t.element_size()]
        assert torch.equal(t.view(iv), ringB.tensors[n].view(iv)), "ring " + n
    for n in ("length", "page_top", "err"):
        assert torch.equal(kvA.tensors[n], kvB.tensors[n]), n
    for pr in range(kvA.c.num_pairs):
        for a, b in zip(read_pool(kvA, pr), read_pool(kvB, pr)):
            assert np.array_equal(a, b), ("pool", pr)


def make_scorer(K, kind, H, inner, Hkv):
    """kind: "linear" / "mlp" (with biases), "linear_nobias" / "mlp_nobias", or "given"."""
    bias = not kind.endswith("_nobias")
    if kind.startswith("linear"):
        W1 = seeded((Hkv, H), 201, torch.bfloat16, scale=1.0 / math.sqrt(H))
        b1 = seeded((Hkv,), 202) * 0.1 - 1.0 if bias else None
        return K.Scorer(K.KVP_SCORER_LINEAR, W1, b1)
    if kind.startswith("mlp"):
        W1 = seeded((inner, H), 201, torch.bfloat16, scale=1.0 / math.sqrt(H))
        b1 = seeded((inner,), 202, scale=0.5) if bias else None
        W2 = seeded((Hkv, inner), 203, scale=1.0 / math.sqrt(inner))
        b2 = seeded((Hkv,), 204) * 0.1 - 0.3 if bias else None
        return K.Scorer(K.KVP_SCORER_MLP, W1, b1, W2, b2)
    return None  # scores given


@pytest.mark.parametrize("kind,B,Hkv,g,d,w,T0,steps,tau,H,inner,empty", [
    ("given", 2, 3, 4, 128, 64, 300, 80, 0.0, 0, 0, False),      # DMS-style tau = 0
    ("linear", 3, 4, 2, 128, 32, 200, 50, 0.2, 1024, 0, False),   # scored inside, tau > 0
    ("mlp", 2, 4, 4, 128, 64, 250, 70, 0.0, 1024, 512, False),   # split-K MLP partials
    ("given", 4, 2, 8, 64, 48, 150, 60, 0.3, 0, 0, True),        # d 64, pairs with empty pools
    ("linear", 1, 8, 1, 64, 128, 400, 40, -0.1, 512, 0, False),  # g 1, ring of 128
    # MLP slices taken inside the attention kernel: 40 tokens (three 16-token tiles) and
    # 32 x 64 = 2048 slices of H 8192 / inner 1024, more than its waves (several each)
    ("mlp", 40, 2, 2, 64, 32, 120, 20, 0.0, 8192, 1024, False),
    ("mlp", 64, 1, 4, 128, 48, 160, 24, -0.2, 2048, 256, False),  # 64 tokens, inner 256
    ("linear_nobias", 2, 2, 16, 128, 32, 180, 40, 0.1, 512, 0, False),  # g 16, no bias
    # g 16, d 64, no biases, inner 768: three first-layer slices, three 256-unit chunks
    ("mlp_nobias", 3, 2, 16, 64, 32, 140, 30, 0.0, 768, 768, False),
])
def test_fused_step_matches_separate_calls(K, kind, B, Hkv, g, d, w, T0, steps, tau, H, inner,
                                           empty):
    P, Hq = B * Hkv, Hkv * g
    total = T0 + steps
    print(f"decode_step case {kind} B={B} Hkv={Hkv} g={g} d={d} w={w} T0={T0} steps={steps}",
          flush=True)
    sc = make_scorer(K, kind, H, inner, Hkv)
    k_all = seeded((B, Hkv, total, d), 211, torch.bfloat16)
    v_all = seeded((B, Hkv, total, d), 212, torch.bfloat16)
    s_all = seeded((B, Hkv, total), 213) - 0.9  # prompt scores, and given step scores
    x_all = seeded((steps, B, 1, max(H, 8)), 214, torch.bfloat16)
    q_all = seeded((steps, B, Hq, d), 215, torch.bfloat16)
    keep0 = oracle.keep_mask(f64(s_all[..., :T0]).reshape(P, T0), tau, w)
    if empty:  # pairs 0 and 3 keep nothing outside the ring
        keep0[0, :T0 - w] = False
        keep0[3, :T0 - w] = False
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
    same_cache(kvF, ringF, kvS, ringS)
    ws_f = K.decode_step_workspace(sc, B, Hq, kvF)
    ws_a = K.decode_attn_workspace(B, Hq, kvS)
    ws_s = torch.empty(max(1, K.kvp_score_workspace_size(sc, B, 1) // 4) if sc else 1,
                       dtype=torch.float32, device=DEV)
    outF = torch.empty((B, Hq, d), device=DEV)
    outS = torch.empty((B, Hq, d), device=DEV)
    sF = torch.full((P,), float("nan"), device=DEV)
    sS = torch.full((P,), float("nan"), device=DEV)
    kf, vf = f64(k_all), f64(v_all)
    for i in range(steps):
        p = T0 + i
        k_new = k_all[:, :, p].contiguous()
        v_new = v_all[:, :, p].contiguous()
        q = q_all[i]
        outF.fill_(float("nan"))
        if sc is None:
            s_in = s_all[:, :, p].contiguous()
            K.kvp_decode_step(None, None, kvF, ringF, k_new, v_new, tauF, posF, q, K.sm_scale(d),
                              outF, ws_f, s_in=s_in)
            K.kvp_step_delayed(kvS, ringS, k_new, v_new, s_in, tauS, posS)
        else:
            K.kvp_decode_step(sc, x_all[i], kvF, ringF, k_new, v_new, tauF, posF, q, K.sm_scale(d),
                              outF, ws_f, s_out=sF)
            K.kvp_score_step_delayed(sc, x_all[i], kvS, ringS, k_new, v_new, tauS, posS, sS, ws_s)
        K.kvp_decode_attn(q, kvS, ringS, K.sm_scale(d), outS, ws_a)
        assert int(posF[0]) == p + 1 and int(posF[1]) == 0
        same_cache(kvF, ringF, kvS, ringS)
        if sc is not None:
            assert torch.equal(sF, sS), i
        diff = (outF - outS).abs().max().item()
        assert diff <= FUSED_VS_SEPARATE_ATOL, (i, diff)
        if i in (0, 1, w - 1, w, w + 1, steps - 1) or i % 16 == 0:
            vis = np.zeros((P, p + 1), bool)
            for pr in range(P):
                vis[pr, visible_positions(kvF, ringF, pr)] = True
            ref = oracle.decode_attention(f64(q), kf[:, :, :p + 1], vf[:, :, :p + 1],
                                          vis.reshape(B, Hkv, p + 1), oracle.sm_scale(d))
            check_attention(outF, ref, torch.bfloat16)
    assert K.kvp_check(kvF) == 0
    # the ring slot turned over at every step and the pools grew only by retained tokens
    for pr in range(P):
        assert len(read_ring(ringF, pr)[0]) == min(w, total)


def test_fused_step_graph_replay_is_bit_exact(K):
    """The fused step captured once and replayed reproduces the eager fused steps bit for
    bit (outputs and cache), with eager work and synchronisations between replays."""
    B, Hkv, g, d, w, T0, steps = 2, 4, 4, 128, 32, 300, 40
    P, Hq = B * Hkv, Hkv * g
    total = T0 + steps
    sc = make_scorer(K, "linear", 512, 0, Hkv)
    k_all = seeded((B, Hkv, total, d), 221, torch.bfloat16)
    v_all = seeded((B, Hkv, total, d), 222, torch.bfloat16)
    s0 = seeded((B, Hkv, T0), 223) - 0.9
    x_all = seeded((steps, B, 1, 512), 224, torch.bfloat16)
    q_all = seeded((steps, B, Hq, d), 225, torch.bfloat16)
    keep0 = oracle.keep_mask(f64(s0).reshape(P, T0), 0.0, w)
    idx, cnt = upload_selection(keep0)
    maxpp = total // 16 + 2
    kv = K.PagedKV.allocate(P, d, P * maxpp, maxpp, torch.bfloat16, DEV, poison=True)
    ring = K.Ring.allocate(P, w, d, torch.bfloat16, DEV, poison=True)
    taud = torch.zeros(1, dtype=torch.float32, device=DEV)
    pos = torch.zeros(2, dtype=torch.int32, device=DEV)
    ws = K.decode_step_workspace(sc, B, Hq, kv)
    cws = torch.empty(K.kvp_compact_workspace_size(B, Hkv) // 4, dtype=torch.int32, device=DEV)
    xb, kb, vb, qb = (torch.empty_like(t) for t in (x_all[0], k_all[:, :, 0].contiguous(),
                                                     v_all[:, :, 0].contiguous(), q_all[0]))
    out = torch.empty((B, Hq, d), device=DEV)

    def prefill():
        K.kvp_compact(k_all[:, :, :T0].contiguous(), v_all[:, :, :T0].contiguous(), idx, cnt, kv,
                      cws, ring=ring, scores=s0.contiguous())
        pos.copy_(torch.tensor([T0, 0], dtype=torch.int32))

    def feed(i):
        xb.copy_(x_all[i])
        kb.copy_(k_all[:, :, T0 + i])
        vb.copy_(v_all[:, :, T0 + i])
        qb.copy_(q_all[i])

    def step(stream=None):
        K.kvp_decode_step(sc, xb, kv, ring, kb, vb, taud, pos, qb, K.sm_scale(d), out, ws,
                          stream=stream)

    prefill()
    eager = []
    for i in range(steps):
        feed(i)
        step()
        eager.append(out.clone())
    final = [t.clone() for t in (kv.length, ring.pos, ring.score, ring.k.view(torch.int16))]
    prefill()
    feed(0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step(side)
    torch.cuda.synchronize()
    prefill()
    junk = torch.randn(1 << 20, device=DEV)
    for i in range(steps):
        feed(i)
        graph.replay()
        junk.mul_(1.0001).add_(0.5)
        torch.cuda.synchronize()
        assert torch.equal(out, eager[i]), i
    for a, b in zip(final, (kv.length, ring.pos, ring.score, ring.k.view(torch.int16))):
        assert torch.equal(a, b)
    assert int(pos[0]) == total and int(pos[1]) == 0
    assert K.kvp_check(kv) == 0


def test_fused_step_argument_errors(K):
    """Requests the fused call does not take are refused on the host, before any launch."""
    B, Hkv, d, w = 1, 2, 128, 32
    P = B * Hkv
    q = torch.zeros((B, 4, d), dtype=torch.bfloat16, device=DEV)
    out = torch.zeros((B, 4, d), device=DEV)
    kn = torch.zeros((B, Hkv, d), dtype=torch.bfloat16, device=DEV)
    taud = torch.zeros(1, device=DEV)
    pos = torch.zeros(2, dtype=torch.int32, device=DEV)
    s_in = torch.zeros(P, device=DEV)
    kv8 = K.PagedKV.allocate(P, d, 8, 4, torch.bfloat16, DEV, num_pages8=8, max_pages8_per_pair=4)
    ring = K.Ring.allocate(P, w, d, torch.bfloat16, DEV)
    ws = K.decode_step_workspace(None, B, 4, kv8)
    with pytest.raises(K.KvpError) as e:  # low-precision pool: separate calls only
        K.kvp_decode_step(None, None, kv8, ring, kn, kn, taud, pos, q, 0.1, out, ws, s_in=s_in)
    assert e.value.status == 6
    kv = K.PagedKV.allocate(P, d, 8, 4, torch.bfloat16, DEV)
    with pytest.raises(K.KvpError) as e:  # a ring is required
        K.kvp_decode_step(None, None, kv, None, kn, kn, taud, pos, q, 0.1, out, ws, s_in=s_in)
    assert e.value.status == 1
    kvf = K.PagedKV.allocate(P, d, 8, 4, torch.float32, DEV)
    ringf = K.Ring.allocate(P, w, d, torch.float32, DEV)
    with pytest.raises(K.KvpError) as e:  # fp32 cache: separate calls only
        K.kvp_decode_step(None, None, kvf, ringf, kn.float(), kn.float(), taud, pos, q.float(), 0.1,
                          out, ws, s_in=s_in)
    assert e.value.status == 6
    with pytest.raises(K.KvpError) as e:  # workspace too small
        K.kvp_decode_step(None, None, kv, ring, kn, kn, taud, pos, q, 0.1, out, ws[:4], s_in=s_in)
    assert e.value.status == 3
    assert int(pos[0]) == 0  # nothing ran
