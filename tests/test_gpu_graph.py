"""The decode step (score the new token -> delayed step -> attention) captured once in a
HIP graph and replayed step after step: every per-step value (threshold, position) is
device-resident, so each replay must produce exactly the eager step's output and
state.  Replays are interleaved with eager work (input refills, host syncs, unrelated
torch kernels) and every replay is checked."""
import numpy as np
import pytest
import torch

import kvp_workloads as W
from kvp_testlib import read_pool, read_ring

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_decode_attention_kvzap_amd as K
    K.load()
    return K


@pytest.mark.parametrize("scorer", ["linear", "mlp"])
def test_graph_replayed_decode_steps_match_eager(K, scorer):
    from sparse_decode_attention_kvzap_amd.pipeline import PrunedKVCache
    wl = W.DMS_DELAYED.scaled(B=2, H=512, Hq=8, Hkv=2, prompt=300, steps=40, w=32, R=32,
                              T=340, scorer=scorer)
    S, P0 = wl.steps, wl.prompt
    sw = W.scorer_weights(wl, DEV)
    scorer_obj = (K.Scorer(K.KVP_SCORER_LINEAR, sw.W1, sw.b1) if scorer == "linear" else
                  K.Scorer(K.KVP_SCORER_MLP, sw.W1, sw.b1, sw.W2, sw.b2))
    hidden = W.hidden_states(wl, P0, DEV)
    kd, vd = W.kv_dense(wl, P0, DEV)
    ins = [W.step_inputs(wl, i, DEV) for i in range(S)]
    cache = PrunedKVCache(wl.B, wl.Hkv, wl.Hq, wl.d, P0 + S, wl.kv_dtype, scorer_obj, wl.w, 0.0,
                          device=DEV, max_prompt=P0)
    hb, kb, vb, qb = (torch.empty_like(x) for x in ins[0])

    def prefill():
        cache.set_tau(0.0)
        cache.prefill(hidden, kd, vd)
        cache.set_position(P0)
        cache.tau = cache.tau_dev

    def feed(i):
        for dst, src in zip((hb, kb, vb, qb), ins[i]):
            dst.copy_(src)

    def state():
        return [np.sort(np.concatenate([read_pool(cache.kv, p)[0], read_ring(cache.ring, p)[0]]))
                for p in range(cache.P)]

    prefill()
    eager_out, eager_state = [], []
    for i in range(S):
        feed(i)
        cache.step(hb, kb, vb, qb)
        eager_out.append(cache.out.clone())
        if i % 8 == 7:
            eager_state.append(state())

    prefill()
    feed(0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        cache.step(hb, kb, vb, qb)
    torch.cuda.synchronize()
    prefill()  # capture ran nothing; start from a fresh prompt state
    junk = torch.randn(1 << 20, device=DEV)
    for i in range(S):
        feed(i)
        graph.replay()
        junk.mul_(1.0001).add_(0.5)  # unrelated eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(cache.out, eager_out[i]), f"replay {i}"
        if i % 8 == 7:
            got = state()
            for a, b in zip(got, eager_state[i // 8]):
                assert np.array_equal(a, b), f"state after replay {i}"
    assert cache.pos_dev.tolist() == [P0 + S, 0]
    assert K.kvp_check(cache.kv) == 0


@pytest.mark.parametrize("scorer", ["linear", "mlp"])
def test_graph_of_several_decode_steps_matches_eager(K, scorer):
    """Four consecutive decode steps captured as one graph (each step reading its own slot
    of fixed input buffers, its output copied out inside the graph), replayed ten times
    with the inputs of the next four steps refilled before each replay: every step's
    output and the cache state match eager steps bit for bit."""
    from sparse_decode_attention_kvzap_amd.pipeline import PrunedKVCache
    wl = W.DMS_DELAYED.scaled(B=2, H=512, Hq=8, Hkv=2, prompt=300, steps=40, w=32, R=32,
                              T=340, scorer=scorer)
    S, P0, G = wl.steps, wl.prompt, 4
    sw = W.scorer_weights(wl, DEV)
    scorer_obj = (K.Scorer(K.KVP_SCORER_LINEAR, sw.W1, sw.b1) if scorer == "linear" else
                  K.Scorer(K.KVP_SCORER_MLP, sw.W1, sw.b1, sw.W2, sw.b2))
    hidden = W.hidden_states(wl, P0, DEV)
    kd, vd = W.kv_dense(wl, P0, DEV)
    ins = [W.step_inputs(wl, i, DEV) for i in range(S)]
    slabs = [torch.stack([ins[i][t] for i in range(S)]) for t in range(4)]  # [S, ...] per input
    bufs = [torch.empty((G,) + x.shape, dtype=x.dtype, device=DEV) for x in ins[0]]
    cache = PrunedKVCache(wl.B, wl.Hkv, wl.Hq, wl.d, P0 + S, wl.kv_dtype, scorer_obj, wl.w, 0.0,
                          device=DEV, max_prompt=P0)
    outs = torch.empty((G,) + tuple(cache.out.shape), dtype=cache.out.dtype, device=DEV)

    def prefill():
        cache.set_tau(0.0)
        cache.prefill(hidden, kd, vd)
        cache.set_position(P0)
        cache.tau = cache.tau_dev

    def state():
        return [np.sort(np.concatenate([read_pool(cache.kv, p)[0], read_ring(cache.ring, p)[0]]))
                for p in range(cache.P)]

    prefill()
    eager_out, eager_state = [], []
    for i in range(S):
        cache.step(*ins[i])
        eager_out.append(cache.out.clone())
        if i % G == G - 1:
            eager_state.append(state())

    prefill()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for k in range(G):
            cache.step(*(b[k] for b in bufs))
            outs[k].copy_(cache.out)
    torch.cuda.synchronize()
    prefill()  # capture ran nothing; start from a fresh prompt state
    junk = torch.randn(1 << 20, device=DEV)
    for r in range(S // G):
        for b, s in zip(bufs, slabs):
            b.copy_(s[r * G:(r + 1) * G])
        graph.replay()
        junk.mul_(1.0001).add_(0.5)  # unrelated eager work between replays
        torch.cuda.synchronize()
        for k in range(G):
            assert torch.equal(outs[k], eager_out[r * G + k]), f"replay {r} step {k}"
        for a, b in zip(state(), eager_state[r]):
            assert np.array_equal(a, b), f"state after replay {r}"
    assert cache.pos_dev.tolist() == [P0 + S, 0]
    assert K.kvp_check(cache.kv) == 0
