"""On-device threshold calibration (kvp_threshold) and the device-tau variants of
select and the delayed step, through the C ABI.

kvp_threshold computes, on the device, the q-quantile of the GPU's own fp32 scores
with numpy's "linear" rule; the oracle's threshold_quantile applied to the same fp32
values (exactly widened to fp64) is the reference, compared exactly (fp32 equality;
both NaN for inputs holding a NaN).
"""
import numpy as np
import pytest
import torch

import oracle
from kvp_testlib import read_pool, read_ring

pytestmark = pytest.mark.gpu
DEV = "cuda"
QS = [0.0, 1e-7, 0.1, 0.25, 0.5, 0.75, 0.9, 0.999999, 1.0]


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_decode_attention_kvzap_amd as K
    K.load()
    return K


def gpu_tau(K, scores, T, q):
    ws = torch.empty(K.kvp_threshold_workspace_size() // 4 + 1, dtype=torch.int32, device=DEV)
    ws.fill_(-1)  # scratch, any contents
    tau = torch.full((1,), 12345.0, device=DEV)
    K.kvp_threshold(scores, T, q, tau, ws)
    return np.float32(tau.item())


def ref_tau(scores, T, q):
    s = scores[:, :, :T].detach().cpu().numpy().astype(np.float64)
    return oracle.threshold_quantile(s, q)


def same(a, b):
    return (np.isnan(a) and np.isnan(b)) or a == b


def scores_of(kind, shape, seed, ld):
    B, Hkv, T = shape
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    if kind == "normal":
        x = torch.randn((B, Hkv, T), generator=g)
    elif kind == "ties":  # few distinct values, many equal ranks
        x = torch.randint(-3, 4, (B, Hkv, T), generator=g).float() * 0.5
    elif kind == "signed_zeros":
        x = torch.randint(-1, 2, (B, Hkv, T), generator=g).float() * 0.0
        x[..., ::3] = -0.0
        x[..., 1::7] = 1.5
    elif kind == "wide":  # magnitudes across the exponent range, and infinities
        x = torch.randn((B, Hkv, T), generator=g) * torch.exp2(
            torch.randint(-120, 120, (B, Hkv, T), generator=g).float())
        x.view(-1)[:: max(1, x.numel() // 5)] = float("inf")
        x.view(-1)[1:: max(1, x.numel() // 7)] = float("-inf")
    else:
        raise ValueError(kind)
    out = torch.full((B, Hkv, ld), float("nan"))  # padding past T must be ignored
    out[..., :T] = x
    return out.to(DEV)


@pytest.mark.parametrize("shape,ld", [((1, 1, 1), 1), ((1, 2, 7), 9), ((2, 3, 1000), 1003),
                                      ((3, 5, 4097), 4100), ((2, 8, 12289), 12289)])
@pytest.mark.parametrize("kind", ["normal", "ties", "signed_zeros", "wide"])
def test_threshold_matches_quantile(K, shape, ld, kind):
    sc = scores_of(kind, shape, 1000 * ["normal", "ties", "signed_zeros", "wide"].index(kind)
                   + shape[2], ld)
    T = shape[2]
    for q in QS:
        g, r = gpu_tau(K, sc, T, q), ref_tau(sc, T, q)
        assert same(g, r), (q, g, r)


def test_threshold_full_size_scores(K):
    """The 16 x 8 x 32767 score matrix of the benchmarked layer (normal scores)."""
    sc = scores_of("normal", (16, 8, 32767), 7, 32767)
    for q in (0.5, 0.75, 0.9):
        g, r = gpu_tau(K, sc, 32767, q), ref_tau(sc, 32767, q)
        assert same(g, r), (q, g, r)


def test_threshold_nan_gives_nan(K):
    sc = scores_of("normal", (2, 2, 300), 5, 300)
    sc[1, 0, 17] = float("nan")
    assert np.isnan(gpu_tau(K, sc, 300, 0.5))
    assert np.isnan(ref_tau(sc, 300, 0.5))


def test_threshold_repeated_calls_reuse_workspace(K):
    ws = torch.empty(K.kvp_threshold_workspace_size() // 4 + 1, dtype=torch.int32, device=DEV)
    tau = torch.zeros(1, device=DEV)
    for i, (shape, q) in enumerate([((4, 8, 5000), 0.75), ((1, 1, 10), 0.3), ((4, 8, 5000), 0.1)]):
        sc = scores_of("normal", shape, 40 + i, shape[2])
        K.kvp_threshold(sc, shape[2], q, tau, ws)
        assert same(np.float32(tau.item()), ref_tau(sc, shape[2], q))


def test_select_and_step_with_device_tau(K):
    """kvp_select_dev_tau / kvp_step_delayed_dev (device tau and position) give
    bit-identical results to the host-argument calls with the same values."""
    B, Hkv, T, d, w = 2, 4, 3000, 128, 64
    P = B * Hkv
    sc = scores_of("normal", (B, Hkv, T), 11, T)
    tau_dev = torch.zeros(1, device=DEV)
    ws_t = torch.empty(K.kvp_threshold_workspace_size() // 4 + 1, dtype=torch.int32, device=DEV)
    K.kvp_threshold(sc, T, 0.7, tau_dev, ws_t)
    tau = float(tau_dev.item())
    res = []
    for t in (tau, tau_dev):
        bits = torch.zeros((P, (T + 31) // 32), dtype=torch.int32, device=DEV)
        idx = torch.zeros((P, T), dtype=torch.int32, device=DEV)
        cnt = torch.zeros((P,), dtype=torch.int32, device=DEV)
        ws = torch.empty(K.kvp_select_workspace_size(B, Hkv, T) // 4 + 1, dtype=torch.int32,
                         device=DEV)
        K.kvp_select(sc, T, t, 128, bits, idx, cnt, ws)
        res.append((bits.cpu(), idx.cpu(), cnt.cpu()))
    for a, b in zip(*res):
        assert torch.equal(a, b)
    # delayed step: same ring/pool evolution for host and device tau
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    ks = torch.randn((B, Hkv, 3 * w, d), generator=g, device=DEV).to(torch.bfloat16)
    vs = torch.randn((B, Hkv, 3 * w, d), generator=g, device=DEV).to(torch.bfloat16)
    ss = torch.randn((B, Hkv, 3 * w), generator=g, device=DEV)
    # the device variant reads the position from device memory and advances it itself
    pos_dev = torch.tensor([0, 0], dtype=torch.int32, device=DEV)
    states = []
    for dev_side in (False, True):
        maxpp = 3 * w // 16 + 2
        kv = K.PagedKV.allocate(P, d, P * maxpp, maxpp, torch.bfloat16, DEV, poison=True)
        ring = K.Ring.allocate(P, w, d, torch.bfloat16, DEV, poison=True)
        K.kvp_reset(kv, ring)
        for p in range(3 * w):
            args = (kv, ring, ks[:, :, p].contiguous(), vs[:, :, p].contiguous(),
                    ss[:, :, p].contiguous())
            if dev_side:
                K.kvp_step_delayed(*args, tau_dev, pos_dev)
            else:
                K.kvp_step_delayed(*args, tau, p)
        states.append([np.concatenate([read_pool(kv, pr)[0], read_ring(ring, pr)[0]])
                       for pr in range(P)])
        if dev_side:
            assert pos_dev.tolist() == [3 * w, 0]
    for a, b in zip(*states):
        assert np.array_equal(np.sort(a), np.sort(b))
