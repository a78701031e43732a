"""Helpers shared by the tests: bit-exact host copies for the oracle, logical read-back
of the paged cache, and the comparison rules (band around the threshold, attention
tolerances).  No method arithmetic lives here beyond what the comparisons need."""
from __future__ import annotations

import numpy as np
import torch

import oracle

BAND = 1e-4           # scores within this distance of tau are reported and excluded
ATOL_BF16 = 2e-3      # max-abs error of attention outputs with bf16 KV
RTOL_F32 = 1e-5       # per-vector relative error of attention outputs with fp32 KV


def np_bits(t: torch.Tensor) -> np.ndarray:
    """Exact host copy: bf16 -> uint16 bit patterns, others as their numpy dtype."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f64(t: torch.Tensor) -> np.ndarray:
    return oracle.as_f64(np_bits(t))


def unpack_bits(bits: torch.Tensor, T: int) -> np.ndarray:
    """keep_bits [P, ceil(T/32)] (int32 storage of u32 words) -> bool [P, T]."""
    w = np_bits(bits).astype(np.uint32)
    out = np.zeros((w.shape[0], w.shape[1] * 32), dtype=bool)
    for bit in range(32):
        out[:, bit::32] = ((w >> np.uint32(bit)) & np.uint32(1)).astype(bool)
    return out[:, :T]


def read_pool(kv, pair: int):
    """Logical content of one pair's main pool: positions, K rows, V rows (bit copies,
    in block-table order)."""
    n = int(kv.length[pair])
    npg = (n + 15) // 16
    bt = kv.block_table[pair, :npg].long()
    if npg == 0:
        d = kv.c.head_dim
        empty = kv.k_pages[:0].reshape(0, d)
        return np.zeros(0, np.int64), np_bits(empty), np_bits(empty)
    pos = kv.page_pos[bt].reshape(-1)[:n]
    K = kv.k_pages[bt].reshape(-1, kv.c.head_dim)[:n]
    V = kv.v_pages[bt].transpose(1, 2).reshape(-1, kv.c.head_dim)[:n]
    return np_bits(pos).astype(np.int64), np_bits(K), np_bits(V)


def unpack_int4(x: torch.Tensor) -> torch.Tensor:
    """int8 bytes [..., n] -> int8 codes [..., 2n]: low nibble first, sign-extended."""
    b = x.to(torch.int32) & 0xFF
    lo = ((b & 0xF) ^ 8) - 8
    hi = (((b >> 4) & 0xF) ^ 8) - 8
    return torch.stack([lo, hi], dim=-1).reshape(*x.shape[:-1], 2 * x.shape[-1]).to(torch.int8)


def read_pool8(kv, pair: int):
    n = int(kv.length8[pair])
    npg = (n + 15) // 16
    d = kv.c.head_dim
    if npg == 0:
        z = np.zeros((0, d), np.int8)
        return np.zeros(0, np.int64), z, z, np.zeros(0, np.float32), np.zeros(0, np.float32)
    bt = kv.block_table8[pair, :npg].long()
    pos = kv.page8_pos[bt].reshape(-1)[:n]
    Kp, Vp = kv.k8_pages[bt], kv.v8_pages[bt]
    if kv.c.lp_bits == 4:  # two codes per byte, the even element in the low nibble
        Kp, Vp = unpack_int4(Kp), unpack_int4(Vp)
    K = Kp.reshape(-1, d)[:n]
    V = Vp.transpose(1, 2).reshape(-1, d)[:n]
    ks = kv.k8_scale[bt].reshape(-1)[:n]
    vs = kv.v8_scale[bt].reshape(-1)[:n]
    return (np_bits(pos).astype(np.int64), np_bits(K), np_bits(V), np_bits(ks), np_bits(vs))


def read_ring(ring, pair: int):
    """Occupied ring slots: positions, K rows, V rows, scores (slot order)."""
    w = ring.c.window
    pos = np_bits(ring.pos[pair]).astype(np.int64)
    K = ring.k[pair].reshape(w, -1)
    V = ring.v[pair].transpose(1, 2).reshape(w, -1)
    occ = pos >= 0
    return pos[occ], np_bits(K)[occ], np_bits(V)[occ], np_bits(ring.score[pair])[occ]


def visible_positions(kv, ring, pair: int) -> np.ndarray:
    p, _, _ = read_pool(kv, pair)
    parts = [p]
    if ring is not None:
        parts.append(read_ring(ring, pair)[0])
    if kv.c.num_pages8 > 0:
        parts.append(read_pool8(kv, pair)[0])
    return np.sort(np.concatenate(parts))


def band_mask(s64: np.ndarray, tau: float) -> np.ndarray:
    return np.abs(s64 - np.float64(tau)) < BAND


def check_attention(out_gpu: torch.Tensor, ref: np.ndarray, kv_dtype: torch.dtype):
    got = out_gpu.detach().cpu().double().numpy()
    if kv_dtype == torch.bfloat16:
        err = np.abs(got - ref).max() if got.size else 0.0
        assert err <= ATOL_BF16, f"max-abs error {err:.3e} > {ATOL_BF16}"
        return err
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    rel = (num / np.maximum(den, 1e-30)).max()
    assert rel <= RTOL_F32, f"relative error {rel:.3e} > {RTOL_F32}"
    return rel
