"""CPU fp64 oracle for learned KV-cache eviction and decode attention over the pruned cache.

TEST INFRASTRUCTURE ONLY.  This module is the correctness authority for the HIP path.
It may be imported only by ``tests/``, by ``__graft_entry__.smoke()`` and by the CPU
baseline leg of ``bench.py``.  The library (``sparse_decode_attention_kvzap_amd``) never
imports, calls or links it, and it imports nothing from the library: the two share no
code.  Inputs arrive as numpy arrays holding exactly the bits the GPU receives
(bf16 as uint16 bit patterns, fp32 as float32); every computation below is float64
unless a step states that the pages' method fixes another precision.

Sources (cited by page title and section; no line numbers):
  [KVzap]    "NVIDIA open-sources KVzap" digest (max5.ai, MarkTechPost summary), section
             "key points" and its bullets on the surrogate model, the two structures,
             practical application, and memory/compute efficiency.
  [DMS]      "Nvidia's new technique cuts LLM reasoning cost 8x" (euno.news, VentureBeat
             translation), sections "How DMS works" (step 3, keep/evict head) and
             "Delayed Eviction"; the "prior attempts" table (sliding window).
  [BeaconKV] "BeaconKV cuts KV-cache memory 4x" paper briefing (jiinsi.com), body
             paragraph on beacon tokens kept at full precision and the rest compressed
             lossily, and the FAQ entry on how memory is saved.

Readings where the pages are silent are listed, one per item, in the design notes of
the repository; each function below states the reading it implements.

Pinned: every function here is checked by ``tests/test_oracle_*.py`` against closed
forms, brute force, library routines or the figures the pages print.  The semantic
quality of the scores (how well a synthetic scorer predicts importance) is
"parity unpinned" and out of scope: there are no trained weights.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np
import scipy.special

# ----------------------------------------------------------------------------------
# Reading input bits
# ----------------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of fp32)."""
    u32 = bits.astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def as_f64(a: np.ndarray) -> np.ndarray:
    """uint16 arrays are bf16 bit patterns; float arrays are converted exactly."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------------
# Step 1: surrogate scoring  [KVzap, key points: surrogate model and structure bullets]
# ----------------------------------------------------------------------------------


def score_linear(x: np.ndarray, W: np.ndarray, c: np.ndarray | None = None,
                 chunk: int = 4096) -> np.ndarray:
    """KVzap-Linear: one linear layer from each token's hidden state to one score per
    KV head.  s[b,h,t] = sum_i x[b,t,i] * W[h,i] + c[h].

    x: [B,T,H] float64, W: [Hkv,H] float64 (nn.Linear layout), c: [Hkv] or None.
    Returns s: [B,Hkv,T] float64.
    """
    B, T, H = x.shape
    Hkv = W.shape[0]
    s = np.empty((B, Hkv, T), dtype=np.float64)
    for t0 in range(0, T, chunk):
        xs = x[:, t0:t0 + chunk, :]
        s[:, :, t0:t0 + chunk] = np.matmul(xs, W.T).transpose(0, 2, 1)
    if c is not None:
        s += np.asarray(c, dtype=np.float64)[None, :, None]
    return s


def gelu_erf(a: np.ndarray) -> np.ndarray:
    """Exact (erf) GELU: 0.5 * a * (1 + erf(a / sqrt(2))).  Reading: the pages name a
    2-layer MLP but not its activation; the exact erf form is taken, not the tanh
    approximation."""
    return 0.5 * a * (1.0 + scipy.special.erf(a / math.sqrt(2.0)))


def score_mlp(x: np.ndarray, W1: np.ndarray, b1: np.ndarray | None, W2: np.ndarray,
              b2: np.ndarray | None, chunk: int = 2048) -> np.ndarray:
    """KVzap-MLP: two layers, hidden -> inner (GELU) -> one score per KV head.

    a = x W1^T + b1 ; u = GELU(a) ; s = u W2^T + b2.
    x: [B,T,H], W1: [inner,H], b1: [inner], W2: [Hkv,inner], b2: [Hkv].
    Returns s: [B,Hkv,T] float64.  Tokens are processed in chunks only to bound memory.
    """
    B, T, H = x.shape
    Hkv = W2.shape[0]
    s = np.empty((B, Hkv, T), dtype=np.float64)
    for t0 in range(0, T, chunk):
        xs = x[:, t0:t0 + chunk, :]
        a = np.matmul(xs, W1.T)
        if b1 is not None:
            a += b1
        u = gelu_erf(a)
        o = np.matmul(u, W2.T)
        if b2 is not None:
            o += b2
        s[:, :, t0:t0 + chunk] = o.transpose(0, 2, 1)
    return s


def scorer_macs(kind: str, H: int, inner: int, Hkv: int) -> int:
    """Multiply-accumulates per token of one scorer (weights of the shape the scorer
    functions above take).  [KVzap, key points: memory/compute efficiency bullet]
    relates these to the model's linear-projection cost."""
    if kind == "linear":
        return H * Hkv
    return H * inner + inner * Hkv


# ----------------------------------------------------------------------------------
# Step 2: threshold.  Reading: one scalar per layer, a linear-interpolation quantile
# over all (b, t, h) scores; "keep fraction k" means quantile 1 - k.
# ----------------------------------------------------------------------------------


def threshold_quantile(s: np.ndarray, q: float) -> np.float32:
    """tau = float32(quantile_q(all scores)); the same fp32 value is given to both
    paths."""
    return np.float32(np.quantile(np.asarray(s, dtype=np.float64).ravel(), q,
                                  method="linear"))


# ----------------------------------------------------------------------------------
# Step 3: keep mask  [KVzap, key points: practical-application bullet]
# ----------------------------------------------------------------------------------


def keep_mask(s: np.ndarray, tau: float, R: int) -> np.ndarray:
    """Entries scoring below the threshold are removed; the most recent R tokens are
    always kept.

    s: [..., T] scores of the T tokens in the cache (T counts the current token).
    keep[..., t] = (s >= tau) or (t >= T - R).  NaN compares false: a NaN score is
    evicted unless recent.  If T <= R every token is kept.
    """
    T = s.shape[-1]
    t = np.arange(T)
    return (np.asarray(s, dtype=np.float64) >= np.float64(tau)) | (t >= T - R)


# ----------------------------------------------------------------------------------
# Step 4: compaction.  Kept entries are listed in ascending position; the evicted ones
# follow, also ascending (a stable partition of the positions).
# ----------------------------------------------------------------------------------


def partition_indices(keep_row: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(kept positions ascending, evicted positions ascending) of one (b, h) row."""
    kept = np.flatnonzero(keep_row)
    evicted = np.flatnonzero(~np.asarray(keep_row, dtype=bool))
    return kept, evicted


# ----------------------------------------------------------------------------------
# Step 5: GQA decode attention over the kept entries
# ----------------------------------------------------------------------------------


def attend_one(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K q) V over the given rows.  Zero rows -> zero output.

    q: [d], K: [n,d], V: [n,d] float64.
    """
    if K.shape[0] == 0:
        return np.zeros(q.shape[0], dtype=np.float64)
    logits = (K @ q) * np.float64(scale)
    m = logits.max()
    e = np.exp(logits - m)
    return (e @ V) / e.sum()


def decode_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, visible: np.ndarray,
                     scale: float) -> np.ndarray:
    """Decode attention of one query per head over the visible cache entries.

    q: [B,Hq,d]; K, V: [B,Hkv,T,d]; visible: [B,Hkv,T] bool.  Query head j reads KV
    head j // g with g = Hq / Hkv (contiguous head groups).  Returns [B,Hq,d].
    """
    B, Hq, d = q.shape
    Hkv = K.shape[1]
    g = Hq // Hkv
    out = np.zeros((B, Hq, d), dtype=np.float64)
    for b in range(B):
        for h in range(Hkv):
            idx = np.flatnonzero(visible[b, h])
            Kc = K[b, h, idx]
            Vc = V[b, h, idx]
            for j in range(h * g, (h + 1) * g):
                out[b, j] = attend_one(q[b, j], Kc, Vc, scale)
    return out


def sm_scale(d: int) -> np.float32:
    """Softmax scale 1/sqrt(d) as the fp32 value both paths use."""
    return np.float32(1.0 / math.sqrt(d))


# ----------------------------------------------------------------------------------
# DMS delayed eviction  [DMS, "How DMS works" step 3 and "Delayed Eviction"]
# ----------------------------------------------------------------------------------


def dms_evict_flags(s: np.ndarray) -> np.ndarray:
    """Binary keep/evict signal per token.  Reading: the scorer's sign stands in for
    the learned head; a token is flagged for eviction iff its score is not >= 0."""
    return ~(np.asarray(s, dtype=np.float64) >= 0.0)


def dms_visible(flags: np.ndarray, p: int, w: int) -> np.ndarray:
    """Visibility at the decode step that appends position p (cache length p+1).

    A flagged token stays in a buffer for w steps and is then removed: token t is
    visible iff it is not flagged, or it was appended fewer than w steps ago
    (p - t < w).  flags: [..., >= p+1].  Returns [..., p+1] bool.
    Recomputed from scratch at every step (no state), so it checks any incremental
    ring/pool implementation.
    """
    t = np.arange(p + 1)
    return (~flags[..., :p + 1]) | (p - t < w)


# ----------------------------------------------------------------------------------
# Prefill attention under eviction  [DMS, "Delayed Eviction"; KVzap, practical
# application]
# ----------------------------------------------------------------------------------


def prefill_visible(keep: np.ndarray, W: int) -> np.ndarray:
    """Which keys each prompt position sees while the prompt itself is processed.

    Reading: every prompt position is a step of the sequence, so query position i sees
    what a decode step at length i + 1 sees: a key j <= i that is kept, or that is one
    of the last W positions (i - j < W).  KVzap: keep = (s >= tau), W = R (the recent
    window); DMS: keep = not flagged, W = w (the eviction delay).
    keep: [..., T] bool.  Returns [..., T (query), T (key)] bool.
    """
    keep = np.asarray(keep, dtype=bool)
    T = keep.shape[-1]
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    return (j <= i) & (keep[..., None, :] | ((i - j) < W))


def prefill_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, keep: np.ndarray, W: int,
                      scale: float) -> np.ndarray:
    """Masked causal attention of every prompt position (GQA, contiguous head groups).

    q: [B,Hq,T,d]; K, V: [B,Hkv,T,d]; keep: [B,Hkv,T] bool.  Row i of query head jq is
    softmax(scale * K q_i) V over the keys prefill_visible marks for position i; a row
    with no visible key is 0.  Returns [B,Hq,T,d] float64.
    """
    B, Hq, T, d = q.shape
    Hkv = K.shape[1]
    g = Hq // Hkv
    out = np.zeros((B, Hq, T, d), dtype=np.float64)
    for b in range(B):
        for h in range(Hkv):
            vis = prefill_visible(keep[b, h], W)
            for jq in range(h * g, (h + 1) * g):
                logits = (q[b, jq] @ K[b, h].T) * np.float64(scale)
                logits = np.where(vis, logits, -np.inf)
                m = logits.max(axis=1, keepdims=True)
                ok = np.isfinite(m[:, 0])
                e = np.where(vis, np.exp(logits - np.where(ok[:, None], m, 0.0)), 0.0)
                den = e.sum(axis=1, keepdims=True)
                out[b, jq] = np.where(ok[:, None], (e @ V[b, h]) / np.where(ok[:, None], den, 1.0), 0.0)
    return out


# ----------------------------------------------------------------------------------
# BeaconKV mixed precision  [BeaconKV, body and FAQ on how memory is saved]
# ----------------------------------------------------------------------------------


# The page names low-precision quantization of the non-beacon entries without fixing a
# format.  Reading: symmetric integer codes with one fp32 absmax scale per (token, head)
# row, in two widths: int8 (codes -127..127) and int4 (codes -7..7, the same rule with
# 7 levels a side; -8 is not used, so the grid stays symmetric).
LP_QMAX = {8: 127, 4: 7}


def quantize_absmax(x: np.ndarray, qmax: int) -> Tuple[np.ndarray, np.float32]:
    """Symmetric codes with one fp32 absmax scale per row (token, head), computed from
    the stored values.  scale = fp32(a / qmax) with a = max |x|; code = clamp(round-
    half-even(x / scale), -qmax, qmax).  A zero row has scale 0 and zero codes.

    Precision: the code is an integer decided by floating point, so it is decided in
    IEEE fp32 (the division of two fp32 values, correctly rounded), which is the
    precision the stored values and the scale have.
    """
    xf = np.asarray(x, dtype=np.float32)
    a = np.float32(np.max(np.abs(xf))) if xf.size else np.float32(0)
    scale = np.float32(a / np.float32(qmax))
    if scale == 0:
        return np.zeros(xf.shape, dtype=np.int8), np.float32(0.0)
    y = xf / scale  # float32 / float32 -> float32, correctly rounded
    codes = np.clip(np.rint(y), -qmax, qmax).astype(np.int8)
    return codes, scale


def quantize_absmax_int8(x: np.ndarray) -> Tuple[np.ndarray, np.float32]:
    """int8 codes -127..127, scale fp32(a / 127) (see quantize_absmax)."""
    return quantize_absmax(x, 127)


def quantize_absmax_int4(x: np.ndarray) -> Tuple[np.ndarray, np.float32]:
    """int4 codes -7..7 (held in int8 here), scale fp32(a / 7) (see quantize_absmax)."""
    return quantize_absmax(x, 7)


def dequantize_int8(codes: np.ndarray, scale: np.float32) -> np.ndarray:
    """x_hat = code * scale (exact in float64); any code width."""
    return codes.astype(np.float64) * np.float64(scale)


# A third reading of "low precision": 8-bit floating-point codes in the OCP FP8 E4M3
# format (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; no infinities; the
# all-ones exponent and mantissa pattern is NaN, so the largest finite magnitude is
# 1.75 * 2^8 = 448; exponent field 0 holds the subnormals m * 2^-9).  One fp32 absmax
# scale per row maps the row's largest magnitude onto 448.  The encoder rounds to the
# nearest code, ties to the even mantissa; a magnitude at or above 448 saturates to 448
# (reading: the scaling keeps every value at most 448 (1 + 2^-23), which rounds to 448
# anyway, so saturation only guards the definition).
FP8_E4M3_MAX = 448.0


def fp8_e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Values (float64) of E4M3 byte codes; NaN for the two NaN codes."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = m * 2.0 ** -9
    val = sign * np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def fp8_e4m3_encode(x: np.ndarray) -> np.ndarray:
    """E4M3 byte codes of float32 values: round to nearest, ties to even; magnitudes at
    or above 448 saturate to 448.  (Not defined for NaN inputs.)"""
    xf = np.asarray(x, dtype=np.float32)
    a = np.abs(xf).astype(np.float64)  # exact
    sign = np.where(np.signbit(xf), 0x80, 0).astype(np.int64)
    out = np.zeros(xf.shape, dtype=np.int64)
    # subnormal range (below the smallest normal 2^-6): the code is the nearest
    # multiple m of 2^-9 (m = 8 is the smallest normal, code 0x08, by the same bits)
    sub = a < 2.0 ** -6
    out[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)
    # normal range: a = 2^k (1 + f), the mantissa f rounded to 3 bits; a carry out of
    # the mantissa moves to the next exponent through the integer addition
    nrm = ~sub
    mant, ex = np.frexp(a[nrm])  # a = mant 2^ex, mant in [0.5, 1)
    k = ex - 1
    frac8 = np.rint((mant * 2.0 - 1.0) * 8.0).astype(np.int64)  # 0..8
    out[nrm] = ((k + 7) << 3) + frac8
    out = np.minimum(out, 0x7E)  # saturate at 448 (0x7F would be NaN)
    out = np.where(a >= FP8_E4M3_MAX, 0x7E, out)
    return (sign | out).astype(np.uint8)


def quantize_absmax_fp8(x: np.ndarray) -> Tuple[np.ndarray, np.float32]:
    """E4M3 codes with one fp32 absmax scale per row: scale = fp32(a / 448) with
    a = max |x|, code = E4M3 rounding of the fp32 quotient x / scale (correctly rounded,
    as for the integer codes).  A zero row has scale 0 and zero codes."""
    xf = np.asarray(x, dtype=np.float32)
    a = np.float32(np.max(np.abs(xf))) if xf.size else np.float32(0)
    scale = np.float32(a / np.float32(FP8_E4M3_MAX))
    if scale == 0:
        return np.zeros(xf.shape, dtype=np.uint8), np.float32(0.0)
    return fp8_e4m3_encode(xf / scale), scale


def dequantize_fp8(codes: np.ndarray, scale: np.float32) -> np.ndarray:
    """x_hat = value(code) * scale (exact in float64)."""
    return fp8_e4m3_decode(codes) * np.float64(scale)


def lp_round_trip(x: np.ndarray, bits):
    """(codes, scale, x_hat) of one row in the low-precision format `bits`: 8 or 4
    (integer codes) or "fp8" (E4M3 codes)."""
    if bits == "fp8":
        c, s = quantize_absmax_fp8(x)
        return c, s, dequantize_fp8(c, s)
    c, s = quantize_absmax(x, LP_QMAX[bits])
    return c, s, dequantize_int8(c, s)


def beacon_kv(K: np.ndarray, V: np.ndarray, beacon: np.ndarray, bits=8):
    """Beacon entries keep their exact values; every other (token, head) row of K and
    of V (separately) is replaced by its round trip through the low-precision format
    `bits`: 8 or 4 (integer codes) or "fp8" (E4M3 codes).

    K, V: [B,Hkv,T,d] float64 holding bf16 values; beacon: [B,Hkv,T] bool.
    Returns K_hat, V_hat float64, plus the codes and scales of the demoted rows.
    """
    Kh = np.array(K, dtype=np.float64, copy=True)
    Vh = np.array(V, dtype=np.float64, copy=True)
    B, Hkv, T, d = K.shape
    cdt = np.uint8 if bits == "fp8" else np.int8
    kc = np.zeros((B, Hkv, T, d), dtype=cdt)
    vc = np.zeros((B, Hkv, T, d), dtype=cdt)
    ks = np.zeros((B, Hkv, T), dtype=np.float32)
    vs = np.zeros((B, Hkv, T), dtype=np.float32)
    for b in range(B):
        for h in range(Hkv):
            for t in np.flatnonzero(~beacon[b, h]):
                kc[b, h, t], ks[b, h, t], Kh[b, h, t] = lp_round_trip(K[b, h, t], bits)
                vc[b, h, t], vs[b, h, t], Vh[b, h, t] = lp_round_trip(V[b, h, t], bits)
    return Kh, Vh, (kc, ks, vc, vs)


# ----------------------------------------------------------------------------------
# Closed-form footprint  [KVzap, key points: need-for-compression bullet]
# ----------------------------------------------------------------------------------


def kv_cache_bytes(layers: int, kv_heads: int, head_dim: int, bytes_per_elem: int,
                   tokens: int) -> int:
    """Bytes of a dense K+V cache: 2 * layers * kv_heads * head_dim * bytes * tokens.
    It grows linearly with the token count."""
    return 2 * layers * kv_heads * head_dim * bytes_per_elem * tokens


# ----------------------------------------------------------------------------------
# Whole-path helpers (compositions of the steps above, in the pages' order)
# ----------------------------------------------------------------------------------


def kvzap_visible_after_prefill(s: np.ndarray, tau: float, R: int) -> np.ndarray:
    """Score -> threshold -> keep recent: the cache content after compressing a
    context of T tokens."""
    return keep_mask(s, tau, R)


def kvzap_visible_at_decode(s: np.ndarray, tau: float, R: int, p: int) -> np.ndarray:
    """Cache content at the decode step that appends position p: the same rule at
    length T = p + 1 (eviction is a pure function of scores, tau and length)."""
    return keep_mask(s[..., :p + 1], tau, R)


def beacon_decode_attention(q, K, V, beacon, scale, bits=8):
    """One softmax over all T tokens: exact values for beacon rows, round trips through
    the low-precision format `bits` (8, 4 or "fp8") for the others."""
    Kh, Vh, _ = beacon_kv(K, V, beacon, bits)
    allvis = np.ones(beacon.shape, dtype=bool)
    return decode_attention(q, Kh, Vh, allvis, scale)
