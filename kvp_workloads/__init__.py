"""Seeded synthetic workloads for learned KV-cache eviction + sparse decode attention.

This module holds the configuration shapes and the seeded input generators that both
the CPU oracle (via tests and the bench's CPU leg) and the HIP path consume.  It holds
none of the method's arithmetic: no scoring, thresholding, masking, compaction,
quantization or attention happens here, only random tensors of the right shapes and
distributions.

Generators produce torch tensors on the requested device with a seeded
``torch.Generator``.  Parity tests generate once (on the GPU for large shapes), hand
the very same bits to the library and, after a host copy, to the oracle.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

PAGE = 16
RECENT = 128
BASE_SEED = 20261202


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and distribution recipe of one synthetic workload.

    Names follow the notation of the pages: B batch, H hidden size, Hq / Hkv query /
    KV heads, d head dim, T context length in the cache counting the current decode
    token, R recent window that is always kept, w delayed-eviction window.
    """

    name: str
    B: int
    H: int
    Hq: int
    Hkv: int
    d: int
    T: int
    kv_dtype: torch.dtype
    scorer: str  # "linear" or "mlp"
    inner: int = 512  # MLP width (first layer output)
    keep_quantiles: tuple = (0.75,)  # tau = quantile q of the scores -> keep ~ 1-q
    R: int = RECENT
    w: int = RECENT  # ring window used in decode (== R for KVzap, == delay for DMS)
    fixed_tau: Optional[float] = None  # DMS: sign of the scorer
    scorer_bias: float = 0.0
    unit_norm_rows: bool = False
    outlier_frac: float = 0.0
    outlier_mult: float = 1.0
    prompt: int = 0  # DMS: prompt length
    steps: int = 0  # DMS: number of decode steps
    int8_demote: bool = False  # evicted tokens go to the low-precision pool
    lp_bits: object = 8  # code format of that pool: 8, 4 (integer codes) or "fp8" (E4M3)
    index: int = 0

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv

    @property
    def hidden_dtype(self) -> torch.dtype:
        return self.kv_dtype

    def seed(self, stream: str) -> int:
        """Per-tensor seed: one independent stream per named tensor."""
        h = 0
        for ch in stream:
            h = (h * 131 + ord(ch)) % 1_000_003
        return BASE_SEED + 1000 * self.index + h

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Probit of 0.875: bias that makes P(score < 0) = 0.875 for a unit-variance score.
DMS_BIAS = -1.1503493803760079

TINY = Workload("tiny", B=1, H=256, Hq=4, Hkv=2, d=64, T=512, kv_dtype=torch.float32,
                scorer="linear", keep_quantiles=(0.5,), index=0)
QWEN3_8B_LAYER = Workload("qwen3_8b_layer", B=16, H=4096, Hq=32, Hkv=8, d=128, T=32768,
                          kv_dtype=torch.bfloat16, scorer="mlp", keep_quantiles=(0.75,),
                          index=1)
DMS_DELAYED = Workload("dms_delayed", B=64, H=4096, Hq=32, Hkv=8, d=128, T=8192 + 1024,
                       kv_dtype=torch.bfloat16, scorer="linear", keep_quantiles=(),
                       fixed_tau=0.0, R=256, w=256, scorer_bias=DMS_BIAS,
                       unit_norm_rows=True, prompt=8192, steps=1024, index=2)
LONG_70B_LAYER = Workload("long_70b_layer", B=4, H=8192, Hq=64, Hkv=8, d=128, T=131072,
                          kv_dtype=torch.bfloat16, scorer="linear",
                          keep_quantiles=(0.5, 0.75), outlier_frac=0.01, outlier_mult=8.0,
                          index=3)
BEACON_MIXED = Workload("beacon_mixed", B=16, H=4096, Hq=32, Hkv=8, d=128, T=32768,
                        kv_dtype=torch.bfloat16, scorer="mlp", keep_quantiles=(0.90,),
                        int8_demote=True, index=4)

# The same inputs as beacon_mixed (same seeds) with an int4 pool for the demoted tokens.
BEACON_INT4 = dataclasses.replace(BEACON_MIXED, name="beacon_int4", lp_bits=4)
# ... and with an fp8 E4M3 pool.
BEACON_FP8 = dataclasses.replace(BEACON_MIXED, name="beacon_fp8", lp_bits="fp8")

ALL = (TINY, QWEN3_8B_LAYER, DMS_DELAYED, LONG_70B_LAYER, BEACON_MIXED, BEACON_INT4, BEACON_FP8)
BY_NAME = {w.name: w for w in ALL}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, dtype, seed: int, device="cpu", std: float = 1.0,
           chunk_elems: int = 1 << 28) -> torch.Tensor:
    """N(0, std^2) drawn in fp32, then rounded (RNE) to ``dtype``.

    Large tensors are drawn chunk by chunk from one generator so memory stays bounded.
    """
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    g = _gen(seed, device)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        tmp = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            tmp.mul_(std)
        flat[s:e].copy_(tmp)
        del tmp
    return out


@dataclasses.dataclass
class ScorerWeights:
    kind: str
    W1: torch.Tensor  # linear: [Hkv, H]; mlp: [inner, H]   (hidden dtype)
    b1: Optional[torch.Tensor]  # linear: [Hkv] fp32 bias; mlp: [inner] fp32
    W2: Optional[torch.Tensor] = None  # mlp: [Hkv, inner] fp32
    b2: Optional[torch.Tensor] = None  # mlp: [Hkv] fp32


def scorer_weights(wl: Workload, device="cpu") -> ScorerWeights:
    """Synthetic surrogate-scorer weights in nn.Linear layout [out, in].

    First-layer weights ~ N(0, 1/fan_in) in the hidden dtype (unit-norm rows for the
    DMS stand-in), biases zero unless the workload sets one, second MLP layer fp32.
    """
    hd = wl.hidden_dtype
    if wl.scorer == "linear":
        if wl.unit_norm_rows:
            w = normal((wl.Hkv, wl.H), torch.float32, wl.seed("W"), device)
            w = w / w.norm(dim=1, keepdim=True)
            W = w.to(hd)
        else:
            W = normal((wl.Hkv, wl.H), hd, wl.seed("W"), device, std=1.0 / math.sqrt(wl.H))
        b = torch.full((wl.Hkv,), wl.scorer_bias, dtype=torch.float32, device=device)
        return ScorerWeights("linear", W, b)
    W1 = normal((wl.inner, wl.H), hd, wl.seed("W1"), device, std=1.0 / math.sqrt(wl.H))
    b1 = torch.zeros(wl.inner, dtype=torch.float32, device=device)
    W2 = normal((wl.Hkv, wl.inner), torch.float32, wl.seed("W2"), device,
                std=1.0 / math.sqrt(wl.inner))
    b2 = torch.full((wl.Hkv,), wl.scorer_bias, dtype=torch.float32, device=device)
    return ScorerWeights("mlp", W1, b1, W2, b2)


def hidden_states(wl: Workload, T: int, device="cpu", stream="hidden") -> torch.Tensor:
    """Hidden states [B, T, H] ~ N(0,1) in the hidden dtype."""
    return normal((wl.B, T, wl.H), wl.hidden_dtype, wl.seed(stream), device)


def kv_dense(wl: Workload, T: int, device="cpu", stream="kv"):
    """Dense K and V [B, Hkv, T, d] ~ N(0,1) with optional outlier tokens.

    Outliers: per batch row, floor(frac*T) token positions drawn without replacement;
    K and V of those tokens are multiplied by ``outlier_mult`` in every KV head (an
    exact power-of-two scaling in bf16).
    """
    K = normal((wl.B, wl.Hkv, T, wl.d), wl.kv_dtype, wl.seed(stream + "K"), device)
    V = normal((wl.B, wl.Hkv, T, wl.d), wl.kv_dtype, wl.seed(stream + "V"), device)
    if wl.outlier_frac > 0:
        n_out = int(math.floor(wl.outlier_frac * T))
        g = _gen(wl.seed(stream + "outliers"), "cpu")
        for b in range(wl.B):
            pos = torch.randperm(T, generator=g)[:n_out].to(device)
            K[b][:, pos, :] *= wl.outlier_mult
            V[b][:, pos, :] *= wl.outlier_mult
    return K, V


def queries(wl: Workload, device="cpu", stream="q") -> torch.Tensor:
    """Decode queries [B, Hq, d] ~ N(0,1) stored in the KV dtype."""
    return normal((wl.B, wl.Hq, wl.d), wl.kv_dtype, wl.seed(stream), device)


def prompt_queries(wl: Workload, T: int, device="cpu", stream="prompt_q") -> torch.Tensor:
    """Queries of every prompt position [B, Hq, T, d] ~ N(0,1) in the KV dtype."""
    return normal((wl.B, wl.Hq, T, wl.d), wl.kv_dtype, wl.seed(stream), device)


def step_inputs(wl: Workload, step: int, device="cpu"):
    """Per-decode-step draws: new hidden [B,1,H], k/v [B,Hkv,d], q [B,Hq,d]."""
    tag = f"step{step}_"
    h = normal((wl.B, 1, wl.H), wl.hidden_dtype, wl.seed(tag + "h"), device)
    k = normal((wl.B, wl.Hkv, wl.d), wl.kv_dtype, wl.seed(tag + "k"), device)
    v = normal((wl.B, wl.Hkv, wl.d), wl.kv_dtype, wl.seed(tag + "v"), device)
    q = normal((wl.B, wl.Hq, wl.d), wl.kv_dtype, wl.seed(tag + "q"), device)
    return h, k, v, q


def random_scores(shape, seed: int, device="cpu") -> torch.Tensor:
    """fp32 N(0,1) scores for unit tests of selection alone."""
    return normal(shape, torch.float32, seed, device)
