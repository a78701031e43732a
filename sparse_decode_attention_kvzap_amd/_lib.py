"""ctypes binding of libkvp (the C ABI declared in include/kvp.h).

Argument marshalling only: every computation runs in the HIP kernels of libkvp.so.
PyTorch provides device memory and the current HIP stream.  The functions keep the C
names; they take torch tensors, pass ``data_ptr()`` and raise ``KvpError`` on any
non-OK status.  There is no fallback: if libkvp.so is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import math
import os
from ctypes import c_float, c_int32, c_int64, c_size_t, c_void_p
from dataclasses import dataclass, field
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvp.so")

KVP_PAGE = 16
KVP_F32, KVP_BF16 = 0, 1
KVP_SCORER_LINEAR, KVP_SCORER_MLP = 0, 1
KVP_COMPACT_EVICT, KVP_COMPACT_DEMOTE_INT8 = 0, 1
STATUS = {0: "KVP_OK", 1: "KVP_E_ARG", 2: "KVP_E_DTYPE", 3: "KVP_E_WORKSPACE",
          4: "KVP_E_CAPACITY", 5: "KVP_E_HIP", 6: "KVP_E_UNSUPPORTED"}
ERR_POOL_FULL, ERR_TABLE_FULL, ERR_POOL8_FULL = 1, 2, 4
KVP_LP_INT8, KVP_LP_INT4, KVP_LP_FP8_E4M3 = 8, 4, 0x108


class KvpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class KvpScorer(ctypes.Structure):
    _fields_ = [("kind", c_int32), ("hidden", c_int32), ("inner", c_int32),
                ("n_kv_heads", c_int32), ("wdtype", c_int32), ("_pad", c_int32),
                ("w1", c_void_p), ("b1", c_void_p), ("w2", c_void_p), ("b2", c_void_p)]


class KvpPagedKV(ctypes.Structure):
    _fields_ = [("dtype", c_int32), ("num_pairs", c_int32), ("head_dim", c_int32),
                ("num_pages", c_int32), ("max_pages_per_pair", c_int32),
                ("num_pages8", c_int32), ("max_pages8_per_pair", c_int32), ("lp_bits", c_int32),
                ("k_pages", c_void_p), ("v_pages", c_void_p), ("page_pos", c_void_p),
                ("block_table", c_void_p), ("length", c_void_p), ("page_top", c_void_p),
                ("err", c_void_p), ("k8_pages", c_void_p), ("v8_pages", c_void_p),
                ("k8_scale", c_void_p), ("v8_scale", c_void_p), ("page8_pos", c_void_p),
                ("block_table8", c_void_p), ("length8", c_void_p), ("page8_top", c_void_p)]


class KvpRing(ctypes.Structure):
    _fields_ = [("window", c_int32), ("_pad", c_int32), ("k", c_void_p), ("v", c_void_p),
                ("score", c_void_p), ("pos", c_void_p)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkvp.so (import torch first so one HIP runtime serves both)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libkvp.so not built at {path}; run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    sig = {
        "kvp_status_str": (ctypes.c_char_p, [c_int32]),
        "kvp_version": (ctypes.c_char_p, []),
        "kvp_score": (c_int32, [P(KvpScorer), c_void_p, c_int32, c_int32, c_int32, c_void_p,
                                c_int64, c_void_p, c_size_t, c_void_p]),
        "kvp_score_workspace_size": (c_size_t, [P(KvpScorer), c_int32, c_int32]),
        "kvp_select": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int64, c_float, c_int32,
                                 c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
        "kvp_select_workspace_size": (c_size_t, [c_int32, c_int32, c_int32]),
        "kvp_select_dev_tau": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int64, c_void_p,
                                         c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                         c_void_p]),
        "kvp_threshold": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int64, ctypes.c_double,
                                    c_void_p, c_void_p, c_size_t, c_void_p]),
        "kvp_threshold_workspace_size": (c_size_t, []),
        "kvp_compact": (c_int32, [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32,
                                  c_void_p, c_void_p, c_void_p, c_int64, c_int32, P(KvpPagedKV),
                                  P(KvpRing), c_void_p, c_size_t, c_void_p]),
        "kvp_compact_workspace_size": (c_size_t, [c_int32, c_int32]),
        "kvp_step_delayed": (c_int32, [P(KvpPagedKV), P(KvpRing), c_void_p, c_void_p, c_int32,
                                       c_void_p, c_int64, c_float, c_int32, c_void_p]),
        "kvp_step_delayed_dev": (c_int32, [P(KvpPagedKV), P(KvpRing), c_void_p, c_void_p,
                                           c_int32, c_void_p, c_int64, c_void_p, c_void_p,
                                           c_void_p]),
        "kvp_score_step_delayed": (c_int32, [P(KvpScorer), c_void_p, c_int32, P(KvpPagedKV),
                                             P(KvpRing), c_void_p, c_void_p, c_int32, c_void_p,
                                             c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
        "kvp_decode_attn": (c_int32, [c_void_p, c_int32, c_int32, c_int32, P(KvpPagedKV),
                                      P(KvpRing), c_float, c_void_p, c_void_p, c_size_t,
                                      c_void_p]),
        "kvp_decode_attn_workspace_size": (c_size_t, [c_int32, c_int32, c_int32, c_int32]),
        "kvp_decode_step": (c_int32, [P(KvpScorer), c_void_p, c_int32, P(KvpPagedKV), P(KvpRing),
                                      c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_void_p,
                                      c_void_p, c_void_p, c_int32, c_int32, c_int32, c_float,
                                      c_void_p, c_void_p, c_size_t, c_void_p]),
        "kvp_decode_step_workspace_size": (c_size_t, [P(KvpScorer), c_int32, c_int32, c_int32,
                                                     c_int32]),
        "kvp_decode_attn_noalloc": (c_int32, [c_void_p, c_int32, c_int32, c_int32,
                                              P(KvpPagedKV), P(KvpRing), c_float, c_void_p,
                                              c_void_p]),
        "kvp_prefill_attn": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                       c_int32, c_int32, c_int32, c_void_p, c_void_p, c_int32,
                                       c_float, c_void_p, c_void_p]),
        "kvp_reset": (c_int32, [P(KvpPagedKV), P(KvpRing), c_void_p]),
        "kvp_clear_error": (c_int32, [P(KvpPagedKV), c_void_p]),
        "kvp_check": (c_int32, [P(KvpPagedKV), c_void_p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ok(status: int, where: str):
    if status != 0:
        raise KvpError(status, where)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KVP_BF16
    if t.dtype == torch.float32:
        return KVP_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("libkvp takes contiguous device tensors")


# ------------------------------------------------------------------ buffers


@dataclass
class Scorer:
    """Surrogate scorer weights (device tensors) and their C descriptor."""
    kind: int
    w1: torch.Tensor
    b1: Optional[torch.Tensor] = None
    w2: Optional[torch.Tensor] = None
    b2: Optional[torch.Tensor] = None
    c: KvpScorer = field(default=None, repr=False)

    def __post_init__(self):
        _cuda(self.w1, self.b1, self.w2, self.b2)
        inner = self.w1.shape[0] if self.kind == KVP_SCORER_MLP else 0
        hkv = self.w2.shape[0] if self.kind == KVP_SCORER_MLP else self.w1.shape[0]
        self.c = KvpScorer(self.kind, self.w1.shape[1], inner, hkv, _dt(self.w1), 0,
                           _p(self.w1), _p(self.b1), _p(self.w2), _p(self.b2))

    @property
    def n_kv_heads(self) -> int:
        return self.c.n_kv_heads


@dataclass
class PagedKV:
    """Paged KV cache buffers (allocated with torch) and their C descriptor."""
    c: KvpPagedKV
    tensors: dict

    @staticmethod
    def allocate(num_pairs: int, head_dim: int, num_pages: int, max_pages_per_pair: int,
                 dtype=torch.bfloat16, device="cuda", num_pages8: int = 0,
                 max_pages8_per_pair: int = 0, poison: bool = False,
                 lp_bits=8) -> "PagedKV":
        """lp_bits: code format of the low-precision pool: 8 (int8 codes), 4 (int4 codes,
        two per byte, so its K pages are [16][d/2] bytes and its V^T pages [d][8]) or
        "fp8" (E4M3 codes, one per byte)."""
        if lp_bits not in (4, 8, "fp8"):
            raise ValueError("lp_bits must be 8, 4 or 'fp8'")
        dev = torch.device(device)
        t = {}
        fill = float("nan") if poison else 0.0
        t["k_pages"] = torch.full((max(num_pages, 1), KVP_PAGE, head_dim), fill, dtype=dtype, device=dev)
        t["v_pages"] = torch.full((max(num_pages, 1), head_dim, KVP_PAGE), fill, dtype=dtype, device=dev)
        t["page_pos"] = torch.full((max(num_pages, 1), KVP_PAGE), -7, dtype=torch.int32, device=dev)
        t["block_table"] = torch.full((num_pairs, max_pages_per_pair), -7, dtype=torch.int32, device=dev)
        t["length"] = torch.zeros(num_pairs, dtype=torch.int32, device=dev)
        t["page_top"] = torch.zeros(1, dtype=torch.int32, device=dev)
        t["err"] = torch.zeros(1, dtype=torch.int32, device=dev)
        if num_pages8 > 0:
            per = 2 if lp_bits == 4 else 1  # codes per byte
            t["k8_pages"] = torch.full((num_pages8, KVP_PAGE, head_dim // per), 0x55, dtype=torch.int8, device=dev)
            t["v8_pages"] = torch.full((num_pages8, head_dim, KVP_PAGE // per), 0x55, dtype=torch.int8, device=dev)
            t["k8_scale"] = torch.full((num_pages8, KVP_PAGE), fill, dtype=torch.float32, device=dev)
            t["v8_scale"] = torch.full((num_pages8, KVP_PAGE), fill, dtype=torch.float32, device=dev)
            t["page8_pos"] = torch.full((num_pages8, KVP_PAGE), -7, dtype=torch.int32, device=dev)
            t["block_table8"] = torch.full((num_pairs, max_pages8_per_pair), -7, dtype=torch.int32, device=dev)
            t["length8"] = torch.zeros(num_pairs, dtype=torch.int32, device=dev)
            t["page8_top"] = torch.zeros(1, dtype=torch.int32, device=dev)
        c = KvpPagedKV()
        c.dtype = KVP_BF16 if dtype == torch.bfloat16 else KVP_F32
        c.num_pairs, c.head_dim, c.num_pages = num_pairs, head_dim, num_pages
        c.max_pages_per_pair = max_pages_per_pair
        c.num_pages8, c.max_pages8_per_pair = num_pages8, max_pages8_per_pair
        c.lp_bits = KVP_LP_FP8_E4M3 if lp_bits == "fp8" else lp_bits
        for name, ten in t.items():
            setattr(c, name, ten.data_ptr())
        return PagedKV(c, t)

    def __getattr__(self, name):
        t = self.__dict__.get("tensors")
        if t is not None and name in t:
            return t[name]
        raise AttributeError(name)


@dataclass
class Ring:
    """Recent-window ring buffers and their C descriptor."""
    c: KvpRing
    tensors: dict

    @staticmethod
    def allocate(num_pairs: int, window: int, head_dim: int, dtype=torch.bfloat16,
                 device="cuda", poison: bool = False) -> "Ring":
        if window % KVP_PAGE:
            raise ValueError("window must be a multiple of 16")
        dev = torch.device(device)
        fill = float("nan") if poison else 0.0
        rp = window // KVP_PAGE
        t = {
            "k": torch.full((num_pairs, rp, KVP_PAGE, head_dim), fill, dtype=dtype, device=dev),
            "v": torch.full((num_pairs, rp, head_dim, KVP_PAGE), fill, dtype=dtype, device=dev),
            "score": torch.zeros((num_pairs, window), dtype=torch.float32, device=dev),
            "pos": torch.full((num_pairs, window), -1, dtype=torch.int32, device=dev),
        }
        c = KvpRing(window, 0, t["k"].data_ptr(), t["v"].data_ptr(), t["score"].data_ptr(),
                    t["pos"].data_ptr())
        return Ring(c, t)

    def __getattr__(self, name):
        t = self.__dict__.get("tensors")
        if t is not None and name in t:
            return t[name]
        raise AttributeError(name)


def _kvref(kv: Optional[PagedKV]):
    return None if kv is None else ctypes.byref(kv.c)


def _ringref(ring: Optional[Ring]):
    return None if ring is None else ctypes.byref(ring.c)


# ------------------------------------------------------------------ entry points


def kvp_status_str(status: int) -> str:
    return load().kvp_status_str(status).decode()


def kvp_version() -> str:
    return load().kvp_version().decode()


def kvp_score_workspace_size(scorer: Scorer, B: int, T: int) -> int:
    return load().kvp_score_workspace_size(ctypes.byref(scorer.c), B, T)


def kvp_score(scorer: Scorer, hidden: torch.Tensor, scores: torch.Tensor,
              ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """scores[b, h, t] for hidden [B, T, H]; scores is [B, Hkv, ld_s] fp32, ld_s >= T."""
    _cuda(hidden, scores, ws)
    B, T, _ = hidden.shape
    ld_s = scores.shape[-1]
    _ok(load().kvp_score(ctypes.byref(scorer.c), hidden.data_ptr(), _dt(hidden), B, T,
                         scores.data_ptr(), ld_s, _p(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                         _stream(stream)), "kvp_score")
    return scores


def kvp_select_workspace_size(B: int, Hkv: int, T: int) -> int:
    return load().kvp_select_workspace_size(B, Hkv, T)


def kvp_select(scores: torch.Tensor, T: int, tau, recent: int, keep_bits: torch.Tensor,
               kept_idx: torch.Tensor, kept_count: torch.Tensor, ws: torch.Tensor,
               stream=None):
    """scores [B, Hkv, ld_s] fp32 -> keep_bits [B*Hkv, ceil(T/32)] i32 (u32 bits),
    kept_idx [B*Hkv, T] i32, kept_count [B*Hkv] i32.  tau: a float, or a one-element
    fp32 device tensor (kvp_select_dev_tau, e.g. written by kvp_threshold)."""
    _cuda(scores, keep_bits, kept_idx, kept_count, ws)
    B, Hkv, ld_s = scores.shape
    args = (keep_bits.data_ptr(), kept_idx.data_ptr(), kept_count.data_ptr(),
            ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream))
    if isinstance(tau, torch.Tensor):
        _cuda(tau)
        assert tau.dtype == torch.float32 and tau.numel() >= 1
        _ok(load().kvp_select_dev_tau(scores.data_ptr(), B, Hkv, T, ld_s, tau.data_ptr(), recent,
                                      *args), "kvp_select_dev_tau")
    else:
        _ok(load().kvp_select(scores.data_ptr(), B, Hkv, T, ld_s, float(tau), recent, *args),
            "kvp_select")


def kvp_prefill_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, keep_bits: torch.Tensor,
                     kept_idx: torch.Tensor, window: int, sm_scale: float, out: torch.Tensor,
                     stream=None) -> torch.Tensor:
    """q [B, Hq, T, d], k/v [B, Hkv, T, d] bf16; keep_bits [B*Hkv, ceil(T/32)] and
    kept_idx [B*Hkv, T] (as written by kvp_select) -> out [B, Hq, T, d] fp32."""
    _cuda(q, k, v, keep_bits, kept_idx, out)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    assert tuple(k.shape) == (B, Hkv, T, d) and k.shape == v.shape and tuple(out.shape) == (B, Hq, T, d)
    assert q.dtype == k.dtype == v.dtype and out.dtype == torch.float32
    assert all(t.is_contiguous() for t in (q, k, v, keep_bits, kept_idx, out))
    assert keep_bits.numel() >= B * Hkv * ((T + 31) // 32) and kept_idx.numel() >= B * Hkv * T
    _ok(load().kvp_prefill_attn(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dt(q), B, Hq, Hkv, T, d,
                                keep_bits.data_ptr(), kept_idx.data_ptr(), int(window),
                                float(sm_scale), out.data_ptr(), _stream(stream)),
        "kvp_prefill_attn")
    return out


def kvp_threshold_workspace_size() -> int:
    return load().kvp_threshold_workspace_size()


def kvp_threshold(scores: torch.Tensor, T: int, q: float, tau_out: torch.Tensor,
                  ws: torch.Tensor, stream=None) -> torch.Tensor:
    """tau_out[0] = fp32 q-quantile (numpy "linear") of scores[:, :, :T], on the device."""
    _cuda(scores, tau_out, ws)
    assert tau_out.dtype == torch.float32 and tau_out.numel() >= 1
    B, Hkv, ld_s = scores.shape
    _ok(load().kvp_threshold(scores.data_ptr(), B, Hkv, T, ld_s, float(q), tau_out.data_ptr(),
                             ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)),
        "kvp_threshold")
    return tau_out


def kvp_compact_workspace_size(B: int, Hkv: int) -> int:
    return load().kvp_compact_workspace_size(B, Hkv)


def kvp_compact(k: torch.Tensor, v: torch.Tensor, kept_idx: torch.Tensor,
                kept_count: torch.Tensor, kv: PagedKV, ws: torch.Tensor,
                ring: Optional[Ring] = None, scores: Optional[torch.Tensor] = None,
                mode: int = KVP_COMPACT_EVICT, stream=None):
    """Dense k, v [B, Hkv, T, d] -> paged cache (and ring)."""
    _cuda(k, v, kept_idx, kept_count, ws, scores)
    B, Hkv, T, d = k.shape
    ld_s = scores.shape[-1] if scores is not None else 0
    _ok(load().kvp_compact(k.data_ptr(), v.data_ptr(), _dt(k), B, Hkv, T, d, kept_idx.data_ptr(),
                           kept_count.data_ptr(), _p(scores), ld_s, mode, _kvref(kv),
                           _ringref(ring), ws.data_ptr(), ws.numel() * ws.element_size(),
                           _stream(stream)), "kvp_compact")


def kvp_step_delayed(kv: PagedKV, ring: Ring, k_new: torch.Tensor, v_new: torch.Tensor,
                     s_new: torch.Tensor, tau, p, ld_s: int = 1, stream=None):
    """Append position p: k_new, v_new [B, Hkv, d]; s_new holds pair i's score at i*ld_s.
    tau float and p int: kvp_step_delayed.  tau a one-element fp32 device tensor and p an
    int32[2] device tensor [position, 0]: kvp_step_delayed_dev, which reads both on the
    device and advances p[0] (graph-replayable)."""
    _cuda(k_new, v_new, s_new)
    if isinstance(tau, torch.Tensor) or isinstance(p, torch.Tensor):
        if not (isinstance(tau, torch.Tensor) and isinstance(p, torch.Tensor)):
            raise ValueError("device tau and device position go together")
        _cuda(tau, p)
        assert tau.dtype == torch.float32 and p.dtype == torch.int32 and p.numel() >= 2
        _ok(load().kvp_step_delayed_dev(_kvref(kv), _ringref(ring), k_new.data_ptr(),
                                        v_new.data_ptr(), _dt(k_new), s_new.data_ptr(), ld_s,
                                        tau.data_ptr(), p.data_ptr(), _stream(stream)),
            "kvp_step_delayed_dev")
    else:
        _ok(load().kvp_step_delayed(_kvref(kv), _ringref(ring), k_new.data_ptr(), v_new.data_ptr(),
                                    _dt(k_new), s_new.data_ptr(), ld_s, float(tau), p,
                                    _stream(stream)), "kvp_step_delayed")


def kvp_score_step_delayed(scorer: Scorer, hidden_new: torch.Tensor, kv: PagedKV, ring: Ring,
                           k_new: torch.Tensor, v_new: torch.Tensor, tau: torch.Tensor,
                           pos: torch.Tensor, s_new: Optional[torch.Tensor] = None,
                           ws: Optional[torch.Tensor] = None, stream=None):
    """Score the new tokens inside the delayed step: hidden_new [B, 1, H] (or [B, H]) in
    the scorer's dtype, k_new / v_new [B, Hkv, d]; tau (fp32[1]) and pos (int32[2]) on the
    device as for kvp_step_delayed_dev; s_new (optional, fp32, B*Hkv elements) receives
    the new tokens' scores; ws: the MLP scorer's workspace (kvp_score_workspace_size for
    B tokens), unused by a linear scorer."""
    _cuda(hidden_new, k_new, v_new, tau, pos, s_new, ws)
    assert tau.dtype == torch.float32 and pos.dtype == torch.int32 and pos.numel() >= 2
    if s_new is not None:
        assert s_new.dtype == torch.float32 and s_new.numel() >= kv.c.num_pairs
    _ok(load().kvp_score_step_delayed(ctypes.byref(scorer.c), hidden_new.data_ptr(),
                                      _dt(hidden_new), _kvref(kv), _ringref(ring),
                                      k_new.data_ptr(), v_new.data_ptr(), _dt(k_new), _p(s_new),
                                      tau.data_ptr(), pos.data_ptr(), _p(ws),
                                      0 if ws is None else ws.numel() * ws.element_size(),
                                      _stream(stream)),
        "kvp_score_step_delayed")


def kvp_decode_attn_workspace_size(B: int, Hq: int, num_pairs: int, head_dim: int) -> int:
    return load().kvp_decode_attn_workspace_size(B, Hq, num_pairs, head_dim)


def decode_attn_workspace(B: int, Hq: int, kv: PagedKV, device="cuda") -> torch.Tensor:
    """A workspace of the size kvp_decode_attn needs (contents are scratch)."""
    n = kvp_decode_attn_workspace_size(B, Hq, kv.c.num_pairs, kv.c.head_dim)
    return torch.empty(max(n, 4) // 4 + 1, dtype=torch.int32, device=device)


def kvp_decode_attn(q: torch.Tensor, kv: PagedKV, ring: Optional[Ring], sm_scale: float,
                    out: torch.Tensor, ws: torch.Tensor, stream=None) -> torch.Tensor:
    """q [B, Hq, d] -> out [B, Hq, d] fp32."""
    _cuda(q, out, ws)
    B, Hq, _ = q.shape
    _ok(load().kvp_decode_attn(q.data_ptr(), _dt(q), B, Hq, _kvref(kv), _ringref(ring),
                               float(sm_scale), out.data_ptr(), ws.data_ptr(),
                               ws.numel() * ws.element_size(), _stream(stream)),
        "kvp_decode_attn")
    return out


def kvp_decode_attn_noalloc(q: torch.Tensor, kv: PagedKV, ring: Optional[Ring], sm_scale: float,
                            out: torch.Tensor, stream=None) -> torch.Tensor:
    """kvp_decode_attn on the library's fixed per-GPU scratch (no workspace argument)."""
    _cuda(q, out)
    B, Hq, _ = q.shape
    _ok(load().kvp_decode_attn_noalloc(q.data_ptr(), _dt(q), B, Hq, _kvref(kv), _ringref(ring),
                                       float(sm_scale), out.data_ptr(), _stream(stream)),
        "kvp_decode_attn_noalloc")
    return out


KVP_NOALLOC_SCRATCH_BYTES = 64 << 20


def kvp_decode_step_workspace_size(scorer: Optional["Scorer"], B: int, Hq: int, num_pairs: int,
                                   head_dim: int) -> int:
    return load().kvp_decode_step_workspace_size(None if scorer is None else ctypes.byref(scorer.c),
                                                 B, Hq, num_pairs, head_dim)


def decode_step_workspace(scorer: Optional["Scorer"], B: int, Hq: int, kv: PagedKV,
                          device="cuda") -> torch.Tensor:
    """A workspace of the size kvp_decode_step needs (contents are scratch)."""
    n = kvp_decode_step_workspace_size(scorer, B, Hq, kv.c.num_pairs, kv.c.head_dim)
    return torch.empty(max(n, 4) // 4 + 1, dtype=torch.int32, device=device)


def kvp_decode_step(scorer: Optional["Scorer"], hidden_new: Optional[torch.Tensor], kv: PagedKV,
                    ring: Ring, k_new: torch.Tensor, v_new: torch.Tensor, tau: torch.Tensor,
                    pos: torch.Tensor, q: torch.Tensor, sm_scale: float, out: torch.Tensor,
                    ws: torch.Tensor, s_in: Optional[torch.Tensor] = None, ld_s: int = 1,
                    s_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One fused decode step: the delayed step (new tokens scored by `scorer` from
    hidden_new, or read from s_in[pair * ld_s] when scorer is None) and the attention of
    q [B, Hq, d] over the cache it leaves -> out [B, Hq, d] fp32."""
    _cuda(hidden_new, k_new, v_new, tau, pos, q, out, ws, s_in, s_out)
    assert tau.dtype == torch.float32 and pos.dtype == torch.int32 and pos.numel() >= 2
    B, Hq, _ = q.shape
    _ok(load().kvp_decode_step(None if scorer is None else ctypes.byref(scorer.c),
                               _p(hidden_new), 0 if hidden_new is None else _dt(hidden_new),
                               _kvref(kv), _ringref(ring), k_new.data_ptr(), v_new.data_ptr(),
                               _p(s_in), ld_s, _p(s_out), tau.data_ptr(), pos.data_ptr(),
                               q.data_ptr(), _dt(q), B, Hq, float(sm_scale), out.data_ptr(),
                               ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)),
        "kvp_decode_step")
    return out


def kvp_reset(kv: PagedKV, ring: Optional[Ring] = None, stream=None):
    _ok(load().kvp_reset(_kvref(kv), _ringref(ring), _stream(stream)), "kvp_reset")


def kvp_clear_error(kv: PagedKV, stream=None):
    _ok(load().kvp_clear_error(_kvref(kv), _stream(stream)), "kvp_clear_error")


def kvp_check(kv: PagedKV, stream=None) -> int:
    """Synchronises; returns the status (KVP_E_CAPACITY = 4 if a pool overflowed)."""
    return load().kvp_check(_kvref(kv), _stream(stream))


def sm_scale(d: int) -> float:
    """1/sqrt(d) rounded to fp32, as passed to the kernels."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
