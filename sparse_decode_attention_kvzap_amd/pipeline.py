"""One attention layer's pruned KV cache driven through the five C-ABI calls.

Prefill (compress a context):  kvp_score -> [kvp_threshold] -> kvp_select -> kvp_compact
Decode step (one new token):   kvp_score -> kvp_step_delayed -> kvp_decode_attn

tau is either a fixed float or, after calibrate(q), a one-element device tensor holding
the q-quantile of the prompt's scores (computed on the device), which select and the
delayed step then read without a host round trip.

KVzap (max5.ai digest, practical application): score every entry, drop low scores,
always keep the most recent tokens.  DMS (euno.news, Delayed Eviction): with tau = 0
and window w the same machinery keeps a flagged token for w steps.  BeaconKV
(jiinsi.com, body): with demote=True evicted entries go to a low-precision pool
instead (int8 codes, int4 with lp_bits=4, or fp8 E4M3 with lp_bits="fp8").

This class only allocates device buffers (torch) and calls libkvp in stream order;
all arithmetic runs in the HIP kernels.
"""
from __future__ import annotations

import contextlib
from typing import Optional

import torch

from . import _lib as L


class PrunedKVCache:
    def __init__(self, B: int, Hkv: int, Hq: int, d: int, T_max: int, dtype: torch.dtype,
                 scorer: L.Scorer, window: int, tau: float, demote: bool = False,
                 device="cuda", max_prompt: Optional[int] = None, lp_bits=8):
        self.B, self.Hkv, self.Hq, self.d = B, Hkv, Hq, d
        self.P = B * Hkv
        self.T_max = T_max
        self.dtype = dtype
        self.scorer = scorer
        self.window = window
        self.tau = float(tau)  # or a device tensor after calibrate()
        self.demote = demote
        self.device = torch.device(device)
        dev = self.device
        Tp = max_prompt or T_max
        self.Tp = Tp
        maxpp = -(-T_max // L.KVP_PAGE) + 1
        kw = {}
        if demote:
            kw = dict(num_pages8=self.P * maxpp, max_pages8_per_pair=maxpp, lp_bits=lp_bits)
        self.kv = L.PagedKV.allocate(self.P, d, self.P * maxpp, maxpp, dtype, dev, **kw)
        self.ring = L.Ring.allocate(self.P, window, d, dtype, dev)
        self.scores = torch.empty((B, Hkv, Tp), dtype=torch.float32, device=dev)
        self.s_new = torch.empty((B, Hkv, 1), dtype=torch.float32, device=dev)
        self.keep_bits = torch.empty((self.P, -(-Tp // 32)), dtype=torch.int32, device=dev)
        self.kept_idx = torch.empty((self.P, Tp), dtype=torch.int32, device=dev)
        self.kept_count = torch.empty((self.P,), dtype=torch.int32, device=dev)
        self.ws_select = torch.empty(max(1, L.kvp_select_workspace_size(B, Hkv, Tp) // 4),
                                     dtype=torch.int32, device=dev)
        self.ws_compact = torch.empty(L.kvp_compact_workspace_size(B, Hkv) // 4,
                                      dtype=torch.int32, device=dev)
        nws = max(L.kvp_score_workspace_size(scorer, B, Tp), L.kvp_score_workspace_size(scorer, B, 1))
        self.ws_score = torch.empty(max(1, nws // 4), dtype=torch.float32, device=dev)
        self.ws_attn = L.decode_attn_workspace(B, Hq, self.kv, dev)
        self.out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
        self.scale = L.sm_scale(d)
        self.tau_dev = torch.full((1,), float(tau), dtype=torch.float32, device=dev)
        self.pos_dev = torch.zeros(2, dtype=torch.int32, device=dev)  # [next position, 0]
        self.ws_threshold = torch.empty(L.kvp_threshold_workspace_size() // 4 + 1,
                                        dtype=torch.int32, device=dev)
        self.T0 = 0
        c = scorer.c
        self._fused_score = (c.kind == L.KVP_SCORER_LINEAR and c.hidden % 8 == 0) or (
            c.wdtype == L.KVP_BF16 and B <= 64 and c.hidden % 256 == 0 and c.hidden <= 8192
            and c.inner % 256 == 0 and c.inner <= 1024)
        # one fused call per decode step (kvp_decode_step) for a bf16 cache without a
        # low-precision pool; otherwise step() makes the separate calls
        self.fused_step = dtype == torch.bfloat16 and not demote
        self.ws_step = (L.decode_step_workspace(scorer if self._fused_score else None, B, Hq,
                                                self.kv, dev) if self.fused_step else None)

    # -- prefill -----------------------------------------------------------------
    def score(self, hidden: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None):
        return L.kvp_score(self.scorer, hidden, self.scores if out is None else out,
                           self.ws_score, stream)

    def calibrate(self, q: float, T: int, stream=None) -> torch.Tensor:
        """tau := the q-quantile of scores[:, :, :T], on the device (keep ~ 1 - q)."""
        L.kvp_threshold(self.scores, T, q, self.tau_dev, self.ws_threshold, stream)
        self.tau = self.tau_dev
        return self.tau_dev

    def select(self, T: int, stream=None):
        L.kvp_select(self.scores, T, self.tau, self.window, self.keep_bits, self.kept_idx,
                     self.kept_count, self.ws_select, stream)

    def prefill_attention(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                          out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """Attention of every prompt position under the current selection (call select(T)
        first): position i sees key j iff j <= i and (j is kept or i - j < window).
        q [B, Hq, T, d], k/v [B, Hkv, T, d] bf16 -> out [B, Hq, T, d] fp32."""
        if self.demote:
            raise ValueError("a demoting cache evicts nothing: its prompt attends densely")
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        # select(T) wrote keep_bits as [P][ceil(T/32)] and kept_idx as [P][T], packed
        return L.kvp_prefill_attn(q, k, v, self.keep_bits, self.kept_idx, self.window, self.scale,
                                  out, stream)

    def compact(self, k: torch.Tensor, v: torch.Tensor, stream=None):
        L.kvp_compact(k, v, self.kept_idx, self.kept_count, self.kv, self.ws_compact,
                      ring=self.ring, scores=self.scores,
                      mode=L.KVP_COMPACT_DEMOTE_INT8 if self.demote else L.KVP_COMPACT_EVICT,
                      stream=stream)

    def prefill(self, hidden: torch.Tensor, k: torch.Tensor, v: torch.Tensor, stream=None):
        """Compress a context of T = hidden.shape[1] tokens (positions 0..T-1)."""
        T = hidden.shape[1]
        self.score(hidden, stream=stream)
        self.select(T, stream)
        self.compact(k, v, stream)
        self.T0 = T

    # -- decode ------------------------------------------------------------------
    @staticmethod
    def _on(stream):
        """Run torch's own writes (fills) on `stream` too, so they stay in order with the
        library calls made on it.  A raw handle is wrapped; None is torch's current stream."""
        if stream is None:
            return contextlib.nullcontext()
        if not isinstance(stream, torch.cuda.Stream):
            stream = torch.cuda.ExternalStream(int(stream))
        return torch.cuda.stream(stream)

    def set_tau(self, tau: float, stream=None):
        """A fixed threshold (also mirrored to the device copy the decode step reads)."""
        self.tau = float(tau)
        with self._on(stream):
            self.tau_dev.fill_(self.tau)

    def set_position(self, p: int, stream=None):
        """The absolute position the next decode step appends (kept on the device)."""
        with self._on(stream):
            self.pos_dev[0] = p
            self.pos_dev[1] = 0

    def advance(self, hidden_new: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                p: Optional[int] = None, stream=None):
        """Append a position (p, or the device-held next position when p is None): score
        the new tokens and run the delayed step.  The scoring runs inside the step
        (kvp_score_step_delayed) for a linear scorer, and for an MLP scorer of the shapes
        that call takes (bf16, B <= 64, H and the width multiples of 256); otherwise
        kvp_score runs first."""
        if p is not None:
            self.set_position(p, stream)
        if not isinstance(self.tau, torch.Tensor):
            with self._on(stream):
                self.tau_dev.fill_(self.tau)
        if self._fused_score:
            L.kvp_score_step_delayed(self.scorer, hidden_new, self.kv, self.ring, k_new, v_new,
                                     self.tau_dev, self.pos_dev, self.s_new, self.ws_score, stream)
        else:
            L.kvp_score(self.scorer, hidden_new, self.s_new, self.ws_score, stream)
            L.kvp_step_delayed(self.kv, self.ring, k_new, v_new, self.s_new, self.tau_dev,
                               self.pos_dev, 1, stream)

    def step(self, hidden_new: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
             q: torch.Tensor, p: Optional[int] = None, stream=None) -> torch.Tensor:
        """Append a position (see advance) and attend with q over the cache that now holds
        it: one kvp_decode_step call (plus kvp_score first when the scorer's shape is not
        one the step scores itself) for a bf16 cache without a low-precision pool, else
        advance() then attend().  Every per-step value lives in device memory, so this
        sequence can be captured in a HIP graph and replayed."""
        if not self.fused_step:
            self.advance(hidden_new, k_new, v_new, p, stream)
            return self.attend(q, stream)
        if p is not None:
            self.set_position(p, stream)
        if not isinstance(self.tau, torch.Tensor):
            with self._on(stream):
                self.tau_dev.fill_(self.tau)
        if self._fused_score:
            L.kvp_decode_step(self.scorer, hidden_new, self.kv, self.ring, k_new, v_new,
                              self.tau_dev, self.pos_dev, q, self.scale, self.out, self.ws_step,
                              s_out=self.s_new, stream=stream)
        else:
            L.kvp_score(self.scorer, hidden_new, self.s_new, self.ws_score, stream)
            L.kvp_decode_step(None, None, self.kv, self.ring, k_new, v_new, self.tau_dev,
                              self.pos_dev, q, self.scale, self.out, self.ws_step, s_in=self.s_new,
                              stream=stream)
        return self.out

    def attend(self, q: torch.Tensor, stream=None) -> torch.Tensor:
        L.kvp_decode_attn(q, self.kv, self.ring, self.scale, self.out, self.ws_attn, stream)
        return self.out

    def visible_token_heads(self) -> int:
        """Token-heads the next decode attention reads (pool + ring + low-precision pool)."""
        n = int(self.kv.length.sum()) + int((self.ring.pos >= 0).sum())
        if self.demote:
            n += int(self.kv.length8.sum())
        return n

    def check(self, stream=None) -> int:
        return L.kvp_check(self.kv, stream)
