"""C-ABI checks that need no GPU: the library builds and loads, exports every function
include/kvp.h declares, the ctypes struct layouts match the C compiler's, and the
host-side argument validation returns the documented status codes before anything
touches a device.  Also guards that the product path never reaches the oracle."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvp.h")
PKG = os.path.join(ROOT, "sparse_decode_attention_kvzap_amd")


@pytest.fixture(scope="module")
def L():
    import torch  # noqa: F401  (load torch's HIP runtime first, as the package does)
    from sparse_decode_attention_kvzap_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from sparse_decode_attention_kvzap_amd import build
        build.build()
    _lib.load()
    return _lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvp_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("kvp_score", "kvp_select", "kvp_compact", "kvp_decode_attn", "kvp_step_delayed"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    lib = L.load()
    for n in declared_functions():
        assert getattr(lib, n) is not None


PROBE_C = r"""
#include <stdio.h>
#include <stddef.h>
#include "kvp.h"
#define F(T, f) printf(#T "." #f " %zu\n", offsetof(T, f))
int main(void) {
  printf("kvp_scorer %zu\n", sizeof(kvp_scorer));
  printf("kvp_paged_kv %zu\n", sizeof(kvp_paged_kv));
  printf("kvp_ring %zu\n", sizeof(kvp_ring));
  F(kvp_scorer, w1); F(kvp_scorer, b2);
  F(kvp_paged_kv, k_pages); F(kvp_paged_kv, err); F(kvp_paged_kv, k8_pages);
  F(kvp_paged_kv, lp_bits);
  F(kvp_paged_kv, page8_top);
  F(kvp_ring, k); F(kvp_ring, pos);
  return 0;
}
"""


def test_struct_layouts_match_c(L, tmp_path):
    src = tmp_path / "probe.c"
    src.write_text(PROBE_C)
    exe = tmp_path / "probe"
    r = subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("cannot compile the C probe here: " + r.stderr[-300:])
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True,
                                                       text=True, check=True).stdout.splitlines())
    assert int(got["kvp_scorer"]) == ctypes.sizeof(L.KvpScorer)
    assert int(got["kvp_paged_kv"]) == ctypes.sizeof(L.KvpPagedKV)
    assert int(got["kvp_ring"]) == ctypes.sizeof(L.KvpRing)
    for key, val in got.items():
        if "." in key:
            t, f = key.split(".")
            cls = {"kvp_scorer": L.KvpScorer, "kvp_paged_kv": L.KvpPagedKV, "kvp_ring": L.KvpRing}[t]
            assert getattr(cls, f).offset == int(val), key


def test_status_strings_and_version(L):
    for code, name in L.STATUS.items():
        assert L.kvp_status_str(code).startswith(name)
    assert L.kvp_status_str(99) == "KVP_E_UNKNOWN"
    assert "gfx950" in L.kvp_version()


def test_workspace_sizes(L):
    assert L.kvp_select_workspace_size(16, 8, 32768) == 16 * 8 * 16 * 4
    assert L.kvp_select_workspace_size(0, 8, 10) == 0
    assert L.kvp_compact_workspace_size(16, 8) >= (6 * 128 + 1) * 4
    n = L.kvp_decode_attn_workspace_size(16, 32, 128, 128)
    assert n >= 128 * 4 * 130 * 4
    assert L.kvp_decode_attn_workspace_size(16, 30, 128, 128) == 0  # Hq % Hkv != 0
    sc = L.KvpScorer(L.KVP_SCORER_MLP, 4096, 512, 8, L.KVP_BF16, 0, 1, 0, 1, 0)
    assert L.load().kvp_score_workspace_size(ctypes.byref(sc), 16, 100) == 2 * 16 * 100 * 16 * 4
    sc.kind = L.KVP_SCORER_LINEAR
    assert L.load().kvp_score_workspace_size(ctypes.byref(sc), 16, 100) == 0


def test_host_validation_without_device(L):
    lib = L.load()
    E_ARG, E_DTYPE, E_WS, E_UNSUP = 1, 2, 3, 6
    fake = 0x1000  # never dereferenced: every case below fails validation first
    # null pointers
    assert lib.kvp_select(None, 1, 1, 10, 10, 0.0, 128, None, None, None, None, 0, None) == E_ARG
    assert lib.kvp_decode_attn(None, 1, 1, 4, None, None, 0.1, None, None, 0, None) == E_ARG
    assert lib.kvp_score(None, None, 1, 1, 1, None, 1, None, 0, None) == E_ARG
    assert lib.kvp_reset(None, None, None) == E_ARG
    assert lib.kvp_clear_error(None, None) == E_ARG
    assert lib.kvp_check(None, None) == E_ARG
    assert lib.kvp_step_delayed(None, None, None, None, 1, None, 1, 0.0, 0, None) == E_ARG
    # select: bad sizes, undersized workspace
    assert lib.kvp_select(fake, 1, 1, 10, 5, 0.0, 128, fake, fake, fake, fake, 64, None) == E_ARG
    assert lib.kvp_select(fake, 1, 1, 10, 10, 0.0, -1, fake, fake, fake, fake, 64, None) == E_ARG
    assert lib.kvp_select(fake, 1, 1, 10, 10, 0.0, 128, fake, fake, fake, fake, 0, None) == E_WS
    # score: dtype mismatch, unsupported MLP shapes, missing workspace
    sc = L.KvpScorer(L.KVP_SCORER_LINEAR, 64, 0, 2, L.KVP_BF16, 0, fake, 0, 0, 0)
    assert lib.kvp_score(ctypes.byref(sc), fake, L.KVP_F32, 1, 4, fake, 4, None, 0, None) == E_DTYPE
    sc.n_kv_heads = 17
    assert lib.kvp_score(ctypes.byref(sc), fake, L.KVP_BF16, 1, 4, fake, 4, None, 0, None) == E_UNSUP
    sc = L.KvpScorer(L.KVP_SCORER_MLP, 100, 512, 8, L.KVP_BF16, 0, fake, 0, fake, 0)
    assert lib.kvp_score(ctypes.byref(sc), fake, L.KVP_BF16, 1, 4, fake, 4, None, 0, None) == E_UNSUP
    sc.hidden = 128
    assert lib.kvp_score(ctypes.byref(sc), fake, L.KVP_BF16, 1, 4, fake, 4, None, 0, None) == E_WS
    # paged cache descriptor checks
    kv = L.KvpPagedKV()
    kv.dtype, kv.num_pairs, kv.head_dim, kv.num_pages, kv.max_pages_per_pair = L.KVP_BF16, 4, 96, 8, 2
    for f in ("k_pages", "v_pages", "page_pos", "block_table", "length", "page_top", "err"):
        setattr(kv, f, fake)
    assert lib.kvp_reset(ctypes.byref(kv), None, None) == E_UNSUP  # head_dim 96
    kv.head_dim = 128
    kv.dtype = 7
    assert lib.kvp_reset(ctypes.byref(kv), None, None) == E_DTYPE
    kv.dtype = L.KVP_BF16
    ring = L.KvpRing(100, 0, fake, fake, fake, fake)  # window not a multiple of 16
    assert lib.kvp_reset(ctypes.byref(kv), ctypes.byref(ring), None) == E_ARG
    # attention: Hq not a multiple of Hkv, g > 16, dtype mismatch, workspace
    assert lib.kvp_decode_attn(fake, L.KVP_BF16, 1, 6, ctypes.byref(kv), None, 0.1, fake, fake,
                               1 << 20, None) == E_ARG
    assert lib.kvp_decode_attn(fake, L.KVP_BF16, 1, 68, ctypes.byref(kv), None, 0.1, fake, fake,
                               1 << 20, None) == E_UNSUP
    assert lib.kvp_decode_attn(fake, L.KVP_F32, 1, 8, ctypes.byref(kv), None, 0.1, fake, fake,
                               1 << 20, None) == E_DTYPE
    assert lib.kvp_decode_attn(fake, L.KVP_BF16, 1, 8, ctypes.byref(kv), None, 0.1, fake, fake,
                               16, None) == E_WS
    # a low-precision pool with a code width other than 8 or 4
    kv.num_pages8, kv.max_pages8_per_pair = 4, 4
    for name in ("k8_pages", "v8_pages", "k8_scale", "v8_scale", "page8_pos", "block_table8",
                 "length8", "page8_top"):
        setattr(kv, name, fake)
    for bad in (3, 0x18, 0x208):  # not int8, int4 or fp8 E4M3
        kv.lp_bits = bad
        assert lib.kvp_reset(ctypes.byref(kv), None, None) == E_ARG
    kv.lp_bits = 4
    kv.num_pages8, kv.max_pages8_per_pair = 0, 0
    # compact: demotion without an int8 pool, wrong pair count
    assert lib.kvp_compact(fake, fake, L.KVP_BF16, 1, 4, 64, 128, fake, fake, None, 0,
                           L.KVP_COMPACT_DEMOTE_INT8, ctypes.byref(kv), None, fake, 1 << 16,
                           None) == E_ARG
    assert lib.kvp_compact(fake, fake, L.KVP_BF16, 1, 3, 64, 128, fake, fake, None, 0,
                           L.KVP_COMPACT_EVICT, ctypes.byref(kv), None, fake, 1 << 16, None) == E_ARG
    # threshold: null pointers, q outside [0, 1] or NaN, too many scores, workspace
    thr_ws = L.kvp_threshold_workspace_size()
    assert thr_ws == 64 + 3 * 8 * 2 * 2048 * 4
    assert lib.kvp_threshold(None, 1, 1, 10, 10, 0.5, fake, fake, thr_ws, None) == E_ARG
    assert lib.kvp_threshold(fake, 1, 1, 10, 10, 0.5, None, fake, thr_ws, None) == E_ARG
    for q in (-0.1, 1.5, float("nan")):
        assert lib.kvp_threshold(fake, 1, 1, 10, 10, q, fake, fake, thr_ws, None) == E_ARG
    assert lib.kvp_threshold(fake, 1, 1, 10, 5, 0.5, fake, fake, thr_ws, None) == E_ARG  # ld_s < T
    assert lib.kvp_threshold(fake, 65535, 1, 1 << 17, 1 << 17, 0.5, fake, fake, thr_ws,
                             None) == E_UNSUP
    assert lib.kvp_threshold(fake, 1, 1, 10, 10, 0.5, fake, fake, thr_ws - 1, None) == E_WS
    # device-tau variants need the tau pointer
    assert lib.kvp_select_dev_tau(fake, 1, 1, 10, 10, None, 128, fake, fake, fake, fake, 64,
                                  None) == E_ARG
    # step: position must be >= 0
    ring = L.KvpRing(64, 0, fake, fake, fake, fake)
    assert lib.kvp_step_delayed(ctypes.byref(kv), ctypes.byref(ring), fake, fake, L.KVP_BF16, fake,
                                1, 0.0, -1, None) == E_ARG
    assert lib.kvp_step_delayed_dev(ctypes.byref(kv), ctypes.byref(ring), fake, fake,
                                    L.KVP_BF16, fake, 1, None, fake, None) == E_ARG
    assert lib.kvp_step_delayed_dev(ctypes.byref(kv), ctypes.byref(ring), fake, fake,
                                    L.KVP_BF16, fake, 1, fake, None, None) == E_ARG
    # fused score + step: matching dtypes, 16-byte rows, a pair count divisible by Hkv,
    # device tau and position; MLP scorers of the small-batch shapes with a workspace
    sst = lib.kvp_score_step_delayed
    kr = (ctypes.byref(kv), ctypes.byref(ring), fake, fake)
    lin = L.KvpScorer(L.KVP_SCORER_LINEAR, 4096, 0, 2, L.KVP_BF16, 0, fake, 0, 0, 0)
    mlp = L.KvpScorer(L.KVP_SCORER_MLP, 4096, 512, 2, L.KVP_BF16, 0, fake, 0, fake, 0)

    def call(sc, x=fake, hdt=L.KVP_BF16, dt=L.KVP_BF16, tau=fake, pos=fake, ws=None, nws=0):
        return sst(None if sc is None else ctypes.byref(sc), x, hdt, *kr, dt, None, tau, pos,
                   ws, nws, None)
    assert call(lin, hdt=L.KVP_F32) == E_DTYPE
    assert call(lin, dt=L.KVP_F32) == E_DTYPE
    assert call(lin, x=fake + 2) == E_ARG
    assert call(lin, tau=None) == E_ARG
    assert call(lin, pos=None) == E_ARG
    assert call(None) == E_ARG
    lin.hidden = 4100  # rows of 8200 bytes are not read in 16-byte pieces
    assert call(lin) == E_UNSUP
    lin.hidden, lin.n_kv_heads = 4096, 3  # 4 pairs are not B x 3 heads
    assert call(lin) == E_ARG
    assert call(mlp) == E_WS  # no workspace for the first layer's partial sums
    assert call(mlp, ws=fake + 4, nws=1 << 20) == E_ARG  # misaligned workspace
    mlp.inner = 384  # the finish takes widths in multiples of 256
    assert call(mlp, ws=fake, nws=1 << 20) == E_UNSUP
    mlp.inner, mlp.hidden = 512, 4000  # the split-K slices are 256 wide
    assert call(mlp, ws=fake, nws=1 << 20) == E_UNSUP
    mlp.hidden, mlp.wdtype = 4096, L.KVP_F32
    assert call(mlp, hdt=L.KVP_F32, ws=fake, nws=1 << 20) == E_UNSUP
    # prefill attention: nulls, fp32 (not built), bad dtype, head ratio, head dim, window
    pf = lib.kvp_prefill_attn
    assert pf(None, fake, fake, L.KVP_BF16, 1, 8, 2, 64, 128, fake, fake, 16, 0.1, fake, None) == E_ARG
    assert pf(fake, fake, fake, L.KVP_BF16, 1, 8, 2, 64, 128, fake, None, 16, 0.1, fake, None) == E_ARG
    assert pf(fake, fake, fake, L.KVP_F32, 1, 8, 2, 64, 128, fake, fake, 16, 0.1, fake, None) == E_UNSUP
    assert pf(fake, fake, fake, 9, 1, 8, 2, 64, 128, fake, fake, 16, 0.1, fake, None) == E_DTYPE
    assert pf(fake, fake, fake, L.KVP_BF16, 1, 6, 4, 64, 128, fake, fake, 16, 0.1, fake, None) == E_ARG
    assert pf(fake, fake, fake, L.KVP_BF16, 1, 64, 2, 64, 128, fake, fake, 16, 0.1, fake, None) == E_UNSUP
    assert pf(fake, fake, fake, L.KVP_BF16, 1, 12, 4, 64, 128, fake, fake, 16, 0.1, fake, None) == E_UNSUP
    assert pf(fake, fake, fake, L.KVP_BF16, 1, 8, 2, 64, 96, fake, fake, 16, 0.1, fake, None) == E_UNSUP
    assert pf(fake, fake, fake, L.KVP_BF16, 1, 8, 2, 64, 128, fake, fake, -1, 0.1, fake, None) == E_ARG
    assert pf(fake, fake, fake, L.KVP_BF16, 1, 8, 2, 0, 128, fake, fake, 16, 0.1, fake, None) == E_ARG
    for bad in (0.0, -0.1, float("inf"), float("nan")):
        assert pf(fake, fake, fake, L.KVP_BF16, 1, 8, 2, 64, 128, fake, fake, 16, bad, fake, None) == E_ARG


def test_missing_library_fails_loudly(L, tmp_path):
    saved = L._lib
    try:
        L._lib = None
        with pytest.raises(ImportError):
            L.load(str(tmp_path / "nope.so"))
    finally:
        L._lib = saved


def test_product_path_never_imports_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "oracle/" not in text, f
