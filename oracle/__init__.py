"""fp64 CPU oracle for paged decode attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``pda_oracle.c`` (plain C,
fp64, OpenMP over (sequence, head) rows) with ctypes and numpy.  It shares no
code with the HIP path and does not import it.

Inputs are numpy arrays that hold the *stored bytes* the GPU would read:

  dtype name  numpy array dtype   meaning
  ----------  -----------------   -----------------------------------
  "f32"       float32             IEEE binary32
  "f16"       float16             IEEE binary16
  "bf16"      uint16              bfloat16 bit patterns
  "e4m3"      uint8               OCP FP8 E4M3FN bit patterns
  "f64"       float64             (oracle-only, for pins)

What is computed is the plain definition (see the header of pda_oracle.c):
softmax(scale * q K^T) V over the tokens gathered through the block table,
with the natural-log LSE of the scaled logits.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_DT = {"f32": 0, "f16": 1, "bf16": 2, "e4m3": 3, "f64": 4}
_NP = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "e4m3": np.uint8,
       "f64": np.float64}
_ERR = {1: "invalid argument", 2: "block-table entry out of range", 3: "out of memory"}

_lib = None
_lib_path = None   # None: the library built from oracle/pda_oracle.c


def use_library(path):
    """Point the wrappers at another build of the oracle (the mutation tests
    load copies with planted mistakes); ``None`` restores the default."""
    global _lib, _lib_path
    _lib, _lib_path = None, path


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _lib_path
    if path is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    I64 = ctypes.c_int64
    D = ctypes.c_double
    lib.orc_decode.argtypes = [I, P, I64, I64, P]
    lib.orc_paged_attention.argtypes = [P, I, P, P, I, P, I, P, P, P, I, I, I, I, I, I, I,
                                        I64, D, D, D, I, P, P, P, I]
    lib.orc_mla_attention.argtypes = [P, I, P, I, P, I, P, P, P, I, I, I, I, I, I, I64, D, D,
                                      I, P, P, P, I]
    lib.orc_combine.argtypes = [P, P, I64, I, I, P, P]
    lib.orc_kv_append.argtypes = [P, I, P, I, P, I, P, I, I, I, I, I, I64, ctypes.c_float]
    lib.orc_max_threads.argtypes = []
    for f in (lib.orc_decode, lib.orc_paged_attention, lib.orc_mla_attention, lib.orc_combine,
              lib.orc_kv_append, lib.orc_max_threads):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc):
    if rc != 0:
        raise ValueError("oracle: " + _ERR.get(rc, "error %d" % rc))


def _as(a, name):
    a = np.ascontiguousarray(a)
    want = _NP[name]
    if a.dtype != want:
        raise TypeError("expected %s storage (%s), got %s" % (name, want, a.dtype))
    return a


def max_threads() -> int:
    return _load().orc_max_threads()


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Decode stored elements to float64 with the oracle's own decoders."""
    a = _as(bits, dtype).reshape(-1)
    out = np.empty(a.size, dtype=np.float64)
    _check(_load().orc_decode(_DT[dtype], _ptr(a), 0, a.size, _ptr(out)))
    return out.reshape(np.shape(bits))


def _i32(a, n=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=np.int32)
    if n is not None and a.size != n:
        raise ValueError("expected %d entries" % n)
    return a


def _queries(q):
    """(q as [B, s_q, H, d], s_q, whether the caller passed [B, H, d])."""
    if q.ndim == 3:
        return q[:, None], 1, True
    if q.ndim != 4:
        raise ValueError("q must be [B, H, d] or [B, s_q, H, d]")
    return q, q.shape[1], False


def _shape_result(out, lse, single):
    """out [B, s_q, H, dv] and lse [B, H, s_q] back to the caller's rank."""
    if single:
        return out[:, 0], lse[:, :, 0]
    return out, lse


def _token_major(cache, kv_layout):
    """A head-major cache [num_pages, H, P, w] as the token-major array
    [num_pages, P, H, w] that holds the same elements: element (page, slot,
    head) is addressed by its own stride in either order ("From MHA to MLA"
    sec. 5, paged loads; the drill page sec. 4)."""
    if kv_layout not in (0, 1):
        raise ValueError("kv_layout must be 0 (token-major) or 1 (head-major)")
    return np.ascontiguousarray(cache.transpose(0, 2, 1, 3)) if kv_layout else cache


def paged_attention(q, k_cache, v_cache, block_tables, context_lens, *, scale,
                    q_dtype, kv_dtype, k_scale=1.0, v_scale=1.0, causal=True,
                    tok_begin=None, tok_end=None, rows=None, num_threads=0, kv_layout=0):
    """GQA/MQA/MHA paged decode attention in fp64.

    q [B, Hq, dk] (one query token) or [B, s_q, Hq, dk] (s_q query tokens,
    the last s_q positions of the sequence); k_cache [num_pages, P, Hkv, dk];
    v_cache [num_pages, P, Hkv, dv]; block_tables [B, max_pages] int32;
    context_lens [B] int32.  causal: query i of s_q sees the first
    n - (s_q - 1 - i) tokens (bottom-right alignment); else all n.
    tok_begin/tok_end: optional [B] token interval per sequence (a split).
    rows: optional bool [B, Hq] / [B, s_q, Hq] selecting the rows to compute
    (others are NaN).
    Returns (out [B, Hq, dv], lse [B, Hq]) for a 3-D q and
    (out [B, s_q, Hq, dv], lse [B, Hq, s_q]) for a 4-D q, float64.
    kv_layout=1: the caches are head-major, [num_pages, Hkv, P, d].
    """
    q = _as(q, q_dtype)
    k_cache = _as(_token_major(np.asarray(k_cache), kv_layout), kv_dtype)
    v_cache = _as(_token_major(np.asarray(v_cache), kv_layout), kv_dtype)
    q, s_q, single = _queries(q)
    B, _, Hq, dk = q.shape
    num_pages, P, Hkv, dk2 = k_cache.shape
    dv = v_cache.shape[3]
    if dk2 != dk or v_cache.shape[:3] != k_cache.shape[:3]:
        raise ValueError("cache shapes do not match q")
    bt = _i32(block_tables)
    if bt.ndim != 2 or bt.shape[0] != B:
        raise ValueError("block_tables must be [B, max_pages]")
    cl = _i32(context_lens, B)
    tb, te = _i32(tok_begin, B), _i32(tok_end, B)
    rm = None if rows is None else np.ascontiguousarray(rows, dtype=np.uint8).reshape(-1)
    out = np.full((B, s_q, Hq, dv), np.nan)
    lse = np.full((B, Hq, s_q), np.nan)
    rc = _load().orc_paged_attention(
        _ptr(q), _DT[q_dtype], _ptr(k_cache), _ptr(v_cache), _DT[kv_dtype], _ptr(bt),
        bt.shape[1], _ptr(cl), _ptr(tb), _ptr(te), B, s_q, Hq, Hkv, dk, dv, P, num_pages,
        float(scale), float(k_scale), float(v_scale), int(bool(causal)), _ptr(rm), _ptr(out),
        _ptr(lse), int(num_threads))
    _check(rc)
    return _shape_result(out, lse, single)


def mla_attention(q, kv_cache, block_tables, context_lens, *, scale, d_latent, q_dtype,
                  kv_dtype, kv_scale=1.0, causal=True, tok_begin=None, tok_end=None,
                  rows=None, num_threads=0):
    """MLA paged decode attention in fp64.

    q [B, Hq, d_latent + d_rope] or [B, s_q, Hq, d_latent + d_rope];
    kv_cache [num_pages, P, d_latent + d_rope].  K is the whole record, V its
    first d_latent values, both times kv_scale (an fp8 latent's dequantization
    scale); s_q and causal as in paged_attention.
    Returns (out [B, Hq, d_latent], lse [B, Hq]) for a 3-D q and
    (out [B, s_q, Hq, d_latent], lse [B, Hq, s_q]) for a 4-D q, float64.
    """
    q = _as(q, q_dtype)
    kv_cache = _as(kv_cache, kv_dtype)
    q, s_q, single = _queries(q)
    B, _, Hq, rec = q.shape
    num_pages, P, rec2 = kv_cache.shape
    if rec2 != rec or not (0 < d_latent <= rec):
        raise ValueError("record widths do not match")
    bt = _i32(block_tables)
    cl = _i32(context_lens, B)
    tb, te = _i32(tok_begin, B), _i32(tok_end, B)
    rm = None if rows is None else np.ascontiguousarray(rows, dtype=np.uint8).reshape(-1)
    out = np.full((B, s_q, Hq, d_latent), np.nan)
    lse = np.full((B, Hq, s_q), np.nan)
    rc = _load().orc_mla_attention(
        _ptr(q), _DT[q_dtype], _ptr(kv_cache), _DT[kv_dtype], _ptr(bt), bt.shape[1],
        _ptr(cl), _ptr(tb), _ptr(te), B, s_q, Hq, d_latent, rec - d_latent, P, num_pages,
        float(scale), float(kv_scale), int(bool(causal)), _ptr(rm), _ptr(out), _ptr(lse),
        int(num_threads))
    _check(rc)
    return _shape_result(out, lse, single)


def combine(part_o, part_lse):
    """LSE-weighted merge of split partials: part_o [..., S, dv], part_lse [..., S]."""
    part_o = np.ascontiguousarray(part_o, dtype=np.float64)
    part_lse = np.ascontiguousarray(part_lse, dtype=np.float64)
    *lead, S, dv = part_o.shape
    if tuple(part_lse.shape) != tuple(lead) + (S,):
        raise ValueError("part_lse shape does not match part_o")
    R = int(np.prod(lead)) if lead else 1
    out = np.empty(tuple(lead) + (dv,))
    lse = np.empty(tuple(lead))
    _check(_load().orc_combine(_ptr(part_o), _ptr(part_lse), R, S, dv, _ptr(out), _ptr(lse)))
    return out, lse


def kv_append(src, cache, block_tables, positions, *, src_dtype, cache_dtype, scale=1.0,
              kv_layout=0):
    """Write s_new new tokens per sequence into a copy of one paged cache tensor.

    src [B, s_new, H, width] (or [B, s_new, width] for a headless MLA cache);
    cache [num_pages, P, H, width] (or [num_pages, P, width]); positions [B]
    int32, the position of each sequence's first new token (< 0: skipped).
    E4M3 caches store the nearest E4M3FN byte to the fp32 quotient x / scale
    (ties to even, saturated at 448).  Returns the updated copy of cache.
    kv_layout=1: cache is head-major, [num_pages, H, P, width] (returned so)."""
    if kv_layout and np.asarray(cache).ndim == 4:
        tm = kv_append(src, _token_major(np.asarray(cache), 1), block_tables, positions,
                       src_dtype=src_dtype, cache_dtype=cache_dtype, scale=scale)
        return np.ascontiguousarray(tm.transpose(0, 2, 1, 3))
    src = _as(src, src_dtype)
    out = _as(cache, cache_dtype).copy()
    if src.ndim == 3:
        src, out4 = src[:, :, None], out[:, :, None]
    else:
        out4 = out
    B, s_new, H, width = src.shape
    num_pages, P, H2, width2 = out4.shape
    if (H2, width2) != (H, width):
        raise ValueError("cache rows do not match src")
    bt = _i32(block_tables)
    pos = _i32(positions, B)
    _check(_load().orc_kv_append(_ptr(src), _DT[src_dtype], _ptr(out), _DT[cache_dtype],
                                 _ptr(bt), bt.shape[1], _ptr(pos), B, s_new, H, width, P,
                                 num_pages, float(scale)))
    return out
