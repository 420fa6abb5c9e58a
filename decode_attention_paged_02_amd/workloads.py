"""Seeded synthetic inputs for paged decode attention.

This module only draws random numbers and lays out the stored bytes of a
paged KV cache; it contains none of the attention arithmetic.  Both the fp64
oracle (in the tests) and the HIP path consume exactly the arrays it returns.

Storage conventions (numpy dtype of the returned arrays):
  "f32" float32, "f16" float16, "bf16" uint16 bit patterns,
  "e4m3" uint8 bit patterns (OCP FP8 E4M3FN).
Values are drawn in fp32 with numpy's PCG64 and rounded to the storage type
by library casts (numpy for fp16, torch for bf16 and fp8), round-to-nearest-even.

Layouts follow the pages ("From MHA to MLA" sec. 5 paged addressing; the drill
page sec. 4 cache strides; FlashMLA-ETAP "Usage" for the latent cache):
  q            [B, Hq, d]
  k/v cache    [num_pages, P, Hkv, d]      (GQA family, token-major pages)
               [num_pages, Hkv, P, d]      (kv_layout=1, head-major pages)
  latent cache [num_pages, P, d_latent + d_rope]   (MLA, one record per token)
  block_tables [B, max_pages] int32, context_lens [B] int32.

Physical pages are a random permutation of the pool.  With ``poison=True``
every byte the method must not read holds NaN: unused pool pages, the slots
of a last partial page past the context, and table entries past
ceil(n_b / P) hold -1.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "e4m3": np.uint8}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}
# A NaN encoding of each storage type.
NAN_BITS = {"f32": np.float32(np.nan), "f16": np.float16(np.nan),
            "bf16": np.uint16(0x7FC0), "e4m3": np.uint8(0x7F)}
E4M3_MAX = 448.0


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 values to the storage type (library casts, RNE)."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.copy()
    if dtype == "f16":
        return x.astype(np.float16)
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    if dtype == "e4m3":
        t = t.clamp(-E4M3_MAX, E4M3_MAX)
        return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    raise ValueError(dtype)


def to_float32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Library decode of stored bytes to fp32 (for building test variants)."""
    if dtype in ("f32", "f16"):
        return np.asarray(a, dtype=np.float32)
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        return t.view(torch.bfloat16).float().numpy()
    if dtype == "e4m3":
        return t.view(torch.float8_e4m3fn).float().numpy()
    raise ValueError(dtype)


@dataclasses.dataclass
class PagedCase:
    """One synthetic decode step for the GQA family (or MLA when ``mla``)."""
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: Optional[np.ndarray]      # None for MLA (K and V share the latent cache)
    block_tables: np.ndarray
    context_lens: np.ndarray
    q_dtype: str
    kv_dtype: str
    page_size: int
    scale: float
    k_scale: float = 1.0
    v_scale: float = 1.0
    mla: bool = False
    d_latent: int = 0
    name: str = ""
    causal: bool = True                # several query tokens: bottom-right causal mask
    kv_layout: int = 0                 # 0: pages [P, Hkv, d]; 1: pages [Hkv, P, d]

    @property
    def batch(self) -> int:
        return self.q.shape[0]

    @property
    def q_len(self) -> int:
        """Query tokens per sequence: q is [B, Hq, d] (1) or [B, s_q, Hq, d]."""
        return self.q.shape[1] if self.q.ndim == 4 else 1

    @property
    def num_q_heads(self) -> int:
        return self.q.shape[-2]

    @property
    def num_kv_heads(self) -> int:
        return 1 if self.mla else self.k_cache.shape[1 if self.kv_layout else 2]

    @property
    def head_dim(self) -> int:
        return self.q.shape[-1]

    @property
    def head_dim_v(self) -> int:
        return self.d_latent if self.mla else self.v_cache.shape[3]

    @property
    def num_pages(self) -> int:
        return self.k_cache.shape[0]

    @property
    def max_pages(self) -> int:
        return self.block_tables.shape[1]


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _layout_pages(rng, context_lens, P, max_pages, extra_pages):
    """Random page assignment: returns (num_pages, block_tables, used_mask)."""
    lens = np.asarray(context_lens, dtype=np.int64)
    npg = [(int(n) + P - 1) // P for n in lens]
    need = max(npg) if len(npg) else 0
    if max_pages is None:
        max_pages = max(1, need)
    if need > max_pages:
        raise ValueError("context does not fit max_pages")
    num_pages = int(sum(npg)) + int(extra_pages)
    perm = rng.permutation(num_pages).astype(np.int32)
    tables = np.full((len(lens), max_pages), -1, dtype=np.int32)
    used = np.zeros(num_pages, dtype=bool)
    off = 0
    for b, k in enumerate(npg):
        tables[b, :k] = perm[off:off + k]
        used[perm[off:off + k]] = True
        off += k
    return num_pages, tables, used


def _poison(cache, tables, lens, used, P, nan_bits):
    """NaN into unused pages and into the slots past the context in last pages."""
    cache[~used] = nan_bits
    for b, n in enumerate(lens):
        n = int(n)
        if n % P and n > 0:
            last = tables[b, (n - 1) // P]
            cache[last, n % P:] = nan_bits


def make_gqa(*, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
             page_size: int, context_lens: Sequence[int], q_dtype: str, kv_dtype: str,
             seed: int, head_dim_v: Optional[int] = None, max_pages: Optional[int] = None,
             extra_pages: int = 0, poison: bool = True, std: float = 1.0,
             scale: Optional[float] = None, q_len: int = 1, causal: bool = True,
             kv_layout: int = 0, name: str = "") -> PagedCase:
    """GQA/MQA/MHA case: q, K, V ~ N(0, std^2) in fp32, then stored as requested.

    q_len > 1 gives q the shape [B, q_len, Hq, d] (several query tokens per
    sequence); q_len = 1 keeps [B, Hq, d].

    fp8 caches get one fp32 scale per tensor, amax / 448 over the values the
    method reads; the stored byte is e4m3(x / scale) (saturating, RNE).

    kv_layout=1 stores the same values with head-major pages [Hkv, P, d]
    (the random draws do not depend on the layout)."""
    dv = head_dim if head_dim_v is None else head_dim_v
    lens = np.asarray(context_lens, dtype=np.int32)
    assert lens.shape == (batch,)
    rng = _rng(seed)
    P = page_size
    num_pages, tables, used = _layout_pages(rng, lens, P, max_pages, extra_pages)
    qshape = (batch, num_q_heads, head_dim) if q_len == 1 else (batch, q_len, num_q_heads, head_dim)
    q32 = _normal(rng, qshape, std)
    k32 = _normal(rng, (num_pages, P, num_kv_heads, head_dim), std)
    v32 = _normal(rng, (num_pages, P, num_kv_heads, dv), std)
    k_scale = v_scale = 1.0
    if kv_dtype == "e4m3":
        # per-tensor scales from the values that are actually read
        k_amax = float(np.abs(k32[used]).max()) if used.any() else 1.0
        v_amax = float(np.abs(v32[used]).max()) if used.any() else 1.0
        k_scale = float(np.float32(k_amax / E4M3_MAX))
        v_scale = float(np.float32(v_amax / E4M3_MAX))
        k32 /= np.float32(k_scale)
        v32 /= np.float32(v_scale)
    k = encode(k32, kv_dtype)
    del k32
    v = encode(v32, kv_dtype)
    del v32
    if poison:
        _poison(k, tables, lens, used, P, NAN_BITS[kv_dtype])
        _poison(v, tables, lens, used, P, NAN_BITS[kv_dtype])
    else:
        tables[tables < 0] = 0
    if kv_layout:
        k = np.ascontiguousarray(k.transpose(0, 2, 1, 3))
        v = np.ascontiguousarray(v.transpose(0, 2, 1, 3))
    return PagedCase(q=encode(q32, q_dtype), k_cache=k, v_cache=v, block_tables=tables,
                     context_lens=lens, q_dtype=q_dtype, kv_dtype=kv_dtype, page_size=P,
                     scale=float(1.0 / math.sqrt(head_dim)) if scale is None else scale,
                     k_scale=k_scale, v_scale=v_scale, name=name, causal=causal,
                     kv_layout=int(kv_layout))


def make_mla(*, batch: int, num_q_heads: int, d_latent: int, d_rope: int, page_size: int,
             context_lens: Sequence[int], dtype: str, seed: int, scale: float,
             max_pages: Optional[int] = None, extra_pages: int = 0, poison: bool = True,
             std: float = 1.0, q_len: int = 1, causal: bool = True,
             kv_dtype: Optional[str] = None, name: str = "") -> PagedCase:
    """MLA case: one latent record [c (d_latent) | k_R (d_rope)] per token
    (q [B, q_len, Hq, rec] when q_len > 1).  kv_dtype "e4m3" stores the
    latent as fp8 with one fp32 scale (amax / 448 over the records read),
    kept in k_scale (and v_scale: V is part of the same record)."""
    kvd = dtype if kv_dtype is None else kv_dtype
    lens = np.asarray(context_lens, dtype=np.int32)
    assert lens.shape == (batch,)
    rng = _rng(seed)
    P = page_size
    rec = d_latent + d_rope
    num_pages, tables, used = _layout_pages(rng, lens, P, max_pages, extra_pages)
    qshape = (batch, num_q_heads, rec) if q_len == 1 else (batch, q_len, num_q_heads, rec)
    q = encode(_normal(rng, qshape, std), dtype)
    kv32 = _normal(rng, (num_pages, P, rec), std)
    kv_scale = 1.0
    if kvd == "e4m3":
        amax = float(np.abs(kv32[used]).max()) if used.any() else 1.0
        kv_scale = float(np.float32(amax / E4M3_MAX))
        kv32 /= np.float32(kv_scale)
    kv = encode(kv32, kvd)
    del kv32
    if poison:
        _poison(kv, tables, lens, used, P, NAN_BITS[kvd])
    else:
        tables[tables < 0] = 0
    return PagedCase(q=q, k_cache=kv, v_cache=None, block_tables=tables, context_lens=lens,
                     q_dtype=dtype, kv_dtype=kvd, page_size=P, scale=scale,
                     k_scale=kv_scale, v_scale=kv_scale, mla=True, d_latent=d_latent,
                     name=name, causal=causal)


def log_uniform_lens(rng: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    """floor(exp(U(ln lo, ln hi))) clipped to [lo, hi]."""
    x = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=n)))
    return np.clip(x, lo, hi).astype(np.int32)


# ------------------------------------------------------------------------------
# The five named workloads.  Seeds are 1000 + workload index (+ a sub-case).

def tiny_gqa(poison: bool = True) -> PagedCase:
    """B=2, Hq=8, Hkv=2 (G=4), d=64, lens [37, 100], P=16, 16-page pool, fp32."""
    return make_gqa(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=16,
                    context_lens=[37, 100], q_dtype="f32", kv_dtype="f32", seed=1000,
                    max_pages=8, extra_pages=16 - 10, poison=poison, name="tiny_gqa_fp32")


def _layout_tag(kv_layout: int) -> str:
    return "_headmajor" if kv_layout else ""


def gqa_batch64(seed_offset: int = 0, kv_layout: int = 0) -> PagedCase:
    """B=64, Hq=32, Hkv=8, d=128, ctx 1024, P=16, fp16, a permuted 4096-page pool
    (kv_layout 1: head-major pages)."""
    return make_gqa(batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                    context_lens=[1024] * 64, q_dtype="f16", kv_dtype="f16",
                    seed=1001 + seed_offset, poison=False, kv_layout=kv_layout,
                    name="gqa_b64_ctx1024_fp16" + _layout_tag(kv_layout))


def gqa_batch64_mtp(q_len: int = 2, kv_layout: int = 0) -> PagedCase:
    """The B=64 / ctx 1024 GQA step with q_len query tokens per sequence (the
    last q_len positions, bottom-right causal mask): multi-token decode."""
    return make_gqa(batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                    context_lens=[1024] * 64, q_dtype="f16", kv_dtype="f16", seed=1101,
                    poison=False, q_len=q_len, kv_layout=kv_layout,
                    name="gqa_b64_ctx1024_fp16_q%d" % q_len + _layout_tag(kv_layout))


def mqa_batch64_8k(kv_layout: int = 0) -> PagedCase:
    """MQA (one KV head for 32 query heads, G = 32): B=64, d=128, ctx 8192, P=16,
    fp16 -- the same 268,435,456 KV bytes per step as the B=64 GQA step."""
    return make_gqa(batch=64, num_q_heads=32, num_kv_heads=1, head_dim=128, page_size=16,
                    context_lens=[8192] * 64, q_dtype="f16", kv_dtype="f16", seed=1105,
                    poison=False, kv_layout=kv_layout,
                    name="mqa_b64_ctx8192_fp16" + _layout_tag(kv_layout))


def gqa_long(batch: int, kv_layout: int = 0) -> PagedCase:
    """B in {1, 4}, Hq=32, Hkv=8, d=128, ctx 32768, P=16, fp16 (split-KV)."""
    return make_gqa(batch=batch, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                    context_lens=[32768] * batch, q_dtype="f16", kv_dtype="f16",
                    seed=1002 * 10 + batch, poison=False, kv_layout=kv_layout,
                    name="gqa_b%d_ctx32768_fp16_split" % batch + _layout_tag(kv_layout))


def mla_b16(ctx: int = 65536, kv_dtype: str = "bf16", d_latent: int = 512) -> PagedCase:
    """B=16, 16 heads, latent 512 + rope 64, P=64, bf16 ~ N(0, 0.5^2), scale 1/sqrt(192)
    (kv_dtype "e4m3": the latent stored as fp8 with one scale, q in bf16;
    d_latent 256: the (320, 256) record)."""
    tag = ("bf16" if kv_dtype == "bf16" else "fp8_latent") + ("" if d_latent == 512 else
                                                             "_rec%d" % (d_latent + 64))
    return make_mla(batch=16, num_q_heads=16, d_latent=d_latent, d_rope=64, page_size=64,
                    context_lens=[ctx] * 16, dtype="bf16", seed=1003, std=0.5,
                    scale=1.0 / math.sqrt(192.0), poison=False, kv_dtype=kv_dtype,
                    name="mla_b16_ctx%d_%s" % (ctx, tag))


def mla_b16_mtp(q_len: int = 2, ctx: int = 65536) -> PagedCase:
    """The MLA B=16 step with q_len query tokens per sequence (causal)."""
    return make_mla(batch=16, num_q_heads=16, d_latent=512, d_rope=64, page_size=64,
                    context_lens=[ctx] * 16, dtype="bf16", seed=1103, std=0.5,
                    scale=1.0 / math.sqrt(192.0), poison=False, q_len=q_len,
                    name="mla_b16_ctx%d_bf16_q%d" % (ctx, q_len))


def ragged_fp8_lens(batch: int = 128, seed: int = 1004) -> np.ndarray:
    rng = _rng(seed * 10 + 1)
    lens = log_uniform_lens(rng, batch, 1, 16384)
    lens[0], lens[1], lens[2] = 1, 16384, 17
    return lens


def ragged_fp8(kv_layout: int = 0) -> PagedCase:
    """B=128, lens log-uniform in [1, 16384] (1, 16384, 17 forced), Hq=64, Hkv=8,
    d=128, P=16, fp8-e4m3 cache with per-tensor scales, fp16 queries."""
    return make_gqa(batch=128, num_q_heads=64, num_kv_heads=8, head_dim=128, page_size=16,
                    context_lens=ragged_fp8_lens(), q_dtype="f16", kv_dtype="e4m3",
                    seed=1004, max_pages=1024, poison=True, kv_layout=kv_layout,
                    name="ragged_b128_fp8" + _layout_tag(kv_layout))
