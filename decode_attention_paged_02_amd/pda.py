"""Thin ctypes binding over libpda.so (include/pda.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the stream.
The library must have been built (``python -m decode_attention_paged_02_amd.build``);
if it is missing, the first call raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpda.so")

PDA_F32, PDA_F16, PDA_BF16, PDA_FP8_E4M3 = 0, 1, 2, 3
PDA_MLA_DEFAULT, PDA_MLA_MFMA, PDA_MLA_VALU, PDA_MLA_MFMA_QM = 0, 1, 2, 3
PDA_GQA_DEFAULT, PDA_GQA_MFMA, PDA_GQA_VALU, PDA_GQA_MFMA_4WAVE, PDA_GQA_MFMA_1WAVE = 0, 1, 2, 3, 4
PDA_SCHEDULE_GRID, PDA_SCHEDULE_BALANCED = 0, 1
PDA_KV_TOKEN_MAJOR, PDA_KV_HEAD_MAJOR = 0, 1
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported configuration",
          3: "workspace missing or too small", 4: "HIP runtime error"}


class PdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s: %s (status %d)" % (where, STATUS.get(status, "?"), status))
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("head_dim_v", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
                ("split_min_tokens", ctypes.c_int32), ("variant", ctypes.c_int32),
                ("q_len", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("schedule", ctypes.c_int32), ("kv_layout", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("max_splits", ctypes.c_int32), ("pages_per_split", ctypes.c_int32),
                ("head_tiles", ctypes.c_int32), ("workgroups", ctypes.c_int32),
                ("num_cus", ctypes.c_int32), ("ordered", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_uint64), ("waves_per_unit", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


EXPORTS = ("pda_plan", "pda_workspace_bytes", "paged_decode_attn", "paged_decode_attn_mla",
           "paged_kv_append", "pda_check_inputs", "pda_stream_probe", "pda_status_string",
           "pda_version", "paged_decode_attn_noalloc")

_lib = None


def load() -> ctypes.CDLL:
    """Load libpda.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libpda.so is not built: run `python -m "
                           "decode_attention_paged_02_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    sp = ctypes.POINTER(Shape)
    lib.pda_plan.argtypes = [sp, i32, i32, i32, ctypes.POINTER(PlanInfo)]
    lib.pda_plan.restype = i32
    lib.pda_workspace_bytes.argtypes = [sp, i32, i32]
    lib.pda_workspace_bytes.restype = sz
    lib.paged_decode_attn.argtypes = [vp, vp, vp, vp, vp, i32, f32, i32, vp, vp, sp, vp, sz, vp]
    lib.paged_decode_attn.restype = i32
    lib.paged_decode_attn_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, f32, i32, vp, vp, sp, vp]
    lib.paged_decode_attn_noalloc.restype = i32
    lib.paged_decode_attn_mla.argtypes = [vp, vp, vp, vp, f32, i32, vp, vp, sp, vp, sz, vp]
    lib.paged_decode_attn_mla.restype = i32
    lib.paged_kv_append.argtypes = [vp, vp, vp, vp, vp, vp, sp, vp]
    lib.paged_kv_append.restype = i32
    lib.pda_check_inputs.argtypes = [sp, vp, vp, vp, vp, vp]
    lib.pda_check_inputs.restype = i32
    lib.pda_stream_probe.argtypes = [vp, vp, vp, vp, sp, i32, i32, vp, vp]
    lib.pda_stream_probe.restype = i32
    lib.pda_status_string.argtypes = [i32]
    lib.pda_status_string.restype = ctypes.c_char_p
    lib.pda_version.argtypes = []
    lib.pda_version.restype = i32
    _lib = lib
    return lib


def _dtype_code(t: torch.Tensor, fp8_ok: bool = False) -> int:
    if t.dtype == torch.float32:
        return PDA_F32
    if t.dtype == torch.float16:
        return PDA_F16
    if t.dtype == torch.bfloat16:
        return PDA_BF16
    if fp8_ok and t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PDA_FP8_E4M3
    raise TypeError("unsupported dtype %s" % t.dtype)


_TORCH_OF = {PDA_F32: torch.float32, PDA_F16: torch.float16, PDA_BF16: torch.bfloat16}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def make_shape(*, batch, num_q_heads, num_kv_heads, head_dim, head_dim_v, page_size,
               max_pages_per_seq, num_pages, q_dtype, kv_dtype, k_scale=1.0, v_scale=1.0,
               split_min_tokens=0, variant=0, q_len=1, causal=True, schedule=0,
               kv_layout=PDA_KV_TOKEN_MAJOR) -> Shape:
    return Shape(batch, num_q_heads, num_kv_heads, head_dim, head_dim_v, page_size,
                 max_pages_per_seq, num_pages, q_dtype, kv_dtype, k_scale, v_scale,
                 split_min_tokens, variant, q_len, int(causal), int(schedule), int(kv_layout))


def _query_dims(q):
    """(B, s_q, Hq, d) of q [B, Hq, d] (s_q = 1) or [B, s_q, Hq, d]."""
    _need(q.dim() in (3, 4), "q must be [B, Hq, d] or [B, s_q, Hq, d]")
    if q.dim() == 3:
        B, Hq, d = q.shape
        return B, 1, Hq, d
    return tuple(q.shape)


def _result_shapes(q, dv):
    """out and lse shapes for q: [B, Hq, dv] / [B, Hq], or [B, s_q, Hq, dv] /
    [B, Hq, s_q] for several query tokens."""
    B, s_q, Hq, _ = _query_dims(q)
    if q.dim() == 3:
        return (B, Hq, dv), (B, Hq)
    return (B, s_q, Hq, dv), (B, Hq, s_q)


def plan(shape: Shape, *, mla: bool = False, num_splits: int = 0, num_cus: int = 0) -> PlanInfo:
    """What the library will launch for these arguments (host only)."""
    info = PlanInfo()
    rc = load().pda_plan(ctypes.byref(shape), int(mla), int(num_splits), int(num_cus),
                         ctypes.byref(info))
    if rc:
        raise PdaError(rc, "pda_plan")
    return info


def gqa_shape(q, k_cache, v_cache, block_tables, *, k_scale=1.0, v_scale=1.0,
              split_min_tokens=0, variant=0, causal=True, schedule=0,
              kv_layout=PDA_KV_TOKEN_MAJOR) -> Shape:
    """Caches are [pages, P, Hkv, d] (token-major) or [pages, Hkv, P, d]
    (kv_layout = PDA_KV_HEAD_MAJOR)."""
    _need(k_cache.dim() == 4 and v_cache.dim() == 4, "bad ranks")
    B, s_q, Hq, d = _query_dims(q)
    if kv_layout == PDA_KV_HEAD_MAJOR:
        num_pages, Hkv, P, dk = k_cache.shape
    else:
        num_pages, P, Hkv, dk = k_cache.shape
    _need(dk == d and v_cache.shape[:3] == k_cache.shape[:3], "cache shapes do not match q")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == B, "block_tables must be [B, *]")
    return make_shape(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                      head_dim_v=v_cache.shape[3], page_size=P,
                      max_pages_per_seq=block_tables.shape[1], num_pages=num_pages,
                      q_dtype=_dtype_code(q), kv_dtype=_dtype_code(k_cache, fp8_ok=True),
                      k_scale=k_scale, v_scale=v_scale, split_min_tokens=split_min_tokens,
                      variant=variant, q_len=s_q, causal=causal, schedule=schedule,
                      kv_layout=kv_layout)


def mla_shape(q, kv_cache, block_tables, *, head_dim_v=512, variant=0,
              split_min_tokens=0, causal=True, schedule=0, kv_scale=1.0) -> Shape:
    _need(kv_cache.dim() == 3, "bad ranks")
    B, s_q, Hq, d = _query_dims(q)
    num_pages, P, dk = kv_cache.shape
    _need(dk == d, "latent width of q and cache differ")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == B, "block_tables must be [B, *]")
    return make_shape(batch=B, num_q_heads=Hq, num_kv_heads=1, head_dim=d,
                      head_dim_v=head_dim_v, page_size=P,
                      max_pages_per_seq=block_tables.shape[1], num_pages=num_pages,
                      q_dtype=_dtype_code(q), kv_dtype=_dtype_code(kv_cache, fp8_ok=True),
                      k_scale=kv_scale, v_scale=kv_scale, split_min_tokens=split_min_tokens,
                      variant=variant, q_len=s_q, causal=causal, schedule=schedule)


def _check_device(*ts):
    for t in ts:
        if t is not None:
            _need(t.is_cuda and t.is_contiguous(), "tensors must be contiguous device tensors")


def workspace_for(shape: Shape, *, mla: bool, num_splits: int, device,
                  stream=None) -> Optional[torch.Tensor]:
    """A workspace for calls with this plan (None when they need none).
    With `stream`, the memory is allocated for use on that stream."""
    nbytes = plan(shape, mla=mla, num_splits=num_splits).workspace_bytes
    if nbytes == 0:
        return None
    with _on_stream(stream):
        return torch.empty(nbytes, dtype=torch.uint8, device=device)


class _on_stream:
    """Make `stream` torch's current stream (no-op for None), so that tensors
    a call allocates for itself belong to the stream its kernels run on: the
    caching allocator then never hands their memory to other work before those
    kernels are done with it."""

    def __init__(self, stream):
        self._ctx = torch.cuda.stream(stream) if stream is not None else None

    def __enter__(self):
        if self._ctx is not None:
            self._ctx.__enter__()

    def __exit__(self, *exc):
        if self._ctx is not None:
            return self._ctx.__exit__(*exc)
        return False


def paged_decode_attn(q, k_cache, v_cache, block_tables, context_lens, *, scale: float,
                      num_splits: int = 0, out=None, lse=None, k_scale: float = 1.0,
                      v_scale: float = 1.0, split_min_tokens: int = 0, workspace=None,
                      stream=None, return_lse: bool = True, variant: int = 0,
                      causal: bool = True, schedule: int = PDA_SCHEDULE_GRID,
                      kv_layout: int = PDA_KV_TOKEN_MAJOR):
    """GQA/MQA/MHA paged decode attention.

    Caches are [pages, P, Hkv, d] (token-major), or [pages, Hkv, P, d] with
    kv_layout = PDA_KV_HEAD_MAJOR.

    q [B, Hq, d] returns (out [B, Hq, dv], lse [B, Hq] fp32); q [B, s_q, Hq, d]
    (s_q query tokens per sequence, the last s_q positions; causal: bottom-right
    mask) returns (out [B, s_q, Hq, dv], lse [B, Hq, s_q] fp32).

    variant: PDA_GQA_DEFAULT / PDA_GQA_MFMA (the planner picks one or four
    waves per work unit of the matrix-core kernel), PDA_GQA_MFMA_4WAVE,
    PDA_GQA_MFMA_1WAVE (grid schedule without a threshold) or PDA_GQA_VALU."""
    shape = gqa_shape(q, k_cache, v_cache, block_tables, k_scale=k_scale, v_scale=v_scale,
                      split_min_tokens=split_min_tokens, variant=variant, causal=causal,
                      schedule=schedule, kv_layout=kv_layout)
    _check_device(q, k_cache, v_cache, block_tables, context_lens, out, lse, workspace)
    _need(block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32,
          "block_tables and context_lens must be int32")
    Hq = shape.num_q_heads
    o_shape, l_shape = _result_shapes(q, shape.head_dim_v)
    with _on_stream(stream):
        if out is None:
            out = torch.empty(o_shape, dtype=q.dtype, device=q.device)
        if lse is None and return_lse:
            lse = torch.empty(l_shape, dtype=torch.float32, device=q.device)
    _need(tuple(out.shape) == o_shape and (lse is None or tuple(lse.shape) == l_shape),
          "out / lse shapes do not match q")
    if workspace is None:
        workspace = workspace_for(shape, mla=False, num_splits=num_splits, device=q.device,
                                  stream=stream)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    group = Hq // shape.num_kv_heads
    rc = load().paged_decode_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                  _ptr(context_lens), group, float(scale), int(num_splits),
                                  _ptr(out), _ptr(lse), ctypes.byref(shape), _ptr(workspace),
                                  wbytes, _stream_handle(stream))
    if rc:
        raise PdaError(rc, "paged_decode_attn")
    return out, lse


def paged_decode_attn_mla(q, kv_cache, block_tables, context_lens, *, scale: float,
                          num_splits: int = 0, out=None, lse=None, variant: int = 0,
                          head_dim_v: int = 512, split_min_tokens: int = 0, workspace=None,
                          stream=None, return_lse: bool = True, causal: bool = True,
                          schedule: int = PDA_SCHEDULE_GRID, kv_scale: float = 1.0):
    """MLA paged decode attention; returns (out [B, Hq, 512], lse [B, Hq] fp32),
    or (out [B, s_q, Hq, 512], lse [B, Hq, s_q]) for q [B, s_q, Hq, 576].  An
    fp8 latent (uint8 storage, E4M3) takes its dequantization scale kv_scale."""
    shape = mla_shape(q, kv_cache, block_tables, head_dim_v=head_dim_v, variant=variant,
                      split_min_tokens=split_min_tokens, causal=causal, schedule=schedule,
                      kv_scale=kv_scale)
    _check_device(q, kv_cache, block_tables, context_lens, out, lse, workspace)
    _need(block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32,
          "block_tables and context_lens must be int32")
    o_shape, l_shape = _result_shapes(q, head_dim_v)
    with _on_stream(stream):
        if out is None:
            out = torch.empty(o_shape, dtype=q.dtype, device=q.device)
        if lse is None and return_lse:
            lse = torch.empty(l_shape, dtype=torch.float32, device=q.device)
    _need(tuple(out.shape) == o_shape and (lse is None or tuple(lse.shape) == l_shape),
          "out / lse shapes do not match q")
    if workspace is None:
        workspace = workspace_for(shape, mla=True, num_splits=num_splits, device=q.device,
                                  stream=stream)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load().paged_decode_attn_mla(_ptr(q), _ptr(kv_cache), _ptr(block_tables),
                                      _ptr(context_lens), float(scale), int(num_splits),
                                      _ptr(out), _ptr(lse), ctypes.byref(shape),
                                      _ptr(workspace), wbytes, _stream_handle(stream))
    if rc:
        raise PdaError(rc, "paged_decode_attn_mla")
    return out, lse


def paged_kv_append(k_new, v_new, block_tables, positions, k_cache, v_cache=None, *,
                    k_scale: float = 1.0, v_scale: float = 1.0, stream=None,
                    kv_layout: int = PDA_KV_TOKEN_MAJOR):
    """Write new tokens' K (and V) rows into the paged cache, in place.

    k_new [B, s_new, Hkv, d] (or [B, s_new, 576] for an MLA latent cache
    [pages, P, 576], with v_new = v_cache = None); v_new [B, s_new, Hkv, dv];
    positions [B] int32, the position of each sequence's first new token
    (< 0: skipped).  fp8 caches (uint8 storage) store e4m3(x / scale).
    Head-major caches (kv_layout = PDA_KV_HEAD_MAJOR) are [pages, Hkv, P, d]."""
    _need((v_new is None) == (v_cache is None), "v_new and v_cache go together")
    kn = k_new if k_new.dim() == 4 else k_new.unsqueeze(2)
    kc = k_cache if k_cache.dim() == 4 else k_cache.unsqueeze(2)
    _need(kn.dim() == 4 and kc.dim() == 4, "bad ranks")
    B, s_new, Hkv, d = kn.shape
    if kv_layout == PDA_KV_HEAD_MAJOR and k_cache.dim() == 4:
        num_pages, Hkv2, P, d2 = kc.shape
    else:
        num_pages, P, Hkv2, d2 = kc.shape
    _need((Hkv2, d2) == (Hkv, d), "k_new rows do not match k_cache")
    dv = 0
    if v_cache is not None:
        _need(v_new.dim() == 4 and v_cache.dim() == 4 and v_new.shape[:3] == kn.shape[:3] and
              v_cache.shape[:3] == kc.shape[:3] and v_new.shape[3] == v_cache.shape[3],
              "v_new / v_cache shapes")
        dv = v_new.shape[3]
    _need(block_tables.dim() == 2 and block_tables.shape[0] == B, "block_tables must be [B, *]")
    _need(positions.dim() == 1 and positions.shape[0] == B, "positions must be [B]")
    _check_device(k_new, v_new, block_tables, positions, k_cache, v_cache)
    _need(block_tables.dtype == torch.int32 and positions.dtype == torch.int32,
          "block_tables and positions must be int32")
    shape = make_shape(batch=B, num_q_heads=Hkv, num_kv_heads=Hkv, head_dim=d,
                       head_dim_v=dv, page_size=P, max_pages_per_seq=block_tables.shape[1],
                       num_pages=num_pages, q_dtype=_dtype_code(k_new),
                       kv_dtype=_dtype_code(k_cache, fp8_ok=True), k_scale=k_scale,
                       v_scale=v_scale, q_len=s_new, kv_layout=kv_layout)
    rc = load().paged_kv_append(_ptr(k_new), _ptr(v_new), _ptr(block_tables), _ptr(positions),
                                _ptr(k_cache), _ptr(v_cache), ctypes.byref(shape),
                                _stream_handle(stream))
    if rc:
        raise PdaError(rc, "paged_kv_append")


class StreamProbe:
    """pda_stream_probe with marshalled arguments: reads the K/V bytes a
    GQA call with `shape` and `num_splits` reads, with its access pattern and
    no arithmetic (the practical bandwidth ceiling of that call).  caches:
    (k_cache, v_cache) pairs to rotate over, as in PreparedCall."""

    def __init__(self, shape: Shape, caches, block_tables, context_lens, *, num_splits=0,
                 steps_in_flight=1, stream=None):
        info = plan(shape, num_splits=num_splits)
        self._lib = load()
        self._sink = torch.empty(max(1, 4 * shape.batch * shape.num_kv_heads * info.max_splits),
                                 dtype=torch.int32, device=block_tables.device)
        self._keep = (shape, caches, block_tables, context_lens)
        st = _stream_handle(stream)
        self._args = [(_ptr(k), _ptr(v), _ptr(block_tables), _ptr(context_lens),
                       ctypes.byref(shape), int(num_splits), int(steps_in_flight),
                       _ptr(self._sink), st) for k, v in caches]

    def __call__(self, i: int = 0):
        rc = self._lib.pda_stream_probe(*self._args[i % len(self._args)])
        if rc:
            raise PdaError(rc, "pda_stream_probe")


def check_inputs(block_tables, context_lens, *, page_size: int, num_pages: int,
                 positions=None, s_new: int = 1, stream=None):
    """Count violations of the device-resident preconditions (pda_check_inputs):
    returns (bad lengths, bad table entries, bad append positions).  Synchronizes."""
    _need(block_tables.dim() == 2 and context_lens.dim() == 1 and
          context_lens.shape[0] == block_tables.shape[0], "block_tables [B, *], context_lens [B]")
    _check_device(block_tables, context_lens, positions)
    _need(block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32 and
          (positions is None or (positions.dtype == torch.int32 and
                                 positions.shape == context_lens.shape)),
          "int32 [B] lengths and positions")
    B, max_pages = block_tables.shape
    shape = make_shape(batch=B, num_q_heads=1, num_kv_heads=1, head_dim=8, head_dim_v=8,
                       page_size=page_size, max_pages_per_seq=max(1, max_pages),
                       num_pages=num_pages, q_dtype=PDA_F16, kv_dtype=PDA_F16, q_len=s_new)
    result = torch.zeros(3, dtype=torch.int32, device=block_tables.device)
    rc = load().pda_check_inputs(ctypes.byref(shape), _ptr(block_tables), _ptr(context_lens),
                                 _ptr(positions), _ptr(result), _stream_handle(stream))
    if rc:
        raise PdaError(rc, "pda_check_inputs")
    torch.cuda.synchronize(block_tables.device)
    return tuple(int(x) for x in result.cpu())


# ----------------------------------------------------------------------------
# Moving a workloads.PagedCase (numpy storage) onto the device.

@dataclass
class DeviceCase:
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: Optional[torch.Tensor]
    block_tables: torch.Tensor
    context_lens: torch.Tensor


def _storage_to_torch(a, dtype: str, device) -> torch.Tensor:
    import numpy as np
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a)
    if dtype == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16) if a.dtype == np.uint16 else t
    elif dtype == "e4m3":
        t = t.view(torch.uint8)
    return t.to(device)


def to_device(case, device="cuda") -> DeviceCase:
    """Copy the stored bytes of a PagedCase to device tensors (no conversion)."""
    return DeviceCase(
        q=_storage_to_torch(case.q, case.q_dtype, device),
        k_cache=_storage_to_torch(case.k_cache, case.kv_dtype, device),
        v_cache=None if case.v_cache is None else _storage_to_torch(case.v_cache,
                                                                    case.kv_dtype, device),
        block_tables=torch.from_numpy(case.block_tables).to(device),
        context_lens=torch.from_numpy(case.context_lens).to(device))


def run_case(case, dev: Optional[DeviceCase] = None, **kw):
    """Run the HIP path on a workloads.PagedCase; returns (out, lse) device tensors."""
    dev = dev or to_device(case)
    kw.setdefault("causal", case.causal)
    if case.mla:
        return paged_decode_attn_mla(dev.q, dev.k_cache, dev.block_tables, dev.context_lens,
                                     scale=case.scale, head_dim_v=case.d_latent,
                                     kv_scale=case.k_scale, **kw)
    kw.setdefault("kv_layout", case.kv_layout)
    return paged_decode_attn(dev.q, dev.k_cache, dev.v_cache, dev.block_tables,
                             dev.context_lens, scale=case.scale, k_scale=case.k_scale,
                             v_scale=case.v_scale, **kw)


class PreparedCall:
    """A call whose arguments are marshalled once; each __call__ only launches.

    caches: list of (k_cache, v_cache) pairs (v_cache None for MLA) that the
    calls rotate over (same shapes, different device copies)."""

    def __init__(self, *, mla, q, caches, block_tables, context_lens, scale, out, lse,
                 shape, num_splits, workspace, stream=None):
        self._lib = load()
        self._mla = mla
        st = _stream_handle(stream)
        wb = 0 if workspace is None else workspace.numel() * workspace.element_size()
        self._keep = (q, caches, block_tables, context_lens, out, lse, shape, workspace)
        self._args = []
        for k, v in caches:
            if mla:
                a = (_ptr(q), _ptr(k), _ptr(block_tables), _ptr(context_lens),
                     ctypes.c_float(scale), int(num_splits), _ptr(out), _ptr(lse),
                     ctypes.byref(shape), _ptr(workspace), wb, st)
            else:
                group = shape.num_q_heads // shape.num_kv_heads
                a = (_ptr(q), _ptr(k), _ptr(v), _ptr(block_tables), _ptr(context_lens), group,
                     ctypes.c_float(scale), int(num_splits), _ptr(out), _ptr(lse),
                     ctypes.byref(shape), _ptr(workspace), wb, st)
            self._args.append(a)
        self._fn = self._lib.paged_decode_attn_mla if mla else self._lib.paged_decode_attn

    def __call__(self, i: int = 0):
        rc = self._fn(*self._args[i % len(self._args)])
        if rc:
            raise PdaError(rc, "paged_decode_attn_mla" if self._mla else "paged_decode_attn")
