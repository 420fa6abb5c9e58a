"""Helpers shared by the GPU parity tests (not collected as tests)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from decode_attention_paged_02_amd import pda

# Tolerances of the GPU result against the fp64 oracle (max-abs / RMSE on the
# output; absolute on the natural-log LSE).  fp16/bf16 and fp8 bars are the
# ones the workload definition states; fp32 gets a tighter internal bar.
TOL = {
    "f32": dict(max_abs=1e-5, rmse=1e-6, lse=1e-5),
    "f16": dict(max_abs=2e-3, rmse=1e-4, lse=1e-3),
    "bf16": dict(max_abs=2e-3, rmse=1e-4, lse=1e-3),
    "e4m3": dict(max_abs=5e-3, rmse=1e-4, lse=1e-3),
}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    """Name the case before a GPU step (flushed, visible with -s)."""
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def oracle_ref(case, rows=None, **kw):
    if case.mla:
        return oracle.mla_attention(case.q, case.k_cache, case.block_tables, case.context_lens,
                                    scale=case.scale, d_latent=case.d_latent,
                                    q_dtype=case.q_dtype, kv_dtype=case.kv_dtype,
                                    kv_scale=case.k_scale, causal=case.causal, rows=rows, **kw)
    return oracle.paged_attention(case.q, case.k_cache, case.v_cache, case.block_tables,
                                  case.context_lens, scale=case.scale, q_dtype=case.q_dtype,
                                  kv_dtype=case.kv_dtype, k_scale=case.k_scale,
                                  v_scale=case.v_scale, causal=case.causal, rows=rows,
                                  kv_layout=case.kv_layout, **kw)


def round_to(ref, dtype):
    """The oracle's fp64 result rounded (RNE, library cast) to the output
    storage type: the nearest answer the output format can hold."""
    t = torch.from_numpy(np.ascontiguousarray(ref))
    return t.to(dtype).double().numpy()


_BITS = {torch.float16: torch.int16, torch.bfloat16: torch.int16, torch.float32: torch.int32}


def errors(out_gpu, out_ref, rows=None):
    """Max-abs and RMSE of the GPU output against the oracle rounded to the
    output type.  One exception: where the GPU value is the other neighbour
    of the exact value (the two adjacent representable values that bracket
    it), the element's error is the exact value's distance from their
    midpoint -- the least error the unrounded GPU result can have had to
    round the other way.  (Without it a fp32 error of 1e-7 next to a tie
    would count as a whole bf16 step, 4e-3 at magnitudes 0.5..1.)"""
    o_t = out_gpu.detach().cpu()
    r_t = torch.from_numpy(np.ascontiguousarray(out_ref)).to(o_t.dtype)
    o, r = o_t.double().numpy(), r_t.double().numpy()
    ref = np.asarray(out_ref, dtype=np.float64)
    ib = _BITS[o_t.dtype]
    ob, rb = o_t.view(ib).numpy().astype(np.int64), r_t.view(ib).numpy().astype(np.int64)
    adjacent = (np.abs(ob - rb) == 1) & ((ob < 0) == (rb < 0))
    brackets = (o - ref) * (r - ref) <= 0
    d = np.abs(o - r)
    flip = adjacent & brackets
    d[flip] = np.abs(ref[flip] - 0.5 * (o[flip] + r[flip]))
    if rows is not None:
        d = d[rows]
    return float(d.max()), float(np.sqrt(np.mean(d * d)))


def check(case, out, lse, ref_out, ref_lse, rows=None, tol=None, label=""):
    """Assert the GPU result is within the tolerance of the oracle.

    Output errors are taken against the oracle rounded to the output dtype
    (fp16/bf16 quantization of O(1) values alone exceeds an RMSE of 1e-4 at
    very short contexts); the LSE is fp32 and compared unrounded.  rows: a
    boolean mask over the rows of out (and of lse), or a pair of masks (out
    rows, lse rows) when the two layouts differ (several query tokens)."""
    t = dict(TOL[case.kv_dtype if case.kv_dtype == "e4m3" else case.q_dtype])
    if tol:
        t.update(tol)
    rows, lse_rows = rows if isinstance(rows, tuple) else (rows, rows)
    mx, rmse = errors(out, ref_out, rows)
    assert np.isfinite(mx), "non-finite output " + label
    assert mx <= t["max_abs"], "%s max-abs %.3g > %.3g" % (label, mx, t["max_abs"])
    assert rmse <= t["rmse"], "%s rmse %.3g > %.3g" % (label, rmse, t["rmse"])
    if lse is not None:
        l = lse.detach().double().cpu().numpy()
        r = ref_lse
        if lse_rows is not None:
            l, r = l[lse_rows], r[lse_rows]
        fin = np.isfinite(r)
        assert np.array_equal(fin, np.isfinite(l)), label + " lse finiteness differs"
        if fin.any():
            dl = float(np.abs(l[fin] - r[fin]).max())
            assert dl <= t["lse"], "%s lse err %.3g > %.3g" % (label, dl, t["lse"])
        assert np.array_equal(l[~fin], r[~fin]), label + " empty rows must give -inf"
    return mx, rmse
