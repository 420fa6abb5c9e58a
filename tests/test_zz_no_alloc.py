"""The GQA entry point that allocates nothing (paged_decode_attn_noalloc):
its workspace is the library's per-GPU device array.  Called through the C
ABI, it gives the same bytes as paged_decode_attn with a caller workspace, on
consecutive calls that reuse the array with different shapes (a smaller input
second), for split, ordered and unsplit calls; and a call whose plan needs
more than the array holds is refused before any device work."""
import ctypes

import pytest
import torch

from decode_attention_paged_02_amd import pda
from decode_attention_paged_02_amd import workloads as W
from gpu_util import check, need_gpu, oracle_ref, say

pytestmark = pytest.mark.gpu
SCRATCH_BYTES = 64 << 20


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _noalloc(dev, case, shape, num_splits):
    o_shape, l_shape = pda._result_shapes(dev.q, case.head_dim_v)
    out = torch.full(o_shape, float("nan"), dtype=dev.q.dtype, device="cuda")
    lse = torch.zeros(l_shape, dtype=torch.float32, device="cuda")
    group = shape.num_q_heads // shape.num_kv_heads
    rc = pda.load().paged_decode_attn_noalloc(
        pda._ptr(dev.q), pda._ptr(dev.k_cache), pda._ptr(dev.v_cache), pda._ptr(dev.block_tables),
        pda._ptr(dev.context_lens), group, ctypes.c_float(case.scale), int(num_splits),
        pda._ptr(out), pda._ptr(lse), ctypes.byref(shape), pda._stream_handle(None))
    assert rc == 0, pda.STATUS.get(rc)
    return out, lse


def _case(seed, lens, B_heads=(32, 8), q_len=1, layout=1):
    Hq, Hkv = B_heads
    return W.make_gqa(batch=len(lens), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=128,
                      page_size=16, context_lens=lens, q_dtype="f16", kv_dtype="f16",
                      seed=seed, q_len=q_len, kv_layout=layout, extra_pages=2)


@pytest.mark.parametrize("kw", [dict(num_splits=16), dict(num_splits=8, split_min_tokens=1000),
                                dict(num_splits=0)],
                         ids=["grid", "ordered", "auto"])
def test_no_alloc_matches_the_workspace_entry_point(kw):
    thr = kw.get("split_min_tokens", 0)
    ns = kw["num_splits"]
    # two calls in a row on the same array: a larger input, then a smaller one
    for seed, lens in ((71, [9000, 17, 3000, 1, 4100]), (72, [2000, 33])):
        case = _case(seed, lens)
        say("no-alloc", kw, lens)
        dev = pda.to_device(case)
        shape = pda.gqa_shape(dev.q, dev.k_cache, dev.v_cache, dev.block_tables,
                              split_min_tokens=thr, kv_layout=case.kv_layout)
        assert pda.plan(shape, num_splits=ns).workspace_bytes <= SCRATCH_BYTES
        out, lse = _noalloc(dev, case, shape, ns)
        ref_o, ref_l = pda.run_case(case, dev, num_splits=ns, split_min_tokens=thr)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), "differs from the workspace call"
        o_ora, l_ora = oracle_ref(case)
        check(case, out, lse, o_ora, l_ora, label="no-alloc %s %s" % (kw, lens))


def test_no_alloc_multi_token_then_smaller():
    for seed, lens in ((73, [5000, 3, 700]), (74, [40])):
        case = _case(seed, lens, B_heads=(16, 4), q_len=3)
        say("no-alloc multi-token", lens)
        dev = pda.to_device(case)
        shape = pda.gqa_shape(dev.q, dev.k_cache, dev.v_cache, dev.block_tables,
                              kv_layout=case.kv_layout)
        out, lse = _noalloc(dev, case, shape, 8)
        ref_o, ref_l = pda.run_case(case, dev, num_splits=8)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)


def test_no_alloc_refuses_plans_beyond_the_array():
    """A plan needing more than 64 MiB is refused with PDA_ERR_WORKSPACE before
    any device work (the pointers are never followed)."""
    s = pda.make_shape(batch=512, num_q_heads=64, num_kv_heads=8, head_dim=128, head_dim_v=128,
                       page_size=16, max_pages_per_seq=1024, num_pages=1 << 20,
                       q_dtype=pda.PDA_F16, kv_dtype=pda.PDA_F16)
    assert pda.plan(s, num_splits=8).workspace_bytes > SCRATCH_BYTES
    fake = ctypes.c_void_p(0x1000)
    rc = pda.load().paged_decode_attn_noalloc(fake, fake, fake, fake, fake, 8,
                                              ctypes.c_float(0.1), 8, fake, None,
                                              ctypes.byref(s), None)
    assert rc == 3
