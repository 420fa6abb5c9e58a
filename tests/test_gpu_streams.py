"""Calls that overlap on two streams.  Every call is asynchronous on the
caller's stream, and calls may overlap when their workspaces and outputs
differ: each result of a run where two streams interleave GQA and MLA calls
(split paths, so the workspaces are in use) matches the same call made alone,
bit for bit."""
import math

import pytest
import torch

from decode_attention_paged_02_amd import pda
from decode_attention_paged_02_amd import workloads as W
from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def test_two_streams_with_their_own_workspaces():
    g = W.make_gqa(batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                   context_lens=[5000, 17, 3000, 900], q_dtype="f16", kv_dtype="f16", seed=41,
                   extra_pages=2)
    m = W.make_mla(batch=3, num_q_heads=16, d_latent=512, d_rope=64, page_size=64,
                   context_lens=[4000, 1, 2500], dtype="bf16", seed=42, std=0.5,
                   scale=1.0 / math.sqrt(192.0), extra_pages=2)
    say("two streams")
    dg, dm = pda.to_device(g), pda.to_device(m)
    S = 8

    def gqa(stream, ws, out, lse):
        return pda.paged_decode_attn(dg.q, dg.k_cache, dg.v_cache, dg.block_tables,
                                     dg.context_lens, scale=g.scale, num_splits=S, out=out,
                                     lse=lse, workspace=ws, stream=stream)

    def mla(stream, ws, out, lse):
        return pda.paged_decode_attn_mla(dm.q, dm.k_cache, dm.block_tables, dm.context_lens,
                                         scale=m.scale, num_splits=S, out=out, lse=lse,
                                         workspace=ws, stream=stream)

    ref_g = gqa(None, None, None, None)
    ref_m = mla(None, None, None, None)
    torch.cuda.synchronize()

    shape_g = pda.gqa_shape(dg.q, dg.k_cache, dg.v_cache, dg.block_tables)
    shape_m = pda.mla_shape(dm.q, dm.k_cache, dm.block_tables, head_dim_v=512)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    slots = []
    for _ in streams:
        slots.append(dict(
            wg=pda.workspace_for(shape_g, mla=False, num_splits=S, device="cuda"),
            wm=pda.workspace_for(shape_m, mla=True, num_splits=S, device="cuda"),
            og=torch.full_like(ref_g[0], float("nan")), lg=torch.zeros_like(ref_g[1]),
            om=torch.full_like(ref_m[0], float("nan")), lm=torch.zeros_like(ref_m[1])))
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for it in range(12):
        for k, (s, sl) in enumerate(zip(streams, slots)):
            with torch.cuda.stream(s):
                if (it + k) % 2 == 0:
                    gqa(s, sl["wg"], sl["og"], sl["lg"])
                else:
                    mla(s, sl["wm"], sl["om"], sl["lm"])
    torch.cuda.synchronize()
    for k, sl in enumerate(slots):
        assert torch.equal(sl["og"], ref_g[0]) and torch.equal(sl["lg"], ref_g[1]), "gqa %d" % k
        assert torch.equal(sl["om"], ref_m[0]) and torch.equal(sl["lm"], ref_m[1]), "mla %d" % k


def test_call_on_a_side_stream_without_workspace():
    """A call given a side stream and no workspace or outputs allocates them on
    that stream: while its kernels may still run, allocations made and written
    on the current stream never receive that memory, so every result matches
    the call made alone, bit for bit."""
    g = W.make_gqa(batch=2, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                   context_lens=[20000, 9000], q_dtype="f16", kv_dtype="f16", seed=43)
    m = W.make_mla(batch=2, num_q_heads=16, d_latent=512, d_rope=64, page_size=64,
                   context_lens=[6000, 300], dtype="bf16", seed=44, std=0.5,
                   scale=1.0 / math.sqrt(192.0))
    say("side stream without workspace")
    dg, dm = pda.to_device(g), pda.to_device(m)
    S = 16

    def gqa(stream):
        return pda.paged_decode_attn(dg.q, dg.k_cache, dg.v_cache, dg.block_tables,
                                     dg.context_lens, scale=g.scale, num_splits=S, stream=stream)

    def mla(stream):
        return pda.paged_decode_attn_mla(dm.q, dm.k_cache, dm.block_tables, dm.context_lens,
                                         scale=m.scale, num_splits=S, stream=stream)

    ref_g, ref_m = gqa(None), mla(None)
    torch.cuda.synchronize()
    wbytes = max(pda.plan(pda.gqa_shape(dg.q, dg.k_cache, dg.v_cache, dg.block_tables),
                          num_splits=S).workspace_bytes,
                 pda.plan(pda.mla_shape(dm.q, dm.k_cache, dm.block_tables), mla=True,
                          num_splits=S).workspace_bytes)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    results = []
    for it in range(6):
        results.append((gqa(side), mla(side)))
        # current-stream work that would overwrite a recycled block
        junk = torch.full((wbytes,), 255, dtype=torch.uint8, device="cuda")
        junk2 = torch.full((wbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
        del junk, junk2
    torch.cuda.synchronize()
    for k, ((og, lg), (om, lm)) in enumerate(results):
        assert torch.equal(og, ref_g[0]) and torch.equal(lg, ref_g[1]), "gqa call %d" % k
        assert torch.equal(om, ref_m[0]) and torch.equal(lm, ref_m[1]), "mla call %d" % k
