"""GPU parity of multi-token decode (several query tokens per sequence, the
last s_q positions, with or without the bottom-right causal mask) against
the fp64 oracle, through the C ABI.  The matrix-core kernels take the
(query token, head) rows of a KV group as their MFMA columns; every column
has its own token limit under the mask."""
import numpy as np
import pytest
import torch

from decode_attention_paged_02_amd import pda
from decode_attention_paged_02_amd import workloads as W
from gpu_util import check, need_gpu, oracle_ref, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _gqa(seed, B, Hq, Hkv, lens, q_len, q_dtype="f16", kv_dtype="f16", d=128, P=16,
         causal=True, **kw):
    return W.make_gqa(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, page_size=P,
                      context_lens=lens, q_dtype=q_dtype, kv_dtype=kv_dtype, seed=seed,
                      q_len=q_len, causal=causal, extra_pages=2, **kw)


@pytest.mark.parametrize("q_len", [2, 3, 4])
@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (8, 8), (64, 8), (16, 1)])
@pytest.mark.parametrize("causal", [True, False])
def test_gqa_rows_and_masks(q_len, Hq, Hkv, causal):
    """Groups of 1 to 16 heads (q_len * group rows: one to four tiles), lengths
    around the page and tile edges and below q_len (empty early queries)."""
    lens = [1, 2, 3, 17, 100, 64]
    case = _gqa(q_len * 1000 + Hq + Hkv, len(lens), Hq, Hkv, lens, q_len, causal=causal)
    say("multi-token gqa", q_len, Hq, Hkv, causal)
    ref_o, ref_l = oracle_ref(case)
    for s in (1, 3):
        out, lse = pda.run_case(case, num_splits=s)
        assert tuple(out.shape) == (len(lens), q_len, Hq, 128)
        assert tuple(lse.shape) == (len(lens), Hq, q_len)
        check(case, out, lse, ref_o, ref_l, label="q_len=%d Hq=%d Hkv=%d S=%d" % (q_len, Hq,
                                                                                 Hkv, s))


@pytest.mark.parametrize("dt", [("bf16", "bf16"), ("f16", "e4m3"), ("bf16", "e4m3")])
@pytest.mark.parametrize("d,P", [(64, 16), (128, 32), (256, 16)])
def test_gqa_dtypes_and_head_dims(dt, d, P):
    case = _gqa(d + P + len(dt[1]), 3, 16, 4, [40, 333, 5], 3, *dt, d=d, P=P)
    say("multi-token dtypes", dt, d, P)
    ref_o, ref_l = oracle_ref(case)
    for s in (1, 4):
        out, lse = pda.run_case(case, num_splits=s)
        check(case, out, lse, ref_o, ref_l, label="%s d=%d P=%d S=%d" % (dt, d, P, s))


def test_gqa_split_empty_for_early_queries():
    """n = 33, P = 16, two pages per split: the second split holds token 32
    only, which queries 0..2 of 4 do not see (their partial is empty and the
    combine must give it weight 0)."""
    case = _gqa(77, 2, 32, 8, [33, 50], 4)
    dev = pda.to_device(case)
    p = pda.plan(pda.gqa_shape(dev.q, dev.k_cache, dev.v_cache, dev.block_tables,
                               causal=True), num_splits=2, num_cus=256)
    assert (p.max_splits, p.pages_per_split) == (2, 2)
    say("multi-token empty partials")
    ref_o, ref_l = oracle_ref(case)
    out, lse = pda.run_case(case, dev, num_splits=2)
    check(case, out, lse, ref_o, ref_l, label="empty partials")


def test_gqa_ordered_ragged_with_draft_tokens():
    """A mixed-length batch with a split threshold (ordered work units)."""
    rng = np.random.default_rng(3)
    lens = W.log_uniform_lens(rng, 24, 1, 6000)
    lens[:3] = [1, 6000, 2]
    case = _gqa(91, 24, 64, 8, lens, 2, "f16", "e4m3")
    say("multi-token ragged fp8 ordered")
    dev = pda.to_device(case)
    ref_o, ref_l = oracle_ref(case)
    out, lse = pda.run_case(case, dev, num_splits=8, split_min_tokens=2048)
    check(case, out, lse, ref_o, ref_l, label="ordered")


def test_gqa_batch64_two_tokens_full_size():
    """B=64, Hq=32, Hkv=8, d=128, ctx 1024, P=16, fp16 with two query tokens."""
    case = W.make_gqa(batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                      context_lens=[1024] * 64, q_dtype="f16", kv_dtype="f16", seed=1001,
                      q_len=2)
    say("multi-token batch64")
    ref_o, ref_l = oracle_ref(case)
    out, lse = pda.run_case(case)
    check(case, out, lse, ref_o, ref_l, label="b64 q_len=2")


def test_single_token_slices_agree_with_single_token_calls():
    """Causal query i equals a single-token call on the first n - (q_len - 1 - i)
    tokens -- on the GPU, within the tolerance (different tilings)."""
    q_len = 3
    case = _gqa(5, 3, 32, 8, [20, 515, 1000], q_len)
    dev = pda.to_device(case)
    out, lse = pda.run_case(case, dev)
    for i in range(q_len):
        lens_i = (dev.context_lens - (q_len - 1 - i)).contiguous()
        o1, l1 = pda.paged_decode_attn(dev.q[:, i].contiguous(), dev.k_cache, dev.v_cache,
                                       dev.block_tables, lens_i, scale=case.scale)
        assert (out[:, i].float() - o1.float()).abs().max().item() < 2e-3
        assert (lse[:, :, i] - l1).abs().max().item() < 1e-3


# ------------------------------------------------------------------- MLA

def _mla(seed, lens, Hq, q_len, causal=True, P=64):
    return W.make_mla(batch=len(lens), num_q_heads=Hq, d_latent=512, d_rope=64, page_size=P,
                      context_lens=lens, dtype="bf16", seed=seed, scale=192 ** -0.5,
                      std=0.5, extra_pages=2, q_len=q_len, causal=causal)


@pytest.mark.parametrize("Hq,q_len", [(16, 2), (8, 3), (32, 2), (1, 4)])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("variant", [pda.PDA_MLA_MFMA, pda.PDA_MLA_MFMA_QM])
def test_mla_rows_and_masks(Hq, q_len, causal, variant):
    lens = [1, 2, 65, 700, 128]
    case = _mla(Hq * 10 + q_len, lens, Hq, q_len, causal)
    say("multi-token mla", Hq, q_len, causal, variant)
    ref_o, ref_l = oracle_ref(case)
    for s in (1, 4):
        out, lse = pda.run_case(case, num_splits=s, variant=variant)
        assert tuple(out.shape) == (len(lens), q_len, Hq, 512)
        check(case, out, lse, ref_o, ref_l, label="mla Hq=%d q_len=%d S=%d" % (Hq, q_len, s))


def test_mla_b16_two_tokens_sampled():
    """The MLA decode shape with two query tokens (speculative decoding):
    B=16, Hq=16, ctx 8192 (a shorter context than the timed one keeps the
    oracle quick), sampled rows."""
    case = _mla(1003, [8192] * 16, 16, 2)
    rng = np.random.default_rng(2)
    rows = rng.random((16, 2, 16)) < 0.2
    rows[0] = True
    say("multi-token mla b16")
    ref_o, ref_l = oracle_ref(case, rows=rows)
    out, lse = pda.run_case(case)
    check(case, out, lse, ref_o, ref_l, rows=(rows, rows.transpose(0, 2, 1)),
          label="mla b16 q_len=2")


def test_mla_b16_two_tokens_full_size():
    """The timed two-token MLA workload: B=16, Hq=16, ctx 65536, two causal
    query tokens per sequence, every (sequence, token, head) row."""
    case = W.mla_b16_mtp(2)
    say(case.name)
    ref_o, ref_l = oracle_ref(case)
    out, lse = pda.run_case(case)
    assert tuple(out.shape) == (16, 2, 16, 512)
    check(case, out, lse, ref_o, ref_l, label=case.name)
