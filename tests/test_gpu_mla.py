"""GPU parity of the MLA latent path (both kernels, through the C ABI) against
the fp64 oracle on the same seeded inputs."""
import math

import numpy as np
import pytest
import torch

from decode_attention_paged_02_amd import pda
from decode_attention_paged_02_amd import workloads as W
from gpu_util import check, need_gpu, oracle_ref, say

pytestmark = pytest.mark.gpu
# keys on the MFMA M dimension, queries on M, vector dot products
VARIANTS = {"mfma": pda.PDA_MLA_MFMA, "qm": pda.PDA_MLA_MFMA_QM, "valu": pda.PDA_MLA_VALU}


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _mla(seed, lens, Hq=16, P=64, std=0.5, **kw):
    return W.make_mla(batch=len(lens), num_q_heads=Hq, d_latent=512, d_rope=64, page_size=P,
                      context_lens=lens, dtype="bf16", seed=seed, std=std,
                      scale=1.0 / math.sqrt(192.0), **kw)


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("lens", [[1], [31, 32, 33], [64, 65, 127, 1], [700, 1500]])
def test_lengths(variant, lens):
    case = _mla(len(lens) * 11 + lens[0], lens, extra_pages=3)
    say("mla", variant, lens)
    for s in (1, 3):
        out, lse = pda.run_case(case, variant=VARIANTS[variant], num_splits=s)
        ref_o, ref_l = oracle_ref(case)
        check(case, out, lse, ref_o, ref_l, label="mla %s %s S=%d" % (variant, lens, s))


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("Hq", [1, 8, 16, 32, 48])
def test_head_counts(variant, Hq):
    """Fewer than 16 heads (padded tile) and several 16-head tiles."""
    case = _mla(Hq, [200, 77], Hq=Hq, extra_pages=2)
    say("mla heads", variant, Hq)
    out, lse = pda.run_case(case, variant=VARIANTS[variant])
    ref_o, ref_l = oracle_ref(case)
    check(case, out, lse, ref_o, ref_l, label="mla %s Hq=%d" % (variant, Hq))


@pytest.mark.parametrize("P", [64, 128])
def test_page_sizes_and_poison(P):
    """NaN in unused pages and stale slots; huge values in table tails."""
    case = _mla(40 + P, [129, 1, 300, 64], P=P, extra_pages=5, max_pages=12)
    case.block_tables[case.block_tables < 0] = 2 ** 30
    say("mla poison", P)
    for name, v in VARIANTS.items():
        out, lse = pda.run_case(case, variant=v)
        assert torch.isfinite(out.float()).all()
        ref_o, ref_l = oracle_ref(case)
        check(case, out, lse, ref_o, ref_l, label="mla poison %s P=%d" % (name, P))


def test_mfma_and_valu_agree_and_are_deterministic():
    case = _mla(50, [3000, 4096, 10], extra_pages=1)
    say("mla agreement")
    dev = pda.to_device(case)
    ref_o, ref_l = oracle_ref(case)
    outs = []
    for name, v in VARIANTS.items():
        for s in (0, 1, 7):
            out, lse = pda.run_case(case, dev, variant=v, num_splits=s)
            check(case, out, lse, ref_o, ref_l, label="%s S=%d" % (name, s))
            out2, lse2 = pda.run_case(case, dev, variant=v, num_splits=s)
            assert torch.equal(out, out2) and torch.equal(lse, lse2)
            outs.append(out.float())
    for o in outs[1:]:
        assert (o - outs[0]).abs().max().item() < 2e-3


def test_constant_rope_columns_shift_lse_only():
    """Rope columns equal across tokens: output unchanged, LSE shifted by
    scale * q_R . k_R (softmax shift invariance), on the GPU path."""
    case = _mla(60, [500, 90], extra_pages=1, poison=False)
    say("mla rope shift")
    base = W.PagedCase(**{**case.__dict__, "k_cache": case.k_cache.copy()})
    base.k_cache[..., 512:] = 0
    out0, lse0 = pda.run_case(base)
    k_r = W.encode(np.random.default_rng(1).standard_normal(64).astype(np.float32) * 0.5, "bf16")
    shifted = W.PagedCase(**{**case.__dict__, "k_cache": base.k_cache.copy()})
    shifted.k_cache[..., 512:] = k_r
    out1, lse1 = pda.run_case(shifted)
    q_r = W.to_float32(case.q[..., 512:], "bf16").astype(np.float64)
    shift = case.scale * (q_r @ W.to_float32(k_r, "bf16").astype(np.float64))
    assert (out1.float() - out0.float()).abs().max().item() < 2e-3
    np.testing.assert_allclose(lse1.double().cpu().numpy(), lse0.double().cpu().numpy() + shift,
                               rtol=0, atol=1e-3)


def test_mla_b16_full_size():
    """B=16, 16 heads, ctx 65536, page 64, bf16 ~ N(0, 0.5^2): the timed MLA
    workload in its launch configuration, every (sequence, head) row (the fp64
    oracle takes about half a minute over them)."""
    case = W.mla_b16()
    say(case.name)
    dev = pda.to_device(case)
    ref_o, ref_l = oracle_ref(case)
    for name, v in VARIANTS.items():
        out, lse = pda.run_case(case, dev, variant=v)
        check(case, out, lse, ref_o, ref_l, label="%s %s" % (case.name, name))
    del dev
    torch.cuda.empty_cache()


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_ordered_work_mixed_lengths(variant):
    """MLA with a split threshold: the longest-first ordering pass, an empty
    sequence, and sequences on both sides of the threshold."""
    case = _mla(70, [0, 2000, 64, 5000, 129], extra_pages=2)
    say("mla ordered", variant)
    out, lse = pda.run_case(case, variant=VARIANTS[variant], num_splits=5, split_min_tokens=1000)
    ref_o, ref_l = oracle_ref(case)
    check(case, out, lse, ref_o, ref_l, label="mla ordered %s" % variant)


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("Hq", [16, 32])
def test_balanced_schedule_mixed_lengths(variant, Hq):
    """MLA under the balanced schedule (device-side chunking of the batch's
    pages), 16- and 32-row workgroups."""
    case = _mla(71 + Hq, [0, 2000, 64, 9000, 129, 1], Hq=Hq, extra_pages=2)
    say("mla balanced", variant, Hq)
    out, lse = pda.run_case(case, variant=VARIANTS[variant], schedule=pda.PDA_SCHEDULE_BALANCED)
    ref_o, ref_l = oracle_ref(case)
    check(case, out, lse, ref_o, ref_l, label="mla balanced %s Hq=%d" % (variant, Hq))


@pytest.mark.parametrize("variant,Hq,q_len", [
    # several query tokens take the matrix-core kernel only
    (v, Hq, ql) for v in VARIANTS for Hq, ql in [(16, 1), (32, 1), (16, 2), (8, 1)]
    if not (v == "valu" and ql > 1)])
def test_fp8_latent(variant, Hq, q_len):
    """An fp8 (E4M3) latent with one dequantization scale: staged into LDS as
    exact bf16, the scale folded into the score and the output."""
    case = _mla(80 + Hq + q_len, [1, 33, 700, 2000], Hq=Hq, extra_pages=2, kv_dtype="e4m3",
                q_len=q_len)
    say("mla fp8 latent", variant, Hq, q_len)
    ref_o, ref_l = oracle_ref(case)
    for s in (1, 4):
        out, lse = pda.run_case(case, variant=VARIANTS[variant], num_splits=s)
        check(case, out, lse, ref_o, ref_l, label="mla fp8 %s Hq=%d q=%d S=%d" % (variant, Hq,
                                                                                q_len, s))


def test_fp8_latent_b16_full_size():
    """The MLA decode shape with an fp8 latent: B=16, Hq=16, ctx 65536, every row."""
    case = W.mla_b16(kv_dtype="e4m3")
    say(case.name)
    ref_o, ref_l = oracle_ref(case)
    out, lse = pda.run_case(case)
    check(case, out, lse, ref_o, ref_l, label=case.name)


def test_record_320_b16_full_size():
    """The timed (320, 256) record workload: B=16, Hq=16, ctx 65536, every row."""
    case = W.mla_b16(d_latent=256)
    say(case.name)
    ref_o, ref_l = oracle_ref(case)
    out, lse = pda.run_case(case)
    assert tuple(out.shape) == (16, 16, 256)
    check(case, out, lse, ref_o, ref_l, label=case.name)


@pytest.mark.parametrize("variant", ["mfma", "qm"])
@pytest.mark.parametrize("Hq,q_len,kv", [(16, 1, "bf16"), (32, 1, "bf16"), (16, 2, "bf16"),
                                         (8, 1, "e4m3"), (16, 1, "e4m3")])
def test_record_320_value_256(Hq, q_len, kv, variant):
    """The (320, 256) record: a 256-wide latent + 64 rope values (FlashMLA-ETAP's
    second head-dimension pair), matrix-core kernel."""
    case = W.make_mla(batch=4, num_q_heads=Hq, d_latent=256, d_rope=64, page_size=64,
                      context_lens=[1, 65, 700, 3000], dtype="bf16", seed=90 + Hq + q_len,
                      std=0.5, scale=1.0 / math.sqrt(192.0), extra_pages=2, q_len=q_len,
                      kv_dtype=kv)
    say("mla 320/256", Hq, q_len, kv, variant)
    ref_o, ref_l = oracle_ref(case)
    v = VARIANTS[variant]
    for s in (1, 5):
        out, lse = pda.run_case(case, num_splits=s, variant=v)
        assert out.shape[-1] == 256
        check(case, out, lse, ref_o, ref_l, label="mla320 Hq=%d q=%d %s S=%d" % (Hq, q_len, kv, s))
    out, lse = pda.run_case(case, schedule=pda.PDA_SCHEDULE_BALANCED, variant=v)
    check(case, out, lse, ref_o, ref_l, label="mla320 balanced")


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_large_pool_64bit_offsets(variant):
    """Latent pages past 5 GiB of the pool (int64 page addressing)."""
    small = _mla(91, [300, 65], poison=False)
    dev = pda.to_device(small)
    page_bytes = dev.k_cache[0].numel() * dev.k_cache.element_size()
    base = (5 << 30) // page_bytes
    say("mla large pool", base + small.num_pages, "pages")
    kv = torch.zeros((base + small.num_pages,) + tuple(dev.k_cache.shape[1:]),
                     dtype=dev.k_cache.dtype, device="cuda")
    kv[base:] = dev.k_cache
    out, lse = pda.paged_decode_attn_mla(dev.q, kv, dev.block_tables + base, dev.context_lens,
                                         scale=small.scale, variant=VARIANTS[variant])
    ref_o, ref_l = oracle_ref(small)
    check(small, out, lse, ref_o, ref_l, label="mla large pool")
    del kv


def test_many_splits_combine_loop():
    """Split counts past the 64 per row that the combine keeps in registers,
    up to one page per split, on the 512-wide rows (four column chunks)."""
    case = _mla(92, [20000, 3, 700], poison=False)
    say("mla many splits")
    dev = pda.to_device(case)
    ref_o, ref_l = oracle_ref(case)
    for splits in (100, 313):
        p = pda.plan(pda.mla_shape(dev.q, dev.k_cache, dev.block_tables), mla=True,
                     num_splits=splits)
        assert p.max_splits > 64
        out, lse = pda.run_case(case, dev, num_splits=splits)
        check(case, out, lse, ref_o, ref_l, label="mla splits %d" % splits)


def test_queries_on_m_full_size():
    """The MLA decode shape (B=16, Hq=16, ctx 65536) with queries on the MFMA
    M dimension, every row, and bitwise run-to-run determinism."""
    case = W.mla_b16()
    say(case.name, "qm")
    dev = pda.to_device(case)
    ref_o, ref_l = oracle_ref(case)
    out, lse = pda.run_case(case, dev, variant=pda.PDA_MLA_MFMA_QM)
    check(case, out, lse, ref_o, ref_l, label="%s qm" % case.name)
    out2, lse2 = pda.run_case(case, dev, variant=pda.PDA_MLA_MFMA_QM)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    del dev
    torch.cuda.empty_cache()
