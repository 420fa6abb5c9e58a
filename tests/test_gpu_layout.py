"""GPU parity with head-major cache pages ([num_pages, Hkv, P, d]) against
the fp64 oracle: both GQA kernels, every cache type, splits, several query
tokens, the balanced schedule, the full-size workloads, and the KV append
(bit-exact) into a head-major cache."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_paged_02_amd import pda
from decode_attention_paged_02_amd import workloads as W
from gpu_util import check, need_gpu, oracle_ref, say

pytestmark = pytest.mark.gpu
HEAD_MAJOR = pda.PDA_KV_HEAD_MAJOR


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("q_dtype,kv_dtype,d,variant", [
    ("f16", "f16", 128, pda.PDA_GQA_MFMA), ("bf16", "bf16", 64, pda.PDA_GQA_MFMA),
    ("f16", "e4m3", 256, pda.PDA_GQA_MFMA), ("bf16", "e4m3", 128, pda.PDA_GQA_MFMA),
    ("f32", "f32", 128, pda.PDA_GQA_VALU), ("f16", "f16", 64, pda.PDA_GQA_VALU),
    ("bf16", "e4m3", 128, pda.PDA_GQA_VALU)])
@pytest.mark.parametrize("num_splits", [1, 3])
def test_head_major_parity(q_dtype, kv_dtype, d, variant, num_splits):
    case = W.make_gqa(batch=4, num_q_heads=16, num_kv_heads=4, head_dim=d, page_size=32,
                      context_lens=[1, 33, 700, 2049], q_dtype=q_dtype, kv_dtype=kv_dtype,
                      seed=61 + d, extra_pages=3, kv_layout=HEAD_MAJOR)
    say("head-major", q_dtype, kv_dtype, d, variant, num_splits)
    ref_o, ref_l = oracle_ref(case)
    out, lse = pda.run_case(case, num_splits=num_splits, variant=variant)
    check(case, out, lse, ref_o, ref_l, label="head-major %s %s d%d v%d S%d" % (
        q_dtype, kv_dtype, d, variant, num_splits))


@pytest.mark.parametrize("q_len,schedule", [(3, pda.PDA_SCHEDULE_GRID),
                                            (1, pda.PDA_SCHEDULE_BALANCED),
                                            (2, pda.PDA_SCHEDULE_BALANCED)])
def test_head_major_multi_token_and_balanced(q_len, schedule):
    case = W.make_gqa(batch=5, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                      context_lens=[5, 16, 3000, 129, 1000], q_dtype="f16", kv_dtype="f16",
                      seed=71 + q_len, extra_pages=2, q_len=q_len, kv_layout=HEAD_MAJOR)
    say("head-major q_len", q_len, "schedule", schedule)
    ref_o, ref_l = oracle_ref(case)
    out, lse = pda.run_case(case, num_splits=4, schedule=schedule)
    check(case, out, lse, ref_o, ref_l, label="head-major q%d sched %d" % (q_len, schedule))


# fp8 caches whose tile rows are contiguous (head-major pages, or one KV
# head) load two 16-token tiles per step: grid and ordered (threshold,
# balanced) calls, odd tile counts and a last step whose second tile lies past
# the range, several query tokens.
@pytest.mark.parametrize("layout,Hkv,q_len,splits,thr,schedule", [
    (HEAD_MAJOR, 4, 1, 3, 0, pda.PDA_SCHEDULE_GRID),
    (HEAD_MAJOR, 4, 1, 4, 256, pda.PDA_SCHEDULE_GRID),
    (HEAD_MAJOR, 4, 1, 4, 0, pda.PDA_SCHEDULE_BALANCED),
    (HEAD_MAJOR, 2, 3, 2, 0, pda.PDA_SCHEDULE_GRID),
    (0, 1, 1, 3, 0, pda.PDA_SCHEDULE_GRID),
    (0, 1, 1, 0, 0, pda.PDA_SCHEDULE_BALANCED)])
def test_fp8_two_tile_steps(layout, Hkv, q_len, splits, thr, schedule):
    case = W.make_gqa(batch=6, num_q_heads=8 * Hkv, num_kv_heads=Hkv, head_dim=128,
                      page_size=16, context_lens=[1, 17, 48, 529, 2000, 3001], q_dtype="f16",
                      kv_dtype="e4m3", seed=83 + Hkv + q_len + splits + schedule, extra_pages=3,
                      q_len=q_len, kv_layout=layout)
    say("fp8 two-tile steps", layout, Hkv, q_len, splits, thr, schedule)
    ref_o, ref_l = oracle_ref(case)
    out, lse = pda.run_case(case, num_splits=splits, split_min_tokens=thr, schedule=schedule)
    check(case, out, lse, ref_o, ref_l, label="fp8 steps L%d Hkv%d q%d S%d t%d s%d" % (
        layout, Hkv, q_len, splits, thr, schedule))


def test_head_major_full_size_batch64():
    case = W.gqa_batch64(kv_layout=HEAD_MAJOR)
    say(case.name)
    ref_o, ref_l = oracle_ref(case)
    out, lse = pda.run_case(case)
    check(case, out, lse, ref_o, ref_l, label=case.name)


@pytest.mark.parametrize("batch", [1, 4])
def test_head_major_full_size_long_split(batch):
    case = W.gqa_long(batch, kv_layout=HEAD_MAJOR)
    say(case.name)
    ref_o, ref_l = oracle_ref(case)
    out, lse = pda.run_case(case)
    check(case, out, lse, ref_o, ref_l, label=case.name)


def test_head_major_full_size_ragged_fp8_balanced():
    """The ragged fp8 batch with head-major pages under the balanced schedule
    (at most 8 splits), as the bench times it: fp8 tiles two per step, units
    planned in the attention kernel; every row checked."""
    case = W.ragged_fp8(kv_layout=HEAD_MAJOR)
    say(case.name, "balanced")
    dev = pda.to_device(case)
    ref_o, ref_l = oracle_ref(case)
    out, lse = pda.run_case(case, dev, num_splits=8, schedule=pda.PDA_SCHEDULE_BALANCED)
    check(case, out, lse, ref_o, ref_l, label="head-major balanced ragged")


def test_mqa_full_size_two_column_tiles():
    """MQA, B=64, 32 query heads on one KV head, ctx 8192, head-major: the
    workgroups carry two 16-row column tiles (one K/V load for 32 heads) and
    the sequences split eight ways."""
    case = W.mqa_batch64_8k(kv_layout=HEAD_MAJOR)
    say(case.name)
    dev = pda.to_device(case)
    shape = pda.gqa_shape(dev.q, dev.k_cache, dev.v_cache, dev.block_tables,
                          kv_layout=HEAD_MAJOR)
    assert pda.plan(shape).head_tiles == 1
    ref_o, ref_l = oracle_ref(case)
    out, lse = pda.run_case(case, dev)
    check(case, out, lse, ref_o, ref_l, label=case.name)


def test_head_major_equals_token_major_bitwise():
    """The two layouts of one case read the same elements in the same order:
    the kernels' outputs are bit-identical."""
    kw = dict(batch=6, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
              context_lens=[1, 17, 100, 640, 1024, 33], q_dtype="bf16", kv_dtype="bf16",
              seed=81, extra_pages=2)
    t = W.make_gqa(kv_layout=0, **kw)
    h = W.make_gqa(kv_layout=HEAD_MAJOR, **kw)
    say("layouts bitwise")
    for v in (pda.PDA_GQA_MFMA, pda.PDA_GQA_MFMA_1WAVE, pda.PDA_GQA_VALU):
        ot, lt = pda.run_case(t, num_splits=2, variant=v)
        oh, lh = pda.run_case(h, num_splits=2, variant=v)
        assert torch.equal(ot.view(torch.int16), oh.view(torch.int16))
        assert torch.equal(lt, lh)


@pytest.mark.parametrize("src,cache", [("f16", "f16"), ("bf16", "e4m3"), ("f32", "f32")])
def test_append_head_major_bit_exact(src, cache):
    case = W.make_gqa(batch=5, num_q_heads=4, num_kv_heads=4, head_dim=128, page_size=16,
                      context_lens=[7, 16, 17, 40, 100],
                      q_dtype=src if cache == "e4m3" else cache, kv_dtype=cache, seed=91,
                      extra_pages=2, kv_layout=HEAD_MAJOR)
    rng = np.random.default_rng(91)
    k_new = W.encode((rng.standard_normal((5, 2, 4, 128)) * 2).astype(np.float32), src)
    v_new = W.encode((rng.standard_normal((5, 2, 4, 128)) * 2).astype(np.float32), src)
    pos = (case.context_lens - 2).astype(np.int32)
    pos[1] = -1
    say("append head-major", src, cache)
    kc = pda._storage_to_torch(case.k_cache, cache, "cuda")
    vc = pda._storage_to_torch(case.v_cache, cache, "cuda")
    pda.paged_kv_append(pda._storage_to_torch(k_new, src, "cuda"),
                        pda._storage_to_torch(v_new, src, "cuda"),
                        torch.from_numpy(case.block_tables).cuda(), torch.from_numpy(pos).cuda(),
                        kc, vc, k_scale=case.k_scale, v_scale=case.v_scale, kv_layout=HEAD_MAJOR)
    torch.cuda.synchronize()
    for new, dev, host, sc in ((k_new, kc, case.k_cache, case.k_scale),
                               (v_new, vc, case.v_cache, case.v_scale)):
        want = oracle.kv_append(new, host, case.block_tables, pos, src_dtype=src,
                                cache_dtype=cache, scale=sc, kv_layout=HEAD_MAJOR)
        got = dev.cpu().view(torch.uint8).numpy() if dev.dtype != torch.uint8 else dev.cpu().numpy()
        assert np.array_equal(got.reshape(-1), want.view(np.uint8).reshape(-1))


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("kv_dtype,num_splits,thr,variant", [
    ("f16", 1, 0, 0), ("f16", 3, 0, 0), ("e4m3", 4, 100, 0), ("bf16", 0, 0, 0),
    ("f16", 1, 0, pda.PDA_GQA_MFMA_1WAVE), ("f16", 3, 0, pda.PDA_GQA_MFMA_1WAVE)])
def test_stream_probe_reads_exactly_the_call_bytes(layout, kv_dtype, num_splits, thr, variant):
    """The streaming probe reads the bytes the attention call reads: each
    workgroup's sink words (one per wave: four, or one with the one-wave
    layout) XOR to the 32-bit words of its K and V rows (its sequence, KV head
    and split range), computed on the host from the stored cache.  Rows past
    the context are NaN-poisoned, so a probe that read them would fold
    different words."""
    import numpy as np
    q_dt = "f16" if kv_dtype != "bf16" else "bf16"
    case = W.make_gqa(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                      context_lens=[37, 300, 1], q_dtype=q_dt, kv_dtype=kv_dtype, seed=61,
                      kv_layout=layout, extra_pages=2)
    say("stream probe", layout, kv_dtype, num_splits, thr)
    dev = pda.to_device(case)
    shape = pda.gqa_shape(dev.q, dev.k_cache, dev.v_cache, dev.block_tables,
                          split_min_tokens=thr, kv_layout=layout, k_scale=case.k_scale,
                          v_scale=case.v_scale, variant=variant)
    info = pda.plan(shape, num_splits=num_splits)
    nw = info.waves_per_unit
    assert nw in (1, 4) and (nw == 1) == (variant == pda.PDA_GQA_MFMA_1WAVE or num_splits == 0)
    probe = pda.StreamProbe(shape, [(dev.k_cache, dev.v_cache)], dev.block_tables,
                            dev.context_lens, num_splits=num_splits, steps_in_flight=2)
    probe()
    torch.cuda.synchronize()
    # one word per wave: the workgroup's XOR is the XOR of its waves' words
    words = probe._sink.cpu().numpy().view(np.uint32)[:info.max_splits * 3 * 2 * nw]
    got = np.bitwise_xor.reduce(words.reshape(info.max_splits, 3, 2, nw), axis=3)
    kc, vc = np.ascontiguousarray(case.k_cache), np.ascontiguousarray(case.v_cache)
    P = case.page_size
    for b in range(3):
        n = int(case.context_lens[b])
        pages = -(-n // P)
        split = n > thr and info.max_splits > 1
        pps = info.pages_per_split if split else max(pages, 1)
        for kvh in range(2):
            for sp in range(info.max_splits):
                t0, t1 = sp * pps * P, min((sp + 1) * pps * P, n)
                want = 0
                for t in range(t0, t1) if (split or sp == 0) else []:
                    pg = int(case.block_tables[b][t // P])
                    for c in (kc, vc):
                        row = c[pg, kvh, t % P] if layout else c[pg, t % P, kvh]
                        want ^= int(np.bitwise_xor.reduce(row.view(np.uint32)))
                assert int(got[sp, b, kvh]) == want, (b, kvh, sp)
