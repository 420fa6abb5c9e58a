"""GPU parity of the GQA-family path (HIP kernels through the C ABI) against
the fp64 oracle, element by element on the same seeded inputs."""
import numpy as np
import pytest
import torch

from decode_attention_paged_02_amd import pda
from decode_attention_paged_02_amd import workloads as W
from gpu_util import check, need_gpu, oracle_ref, say

pytestmark = pytest.mark.gpu
# both GQA kernels; the matrix-core one takes f16 / bf16 queries only.  "mfma"
# lets the planner choose its wave layout (one wave per unit on the GRID
# schedule with 16-bit caches and d >= 128, else four), "mfma4" keeps four
# waves per unit everywhere.
VARIANTS = {"mfma": pda.PDA_GQA_MFMA, "mfma4": pda.PDA_GQA_MFMA_4WAVE, "valu": pda.PDA_GQA_VALU}


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _supported(variant, q_dtype):
    # the matrix-core kernel takes f16 / bf16 queries only
    return not (variant.startswith("mfma") and q_dtype == "f32")


def _gqa(seed, B, Hq, Hkv, d, P, lens, q_dtype="f16", kv_dtype="f16", **kw):
    return W.make_gqa(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, page_size=P,
                      context_lens=lens, q_dtype=q_dtype, kv_dtype=kv_dtype, seed=seed, **kw)


@pytest.mark.parametrize("num_splits", [1, 2, 3, 7, 0])
def test_tiny_gqa_fp32(num_splits):
    case = W.tiny_gqa()
    say("tiny_gqa fp32", "splits", num_splits)
    out, lse = pda.run_case(case, num_splits=num_splits)
    ref_o, ref_l = oracle_ref(case)
    check(case, out, lse, ref_o, ref_l, label="tiny S=%d" % num_splits)


def test_gqa_batch64_full_size():
    """B=64, Hq=32, Hkv=8, d=128, ctx 1024, P=16, fp16; no split (the timed workload)."""
    case = W.gqa_batch64()
    say(case.name)
    dev = pda.to_device(case)
    p = pda.plan(pda.gqa_shape(dev.q, dev.k_cache, dev.v_cache, dev.block_tables))
    assert p.max_splits == 1
    ref_o, ref_l = oracle_ref(case)
    for name, v in VARIANTS.items():
        out, lse = pda.run_case(case, dev, variant=v)
        check(case, out, lse, ref_o, ref_l, label="%s %s" % (case.name, name))


@pytest.mark.parametrize("batch", [1, 4])
def test_gqa_long_context_split(batch):
    """ctx 32768, splits chosen to fill the CUs, merged by the combine pass."""
    case = W.gqa_long(batch)
    say(case.name)
    dev = pda.to_device(case)
    p = pda.plan(pda.gqa_shape(dev.q, dev.k_cache, dev.v_cache, dev.block_tables))
    assert p.max_splits > 1
    ref_o, ref_l = oracle_ref(case)
    for name, v in VARIANTS.items():
        out, lse = pda.run_case(case, dev, variant=v)
        check(case, out, lse, ref_o, ref_l, label="%s %s" % (case.name, name))


def test_ragged_fp8_full_size():
    """B=128, log-uniform lengths in [1, 16384], Hq=64, Hkv=8, fp8-e4m3 cache with
    per-tensor scales, fp16 q; sequences longer than 4096 tokens split (up to 8
    ways); every (sequence, head) row."""
    case = W.ragged_fp8()
    say(case.name)
    dev = pda.to_device(case)
    ref_o, ref_l = oracle_ref(case)
    for name, v in VARIANTS.items():
        out, lse = pda.run_case(case, dev, num_splits=8, split_min_tokens=4096, variant=v)
        check(case, out, lse, ref_o, ref_l, label="%s %s" % (case.name, name))


@pytest.mark.parametrize("lens", [[1], [15, 16, 17], [31, 32, 33, 47], [100, 1, 64, 129]])
@pytest.mark.parametrize("dt,variant", [
    (dt, v) for dt in [("f16", "f16"), ("bf16", "bf16"), ("f32", "f32"), ("f16", "e4m3"),
                       ("bf16", "e4m3")]
    for v in VARIANTS if _supported(v, dt[0])])
def test_page_boundaries_and_dtypes(lens, dt, variant):
    case = _gqa(len(lens) * 7 + len(dt[1]), len(lens), 8, 2, 128, 16, lens, *dt, extra_pages=3)
    say("boundaries", lens, dt, variant)
    out, lse = pda.run_case(case, variant=VARIANTS[variant])
    ref_o, ref_l = oracle_ref(case)
    check(case, out, lse, ref_o, ref_l, label="lens=%s %s" % (lens, dt))


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 1), (16, 1), (12, 4), (24, 4), (48, 4),
                                    (64, 8), (32, 2)])
@pytest.mark.parametrize("variant", list(VARIANTS))
def test_group_sizes(Hq, Hkv, variant):
    """G=1 (MHA), MQA (Hkv=1), non-power-of-two groups (padded head tiles), G=16."""
    case = _gqa(Hq * 100 + Hkv, 3, Hq, Hkv, 128, 16, [5, 200, 77], extra_pages=2)
    say("groups", Hq, Hkv, variant)
    out, lse = pda.run_case(case, variant=VARIANTS[variant])
    ref_o, ref_l = oracle_ref(case)
    check(case, out, lse, ref_o, ref_l, label="Hq=%d Hkv=%d" % (Hq, Hkv))


@pytest.mark.parametrize("Hq,Hkv,B", [(32, 1, 3), (64, 1, 9), (40, 1, 9), (64, 2, 11)])
@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("thr", [0, 100])
def test_large_groups_several_head_tiles(Hq, Hkv, B, variant, thr, ):
    """Groups beyond one head tile (G = 20 to 64): the tiles of one (sequence,
    KV head) run as separate workgroups placed 8 apart in the grid; eight or
    more groups take the interleaved placement, the rest the adjacent one.
    thr > 0 orders the work (unit list)."""
    lens = list(np.random.default_rng(Hq + B).integers(1, 600, B))
    case = _gqa(Hq * 10 + B, B, Hq, Hkv, 128, 16, lens, extra_pages=2)
    say("large groups", Hq, Hkv, B, variant, thr)
    out, lse = pda.run_case(case, num_splits=3, split_min_tokens=thr, variant=VARIANTS[variant])
    ref_o, ref_l = oracle_ref(case)
    check(case, out, lse, ref_o, ref_l, label="Hq=%d Hkv=%d B=%d thr=%d" % (Hq, Hkv, B, thr))


@pytest.mark.parametrize("d,P,dt,variant", [
    (d, P, dt, v) for d, P, dt in [(64, 16, "f16"), (64, 32, "bf16"), (256, 16, "f16"),
                                   (128, 64, "f16"), (64, 16, "f32"), (128, 32, "f32"),
                                   (256, 16, "bf16")]
    for v in VARIANTS if _supported(v, dt)])
def test_head_dims_and_page_sizes(d, P, dt, variant):
    case = _gqa(d + P, 2, 16, 4, d, P, [333, 70], dt, dt, extra_pages=2)
    say("d/P", d, P, dt, variant)
    for s in (1, 3):
        out, lse = pda.run_case(case, num_splits=s, variant=VARIANTS[variant])
        ref_o, ref_l = oracle_ref(case)
        check(case, out, lse, ref_o, ref_l, label="d=%d P=%d %s S=%d" % (d, P, dt, s))


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_split_counts_agree_and_runs_are_deterministic(variant):
    case = _gqa(9, 2, 32, 8, 128, 16, [4000, 2500])
    say("split invariance", variant)
    dev = pda.to_device(case)
    ref_o, ref_l = oracle_ref(case)
    outs = {}
    for s in (1, 2, 5, 16, 250):
        out, lse = pda.run_case(case, dev, num_splits=s, variant=VARIANTS[variant])
        check(case, out, lse, ref_o, ref_l, label="S=%d" % s)
        out2, lse2 = pda.run_case(case, dev, num_splits=s, variant=VARIANTS[variant])
        assert torch.equal(out, out2) and torch.equal(lse, lse2), "run-to-run differs"
        outs[s] = out.float()
    for s in outs:
        assert (outs[s] - outs[1]).abs().max().item() < 2e-3


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_split_threshold(variant):
    """Sequences at or below split_min_tokens are never split; longer ones are."""
    case = _gqa(10, 4, 16, 4, 128, 16, [4096, 4097, 100, 9000], extra_pages=1)
    say("split threshold", variant)
    ref_o, ref_l = oracle_ref(case)
    out, lse = pda.run_case(case, num_splits=8, split_min_tokens=4096, variant=VARIANTS[variant])
    check(case, out, lse, ref_o, ref_l, label="threshold")


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_page_permutation_bit_identical(variant):
    case = _gqa(11, 3, 16, 4, 128, 16, [90, 300, 17], extra_pages=9)
    say("permutation", variant)
    out1, lse1 = pda.run_case(case, variant=VARIANTS[variant])
    perm = np.random.default_rng(3).permutation(case.num_pages)
    inv = np.argsort(perm)
    case.k_cache = case.k_cache[perm].copy()
    case.v_cache = case.v_cache[perm].copy()
    bt = case.block_tables.copy()
    bt[bt >= 0] = inv[bt[bt >= 0]]
    case.block_tables = bt
    out2, lse2 = pda.run_case(case, variant=VARIANTS[variant])
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_poisoned_slots_and_table_tail_never_used(variant):
    """Unused pages and stale slots hold NaN, table tails hold -1 (the generator's
    poison); on top, fill every table entry past the context with a huge index."""
    case = _gqa(12, 4, 16, 4, 128, 16, [1, 17, 250, 33], extra_pages=6, max_pages=40)
    case.block_tables[case.block_tables < 0] = 2 ** 30
    say("poison", variant)
    out, lse = pda.run_case(case, variant=VARIANTS[variant])
    assert torch.isfinite(out).all()
    ref_o, ref_l = oracle_ref(case)   # the oracle reports any out-of-range entry it reads
    check(case, out, lse, ref_o, ref_l, label="poison")


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_empty_sequence_and_no_lse(variant):
    case = _gqa(13, 3, 8, 2, 128, 16, [0, 5, 40], extra_pages=1)
    say("empty sequence", variant)
    out, lse = pda.run_case(case, variant=VARIANTS[variant])
    o = out.float().cpu()
    assert (o[0] == 0).all() and torch.isinf(lse[0]).all() and (lse[0] < 0).all()
    ref_o, ref_l = oracle_ref(case)
    check(case, out, lse, ref_o, ref_l, label="empty")
    out2, lse2 = pda.run_case(case, return_lse=False, variant=VARIANTS[variant])
    assert lse2 is None and torch.equal(out, out2)


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_large_pool_64bit_offsets(variant):
    """Physical pages beyond 4 GiB of the pool (int64 page addressing)."""
    B, Hkv, d, P = 2, 1, 128, 16
    lens = [100, 37]
    small = _gqa(14, B, 4, Hkv, d, P, lens, poison=False)
    page_bytes = P * Hkv * d * 2
    base = (5 << 30) // page_bytes                    # first page past 5 GiB
    num_pages = base + small.num_pages
    say("large pool", num_pages, "pages")
    k = torch.zeros((num_pages, P, Hkv, d), dtype=torch.float16, device="cuda")
    v = torch.zeros_like(k)
    k[base:] = torch.from_numpy(small.k_cache).cuda()
    v[base:] = torch.from_numpy(small.v_cache).cuda()
    bt = torch.from_numpy(small.block_tables + base).cuda()
    q = torch.from_numpy(small.q).cuda()
    cl = torch.from_numpy(small.context_lens).cuda()
    out, lse = pda.paged_decode_attn(q, k, v, bt, cl, scale=small.scale, variant=VARIANTS[variant])
    ref_o, ref_l = oracle_ref(small)
    check(small, out, lse, ref_o, ref_l, label="large pool")
    del k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_ordered_work_with_empty_and_mixed_lengths(variant):
    """A split threshold turns on the longest-first ordering pass: empty
    sequences, sequences at and around the threshold and long split ones."""
    lens = [0, 4096, 1, 9000, 4097, 17, 0, 2500]
    case = _gqa(15, len(lens), 16, 4, 128, 16, lens, extra_pages=3)
    say("ordered", variant)
    dev = pda.to_device(case)
    shape = pda.gqa_shape(dev.q, dev.k_cache, dev.v_cache, dev.block_tables, split_min_tokens=4096)
    assert pda.plan(shape, num_splits=6).ordered == 1
    ref_o, ref_l = oracle_ref(case)
    out, lse = pda.run_case(case, dev, num_splits=6, split_min_tokens=4096,
                            variant=VARIANTS[variant])
    check(case, out, lse, ref_o, ref_l, label="ordered")
    # the same call without ordering gives the same values
    out2, lse2 = pda.run_case(case, dev, num_splits=6, variant=VARIANTS[variant])
    assert (out.float() - out2.float()).abs().max().item() < 2e-3


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("schedule", [pda.PDA_SCHEDULE_GRID, pda.PDA_SCHEDULE_BALANCED])
def test_ordered_batch_beyond_staged_lengths(variant, schedule):
    """More sequences than the planning pass stages in LDS (8192): it then
    reads each length from memory whenever it needs it.  9000 short and a few
    long sequences (MQA, G = 8), every row checked."""
    rng = np.random.default_rng(31)
    lens = rng.integers(0, 49, 9000)
    lens[:6] = [0, 1, 3000, 17, 2049, 4096]
    lens[-3:] = [5000, 0, 33]
    case = _gqa(77 + schedule, len(lens), 8, 1, 64, 16, lens.tolist(), extra_pages=2)
    say("ordered large batch", variant, schedule)
    dev = pda.to_device(case)
    shape = pda.gqa_shape(dev.q, dev.k_cache, dev.v_cache, dev.block_tables,
                          split_min_tokens=1024, schedule=schedule)
    assert pda.plan(shape, num_splits=4).ordered == 1
    ref_o, ref_l = oracle_ref(case)
    out, lse = pda.run_case(case, dev, num_splits=4, split_min_tokens=1024, schedule=schedule,
                            variant=VARIANTS[variant])
    check(case, out, lse, ref_o, ref_l, label="large batch %d" % schedule)


def test_graph_capture_and_replay():
    """The entry point is capture-safe (no allocation, no memset, no host sync):
    a call with splits, the combine and the ordering pass is captured into a
    HIP graph and replayed several times, with eager work and synchronizations
    between replays; every replay matches the eager result bit for bit."""
    lens = [3000, 17, 0, 5000]
    case = _gqa(16, len(lens), 16, 4, 128, 16, lens, extra_pages=2)
    say("graph capture")
    dev = pda.to_device(case)
    kw = dict(scale=case.scale, num_splits=4, split_min_tokens=1024)
    eager_o, eager_l = pda.paged_decode_attn(dev.q, dev.k_cache, dev.v_cache, dev.block_tables,
                                             dev.context_lens, **kw)
    shape = pda.gqa_shape(dev.q, dev.k_cache, dev.v_cache, dev.block_tables, split_min_tokens=1024)
    ws = pda.workspace_for(shape, mla=False, num_splits=4, device="cuda")
    out = torch.empty_like(eager_o)
    lse = torch.empty_like(eager_l)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up on the capture stream
        pda.paged_decode_attn(dev.q, dev.k_cache, dev.v_cache, dev.block_tables,
                              dev.context_lens, out=out, lse=lse, workspace=ws, **kw)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pda.paged_decode_attn(dev.q, dev.k_cache, dev.v_cache, dev.block_tables,
                              dev.context_lens, out=out, lse=lse, workspace=ws, **kw)
    for i in range(4):
        out.fill_(float("nan"))
        lse.fill_(0.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_o) and torch.equal(lse, eager_l), "replay %d" % i
        # unrelated eager work between replays
        pda.paged_decode_attn(dev.q, dev.k_cache, dev.v_cache, dev.block_tables,
                              dev.context_lens, **kw)
        torch.cuda.synchronize()


BAL = pda.PDA_SCHEDULE_BALANCED


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("num_splits,thr", [(0, 0), (8, 0), (8, 4096)])
def test_balanced_schedule_mixed_lengths(variant, num_splits, thr):
    """The balanced schedule: the device-side planning pass cuts the batch's
    pages into near-equal chunks; empty, tiny, threshold-length and long
    sequences."""
    lens = [0, 4096, 1, 9000, 4097, 17, 0, 2500, 16384, 700]
    case = _gqa(17, len(lens), 16, 4, 128, 16, lens, extra_pages=3)
    say("balanced", variant, num_splits, thr)
    dev = pda.to_device(case)
    shape = pda.gqa_shape(dev.q, dev.k_cache, dev.v_cache, dev.block_tables, schedule=BAL,
                          split_min_tokens=thr, variant=VARIANTS[variant])
    p = pda.plan(shape, num_splits=num_splits)
    assert p.ordered == 1 and p.pages_per_split == 0
    ref_o, ref_l = oracle_ref(case)
    out, lse = pda.run_case(case, dev, num_splits=num_splits, split_min_tokens=thr,
                            variant=VARIANTS[variant], schedule=BAL)
    check(case, out, lse, ref_o, ref_l, label="balanced")
    out2, lse2 = pda.run_case(case, dev, num_splits=num_splits, split_min_tokens=thr,
                              variant=VARIANTS[variant], schedule=BAL)
    assert torch.equal(out, out2) and torch.equal(lse, lse2), "run-to-run differs"


@pytest.mark.parametrize("batch", [1, 4])
def test_balanced_schedule_long_context(batch):
    case = W.gqa_long(batch)
    say("balanced", case.name)
    dev = pda.to_device(case)
    ref_o, ref_l = oracle_ref(case)
    out, lse = pda.run_case(case, dev, schedule=BAL)
    check(case, out, lse, ref_o, ref_l, label="balanced %s" % case.name)


def test_balanced_schedule_ragged_fp8_full_size():
    """The ragged fp8 workload (B=128, log-uniform lengths up to 16384) under
    the balanced schedule with no split threshold, up to 8 splits; every row."""
    case = W.ragged_fp8()
    say("balanced", case.name)
    dev = pda.to_device(case)
    ref_o, ref_l = oracle_ref(case)
    out, lse = pda.run_case(case, dev, num_splits=8, schedule=BAL)
    check(case, out, lse, ref_o, ref_l, label="balanced ragged")


def test_balanced_schedule_multi_token():
    case = W.make_gqa(batch=5, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                      context_lens=[3, 5000, 100, 1, 2048], q_dtype="bf16", kv_dtype="bf16",
                      seed=18, q_len=3, extra_pages=2)
    say("balanced multi-token")
    ref_o, ref_l = oracle_ref(case)
    out, lse = pda.run_case(case, schedule=BAL)
    check(case, out, lse, ref_o, ref_l, label="balanced q_len=3")


@pytest.fixture(scope="module")
def very_long():
    case = _gqa(31, 2, 16, 2, 128, 16, [262144, 5000], poison=False)
    return case, oracle_ref(case)


@pytest.mark.parametrize("splits", [0, 200, 1024])
def test_very_long_context_many_splits(very_long, splits):
    """262144 and 5000 tokens: 16384 table entries per row, and split counts
    past the 64 per row that the combine keeps in registers (the rest take its
    loop)."""
    case, (ref_o, ref_l) = very_long
    say("very long context", splits)
    dev = pda.to_device(case)
    p = pda.plan(pda.gqa_shape(dev.q, dev.k_cache, dev.v_cache, dev.block_tables),
                 num_splits=splits)
    assert splits == 0 or p.max_splits > 64
    for name, v in VARIANTS.items():
        out, lse = pda.run_case(case, dev, num_splits=splits, variant=v)
        check(case, out, lse, ref_o, ref_l, label="very long %d %s" % (splits, name))



@pytest.mark.parametrize("d,dt", [(64, "f16"), (128, "bf16"), (256, "f16")])
@pytest.mark.parametrize("num_splits,thr", [(2, 0), (7, 0), (16, 0), (8, 600)])
def test_combine_of_many_rows_with_few_splits(d, dt, num_splits, thr):
    """Batches with many (sequence, head) rows and at most 16 splits merge in
    the row-per-thread combine (at least 64 workgroups of rows); lengths from 1
    token to several splits, with and without a split threshold."""
    rng = np.random.default_rng(d + num_splits + thr)
    lens = [int(x) for x in rng.integers(1, 2500, 32)]
    lens[:3] = [1, 17, 2499]
    case = _gqa(200 + d + num_splits, 32, 32, 8, d, 16, lens, q_dtype=dt, kv_dtype=dt)
    say("combine rows", d, dt, num_splits, thr)
    out, lse = pda.run_case(case, num_splits=num_splits, split_min_tokens=thr)
    ref_o, ref_l = oracle_ref(case)
    check(case, out, lse, ref_o, ref_l, label="rows combine d=%d S=%d thr=%d" % (d, num_splits, thr))


def test_combine_of_many_rows_multi_token():
    lens = [int(x) for x in np.random.default_rng(5).integers(2, 3000, 24)]
    case = W.make_gqa(batch=24, num_q_heads=16, num_kv_heads=4, head_dim=128, page_size=16,
                      context_lens=lens, q_dtype="f16", kv_dtype="f16", seed=207, q_len=2,
                      causal=True)
    say("combine rows multi-token")
    for s in (4, 12):
        out, lse = pda.run_case(case, num_splits=s)
        ref_o, ref_l = oracle_ref(case)
        check(case, out, lse, ref_o, ref_l, label="rows combine q_len=2 S=%d" % s)


@pytest.mark.parametrize("d,dt,kv", [(128, "f16", "f16"), (128, "bf16", "bf16"), (64, "f16", "f16"),
                                     (256, "bf16", "bf16"), (128, "f16", "e4m3"),
                                     (128, "bf16", "e4m3"), (64, "bf16", "e4m3")])
@pytest.mark.parametrize("layout", [0, 1])
def test_one_wave_variant(d, dt, kv, layout):
    """The matrix-core kernel with one wave per work unit (PDA_GQA_MFMA_1WAVE),
    requested explicitly for every cache type and head dim it takes: lengths
    across page and tile boundaries, an empty sequence, no split and several
    splits, both page layouts."""
    lens = [0, 1, 15, 16, 17, 333, 1030, 70]
    case = _gqa(d * 3 + len(kv) + layout, len(lens), 32, 8, d, 16, lens, dt, kv, extra_pages=3,
                kv_layout=layout)
    say("one wave", d, dt, kv, layout)
    dev = pda.to_device(case)
    ref_o, ref_l = oracle_ref(case)
    for s in (1, 4, 0):
        sh = pda.gqa_shape(dev.q, dev.k_cache, dev.v_cache, dev.block_tables,
                           variant=pda.PDA_GQA_MFMA_1WAVE, kv_layout=layout)
        assert pda.plan(sh, num_splits=s).waves_per_unit == 1
        out, lse = pda.run_case(case, dev, num_splits=s, variant=pda.PDA_GQA_MFMA_1WAVE)
        check(case, out, lse, ref_o, ref_l, label="one wave d=%d %s/%s S=%d" % (d, dt, kv, s))
        out2, lse2 = pda.run_case(case, dev, num_splits=s, variant=pda.PDA_GQA_MFMA_1WAVE)
        assert torch.equal(out, out2) and torch.equal(lse, lse2), "run-to-run differs"
        # against the four-wave layout: the same rows, another summation order
        out4, _ = pda.run_case(case, dev, num_splits=s, variant=pda.PDA_GQA_MFMA_4WAVE)
        assert (out4.float() - out.float()).abs().max().item() < 2e-3


@pytest.mark.parametrize("Hq,Hkv,q_len", [(32, 8, 2), (32, 8, 4), (64, 8, 3), (32, 1, 1),
                                         (24, 1, 1)])
def test_one_wave_variant_multi_token(Hq, Hkv, q_len):
    """Several query tokens (causal) and large groups on one-wave workgroups:
    the (query token, head) rows of a KV group fill one 16-column tile (G = 4,
    q_len <= 4) or two (G = 8 with three tokens, MQA with 32 and 24 heads:
    32-row units, the last with 8 padded columns)."""
    case = _gqa(70 + q_len + Hq + Hkv, 3, Hq, Hkv, 128, 16, [q_len, 200, 2500], q_len=q_len,
                extra_pages=2)
    say("one wave multi-token", Hq, Hkv, q_len)
    dev = pda.to_device(case)
    ref_o, ref_l = oracle_ref(case)
    for s in (1, 5):
        out, lse = pda.run_case(case, dev, num_splits=s, variant=pda.PDA_GQA_MFMA_1WAVE)
        check(case, out, lse, ref_o, ref_l, label="one wave Hq=%d Hkv=%d q_len=%d S=%d"
              % (Hq, Hkv, q_len, s))


@pytest.mark.parametrize("Hq,Hkv,d,lens", [(24, 1, 128, [700, 5, 1200]), (48, 2, 256, [300, 999, 64]),
                                          (40, 1, 128, [3000, 1, 2100])])
def test_one_wave_several_head_tiles(Hq, Hkv, d, lens):
    """One-wave units of groups that take several workgroups per KV group:
    16-row head tiles (G = 24 with a short table, G = 24 at d = 256) and
    32-row ones (G = 40 with a long table: two column tiles, two head
    tiles), with and without splits, against the oracle and the four-wave
    layout."""
    case = _gqa(Hq + d + len(lens), len(lens), Hq, Hkv, d, 16, lens, extra_pages=1)
    say("one wave head tiles", Hq, Hkv, d, lens)
    dev = pda.to_device(case)
    sh = pda.gqa_shape(dev.q, dev.k_cache, dev.v_cache, dev.block_tables,
                       variant=pda.PDA_GQA_MFMA_1WAVE)
    assert pda.plan(sh, num_splits=1).head_tiles >= 2
    ref_o, ref_l = oracle_ref(case)
    for s in (1, 3):
        out, lse = pda.run_case(case, dev, num_splits=s, variant=pda.PDA_GQA_MFMA_1WAVE)
        check(case, out, lse, ref_o, ref_l, label="one wave Hq=%d Hkv=%d d=%d S=%d"
              % (Hq, Hkv, d, s))
        out4, _ = pda.run_case(case, dev, num_splits=s, variant=pda.PDA_GQA_MFMA_4WAVE)
        assert (out4.float() - out.float()).abs().max().item() < 2e-3
