"""Pins for the fp64 oracle: each test ties it to something other than itself.

 - element decoders vs library dtype casts (every bit pattern);
 - a pure-Python brute force on tiny inputs that reaches the paged tokens by
   scanning the physical pool (not through the block table) and uses the
   unshifted softmax exp(s)/sum exp(s);
 - torch's scaled_dot_product_attention (fp64, CPU) on K/V gathered with numpy
   fancy indexing and expanded with repeat_interleave (contiguous grouping);
 - closed forms (q = 0, ctx = 1, constant keys) and invariants (page
   permutation, MHA equivalence, split + combine == unsplit, NaN poison);
 - the numbers the pages print (the drill's worked example, the absorption
   demo output).
"""
import math
import random

import numpy as np
import pytest
import torch

import oracle
from decode_attention_paged_02_amd import workloads as W


# ----------------------------------------------------------------- decoders

def _same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(
        a[~np.isnan(a)], b[~np.isnan(b)])


def test_decode_f16_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    assert _same(oracle.decode(bits.view(np.float16), "f16"), ref)


def test_decode_bf16_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert _same(oracle.decode(bits, "bf16"), ref)


def test_decode_e4m3_all_patterns():
    bits = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(bits).view(torch.float8_e4m3fn).double().numpy()
    got = oracle.decode(bits, "e4m3")
    assert _same(got, ref)
    # OCP E4M3FN facts: max 448, min subnormal 2^-9, only 0x7F/0xFF are NaN
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9
    assert np.isnan(got).sum() == 2 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def test_decode_f32_roundtrip():
    x = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    assert np.array_equal(oracle.decode(x, "f32"), x.astype(np.float64))


# ---------------------------------------------------------------- helpers

def _dense_from_pool(case, b):
    """K/V rows of sequence b in logical order, found by scanning the pool.

    Walks every physical page of the pool and asks which logical page of
    sequence b (if any) it holds -- an independent route to the paging."""
    P = case.page_size
    n = int(case.context_lens[b])
    npages = (n + P - 1) // P
    where = {}
    for lp in range(npages):
        where[int(case.block_tables[b, lp])] = lp
    k = W.to_float32(case.k_cache, case.kv_dtype).astype(np.float64) * case.k_scale
    v = W.to_float32(case.v_cache, case.kv_dtype).astype(np.float64) * case.v_scale
    K = [None] * n
    V = [None] * n
    for phys in range(case.num_pages):
        if phys not in where:
            continue
        lp = where[phys]
        for slot in range(P):
            j = lp * P + slot
            if j < n:
                K[j] = k[phys, slot]
                V[j] = v[phys, slot]
    return K, V


def _brute(case):
    """Pure-Python fp64 attention with the unshifted softmax (tiny inputs only)."""
    B, Hq = case.batch, case.num_q_heads
    G = Hq // case.num_kv_heads
    q = W.to_float32(case.q, case.q_dtype).astype(np.float64)
    out = np.zeros((B, Hq, case.head_dim_v))
    lse = np.zeros((B, Hq))
    for b in range(B):
        K, V = _dense_from_pool(case, b)
        for h in range(Hq):
            kvh = h // G
            s = [case.scale * sum(float(a) * float(c) for a, c in zip(q[b, h], K[j][kvh]))
                 for j in range(len(K))]
            e = [math.exp(x) for x in s]
            z = sum(e)
            for d in range(case.head_dim_v):
                out[b, h, d] = sum(e[j] * float(V[j][kvh][d]) for j in range(len(K))) / z
            lse[b, h] = math.log(z)
    return out, lse


def _run(case, **kw):
    return oracle.paged_attention(case.q, case.k_cache, case.v_cache, case.block_tables,
                                  case.context_lens, scale=case.scale, q_dtype=case.q_dtype,
                                  kv_dtype=case.kv_dtype, k_scale=case.k_scale,
                                  v_scale=case.v_scale, **kw)


def _tiny(seed, *, B=None, Hkv=None, G=None, d=None, P=None, lens=None, dtype="f32",
          q_dtype=None, poison=True, extra=3):
    r = random.Random(seed)
    B = B or r.randint(1, 3)
    Hkv = Hkv or r.choice([1, 2])
    G = G or r.choice([1, 2, 3])
    d = d or r.choice([1, 3, 4, 8])
    P = P or r.choice([1, 2, 4, 16])
    lens = lens or [r.randint(1, 40) for _ in range(B)]
    return W.make_gqa(batch=B, num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=d,
                      page_size=P, context_lens=lens, q_dtype=q_dtype or dtype,
                      kv_dtype=dtype, seed=seed, extra_pages=extra, poison=poison)


# -------------------------------------------------------------- brute force

@pytest.mark.parametrize("seed", range(12))
def test_oracle_matches_bruteforce_tiny(seed):
    case = _tiny(seed)
    out, lse = _run(case)
    bo, bl = _brute(case)
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-12)


def test_oracle_matches_bruteforce_tiny_gqa_config():
    case = W.tiny_gqa()
    out, lse = _run(case)
    bo, bl = _brute(case)
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-12)


@pytest.mark.parametrize("dtype,q_dtype", [("f16", "f16"), ("bf16", "bf16"), ("e4m3", "f16")])
def test_oracle_matches_bruteforce_stored_types(dtype, q_dtype):
    case = _tiny(77, B=2, Hkv=2, G=2, d=8, P=4, lens=[9, 13], dtype=dtype, q_dtype=q_dtype)
    if dtype == "e4m3":
        case.k_scale, case.v_scale = 0.37, 1.9
    out, lse = _run(case)
    bo, bl = _brute(case)
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-12)


# ------------------------------------------------------------ library SDPA

def _gather_np(case, b):
    P = case.page_size
    n = int(case.context_lens[b])
    j = np.arange(n)
    pages = case.block_tables[b, j // P]
    k = W.to_float32(case.k_cache, case.kv_dtype)[pages, j % P].astype(np.float64)
    v = W.to_float32(case.v_cache, case.kv_dtype)[pages, j % P].astype(np.float64)
    return k * case.k_scale, v * case.v_scale        # [n, Hkv, d]


@pytest.mark.parametrize("seed,dtype", [(3, "f32"), (4, "f16"), (5, "bf16"), (6, "e4m3")])
def test_oracle_matches_torch_sdpa(seed, dtype):
    case = W.make_gqa(batch=3, num_q_heads=12, num_kv_heads=3, head_dim=32, page_size=16,
                      context_lens=[1, 45, 130], q_dtype="f16" if dtype == "e4m3" else dtype,
                      kv_dtype=dtype, seed=seed, extra_pages=5)
    if dtype == "e4m3":
        case.k_scale, case.v_scale = 0.021, 0.013
    out, lse = _run(case)
    G = case.num_q_heads // case.num_kv_heads
    q = torch.from_numpy(W.to_float32(case.q, case.q_dtype).astype(np.float64))
    for b in range(case.batch):
        k, v = _gather_np(case, b)
        kt = torch.from_numpy(k).transpose(0, 1).repeat_interleave(G, dim=0).contiguous()
        vt = torch.from_numpy(v).transpose(0, 1).repeat_interleave(G, dim=0).contiguous()
        qb = q[b].unsqueeze(1)                                     # [Hq, 1, d]
        ref = torch.nn.functional.scaled_dot_product_attention(qb, kt, vt, scale=case.scale)
        np.testing.assert_allclose(out[b], ref[:, 0].numpy(), rtol=0, atol=1e-12)
        ref_lse = torch.logsumexp(case.scale * (qb @ kt.transpose(1, 2))[:, 0], dim=-1)
        np.testing.assert_allclose(lse[b], ref_lse.numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------------------- closed forms

@pytest.mark.parametrize("n", [1, 15, 16, 17, 37, 100])
def test_zero_query_gives_mean_of_values(n):
    case = W.make_gqa(batch=1, num_q_heads=4, num_kv_heads=2, head_dim=16, page_size=16,
                      context_lens=[n], q_dtype="f32", kv_dtype="f32", seed=n, extra_pages=4)
    case.q[:] = 0
    out, lse = _run(case)
    _, v = _gather_np(case, 0)
    for h in range(4):
        np.testing.assert_allclose(out[0, h], v[:, h // 2].mean(axis=0), rtol=0, atol=1e-12)
        assert abs(lse[0, h] - math.log(n)) < 1e-12


def test_single_token_returns_that_value_row():
    case = W.make_gqa(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=16,
                      context_lens=[1, 1], q_dtype="f32", kv_dtype="f32", seed=11,
                      extra_pages=3)
    out, lse = _run(case)
    q = case.q.astype(np.float64)
    for b in range(2):
        k, v = _gather_np(case, b)
        for h in range(8):
            np.testing.assert_array_equal(out[b, h], v[0, h // 4])
            assert abs(lse[b, h] - case.scale * float(q[b, h] @ k[0, h // 4])) < 1e-12


def test_constant_keys_give_mean_value_and_shifted_lse():
    case = W.make_gqa(batch=1, num_q_heads=2, num_kv_heads=1, head_dim=8, page_size=4,
                      context_lens=[23], q_dtype="f32", kv_dtype="f32", seed=12, extra_pages=2)
    key = np.random.default_rng(1).standard_normal(8).astype(np.float32)
    case.k_cache[:] = key
    out, lse = _run(case)
    _, v = _gather_np(case, 0)
    for h in range(2):
        s = case.scale * float(case.q[0, h].astype(np.float64) @ key.astype(np.float64))
        np.testing.assert_allclose(out[0, h], v[:, 0].mean(axis=0), rtol=0, atol=1e-12)
        assert abs(lse[0, h] - (s + math.log(23))) < 1e-12


# --------------------------------------------------------------- invariants

def test_page_permutation_is_bit_identical():
    case = W.make_gqa(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=32, page_size=16,
                      context_lens=[5, 64, 99], q_dtype="f16", kv_dtype="f16", seed=21,
                      extra_pages=7)
    out, lse = _run(case)
    perm = np.random.default_rng(5).permutation(case.num_pages)   # new_pos -> old page
    inv = np.argsort(perm)                                        # old page -> new_pos
    case.k_cache = case.k_cache[perm].copy()
    case.v_cache = case.v_cache[perm].copy()
    bt = case.block_tables.copy()
    valid = bt >= 0
    bt[valid] = inv[bt[valid]]
    case.block_tables = bt
    out2, lse2 = _run(case)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_gqa_equals_mha_on_repeat_interleaved_cache():
    """Contiguous grouping: GQA equals MHA over K/V repeated G times along heads
    with repeat_interleave (an interleaved h % Hkv mapping fails this)."""
    case = W.make_gqa(batch=2, num_q_heads=12, num_kv_heads=3, head_dim=16, page_size=8,
                      context_lens=[19, 40], q_dtype="f32", kv_dtype="f32", seed=31,
                      extra_pages=2)
    out, lse = _run(case)
    G = 4
    mha = W.PagedCase(**{**case.__dict__})
    mha.k_cache = np.repeat(case.k_cache, G, axis=2)
    mha.v_cache = np.repeat(case.v_cache, G, axis=2)
    out2, lse2 = _run(mha)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_g1_is_plain_mha():
    case = W.make_gqa(batch=2, num_q_heads=4, num_kv_heads=4, head_dim=8, page_size=4,
                      context_lens=[7, 12], q_dtype="f32", kv_dtype="f32", seed=41,
                      extra_pages=1)
    out, _ = _run(case)
    q = case.q.astype(np.float64)
    for b in range(2):
        k, v = _gather_np(case, b)
        for h in range(4):
            s = case.scale * (k[:, h] @ q[b, h])
            p = np.exp(s - s.max())
            np.testing.assert_allclose(out[b, h], (p / p.sum()) @ v[:, h], rtol=0, atol=1e-12)


@pytest.mark.parametrize("S", [2, 3, 7])
def test_split_then_combine_equals_unsplit(S):
    case = W.tiny_gqa()
    out, lse = _run(case)
    B, Hq = case.batch, case.num_q_heads
    P = case.page_size
    po = np.zeros((B, Hq, S, case.head_dim_v))
    pl = np.zeros((B, Hq, S))
    for s in range(S):
        tb = np.zeros(B, np.int32)
        te = np.zeros(B, np.int32)
        for b, n in enumerate(case.context_lens):
            pages = -(-int(n) // P)
            per = -(-pages // S)
            tb[b] = min(s * per * P, n)
            te[b] = min((s + 1) * per * P, n)
        o_s, l_s = _run(case, tok_begin=tb, tok_end=te)
        po[:, :, s], pl[:, :, s] = o_s, l_s
    # S=7 leaves the 37-token sequence (3 pages) with empty splits: lse -inf, weight 0
    if S == 7:
        assert np.isneginf(pl[0, :, 3:]).all() and (po[0, :, 3:] == 0).all()
    co, cl = oracle.combine(po, pl)
    np.testing.assert_allclose(co, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(cl, lse, rtol=0, atol=1e-12)
    w = np.exp(pl - cl[..., None])
    np.testing.assert_allclose(w.sum(-1), 1.0, rtol=0, atol=1e-12)


def test_combine_all_empty_row():
    co, cl = oracle.combine(np.zeros((1, 3, 4)), np.full((1, 3), -np.inf))
    assert (co == 0).all() and np.isneginf(cl).all()


def test_nan_poison_never_reaches_the_result():
    clean = W.tiny_gqa(poison=False)
    dirty = W.tiny_gqa(poison=True)
    assert np.isnan(dirty.k_cache).any() and (dirty.block_tables < 0).any()
    o1, l1 = _run(clean)
    o2, l2 = _run(dirty)
    assert np.isfinite(o2).all() and np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_table_entry_out_of_range_is_reported():
    case = W.tiny_gqa()
    case.block_tables[0, 0] = case.num_pages   # one past the pool
    with pytest.raises(ValueError, match="out of range"):
        _run(case)


def test_empty_context_defensive_definition():
    case = W.make_gqa(batch=2, num_q_heads=2, num_kv_heads=1, head_dim=4, page_size=4,
                      context_lens=[0, 3], q_dtype="f32", kv_dtype="f32", seed=2,
                      max_pages=1)
    out, lse = _run(case)
    assert (out[0] == 0).all() and np.isneginf(lse[0]).all() and np.isfinite(lse[1]).all()


# ------------------------------------------------- the pages' printed numbers

def test_drill_worked_example(golden_dir):
    """ctx=37, P=16, table [9, 3, 7, ...]: three pages are read; nothing past
    the third table entry is touched (the tail holds an out-of-range index,
    which the oracle would report if it read it)."""
    import json
    import os
    g = json.load(open(os.path.join(golden_dir, "drill_worked_example.json")))
    P, n = g["page_size"], g["ctx"]
    assert -(-n // P) == g["pages_read"]
    rng = np.random.default_rng(37)
    num_pages, d = 12, 8
    k = rng.standard_normal((num_pages, P, 1, d)).astype(np.float32)
    v = rng.standard_normal((num_pages, P, 1, d)).astype(np.float32)
    touched = g["block_table_prefix"]
    for p in range(num_pages):
        if p not in touched:
            k[p], v[p] = np.nan, np.nan
    last = touched[-1]
    k[last, n - 2 * P:], v[last, n - 2 * P:] = np.nan, np.nan       # slots 5..15 of page 7
    table = np.array([touched + [2 ** 31 - 1] * 5], dtype=np.int32)
    q = rng.standard_normal((1, 2, d)).astype(np.float32)
    out, lse = oracle.paged_attention(q, k, v, table, np.array([n], np.int32), scale=0.3,
                                      q_dtype="f32", kv_dtype="f32")
    rows = [(touched[j // P], j % P) for j in range(n)]
    K = np.stack([k[p, s, 0] for p, s in rows]).astype(np.float64)
    V = np.stack([v[p, s, 0] for p, s in rows]).astype(np.float64)
    for h in range(2):
        s = 0.3 * (K @ q[0, h].astype(np.float64))
        p_ = np.exp(s - s.max())
        np.testing.assert_allclose(out[0, h], p_ @ V / p_.sum(), rtol=0, atol=1e-12)
        assert abs(lse[0, h] - (s.max() + math.log(p_.sum()))) < 1e-12


def _lcg(seed):
    state = seed
    while True:
        state = (state * 6364136223846793005 + 1442695040888963407) % (1 << 64)
        yield state / float(1 << 63) - 1.0


def test_absorption_demo_printed_score(golden_dir):
    """A single cached latent makes the LSE equal the score itself; the page
    prints that score for its toy absorbed-MLA example."""
    import json
    import os
    g = json.load(open(os.path.join(golden_dir, "absorption_demo.json")))
    c, d = g["latent_dim"], g["model_dim"]
    gen = _lcg(42)
    draw = lambda r, k: np.array([[next(gen) for _ in range(k)] for _ in range(r)])
    W_dkv, W_uk = draw(c, d), draw(d, c)
    h_t, q = draw(1, d)[0], draw(1, d)[0]
    c_kv = W_dkv @ h_t
    q_abs = W_uk.T @ q
    # absorbed path: MLA oracle, latent width c, no rope, one token, scale 1
    _, lse_abs = oracle.mla_attention(q_abs.reshape(1, 1, c), c_kv.reshape(1, 1, c),
                                      np.zeros((1, 1), np.int32), np.array([1], np.int32),
                                      scale=1.0, d_latent=c, q_dtype="f64", kv_dtype="f64")
    # materialized path: per-head key W_UK c through the GQA oracle
    k_mat = (W_uk @ c_kv).reshape(1, 1, 1, d)
    _, lse_mat = oracle.paged_attention(q.reshape(1, 1, d), k_mat, k_mat,
                                        np.zeros((1, 1), np.int32), np.array([1], np.int32),
                                        scale=1.0, q_dtype="f64", kv_dtype="f64")
    tol = 0.5 * 10.0 ** -g["printed_decimals"]
    assert abs(lse_abs[0, 0] - g["score_printed"]) <= tol
    assert abs(lse_mat[0, 0] - g["score_printed"]) <= tol
    assert abs(lse_abs[0, 0] - lse_mat[0, 0]) < 1e-15 + 2 * g["abs_diff_printed"]
