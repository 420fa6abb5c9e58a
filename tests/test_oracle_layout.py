"""Pins for the head-major page layout ([num_pages, Hkv, P, d] instead of
[num_pages, P, Hkv, d]).  The pages address a cached element through
separate page, slot and head strides ("From MHA to MLA" sec. 5, paged
loads; the drill page sec. 4, the page loop), so a layout only moves
elements: the attention of a case must not depend on it.

 - the generator stores the same values in both orders (explicit indexing);
 - the oracle gives bit-identical results for the two orders of one case
   (one query token, several with a causal mask, fp8 with scales, splits);
 - the oracle's append into a head-major cache writes element (page, head,
   slot) from (sequence, token, head), checked by explicit indexing, and
   equals the token-major append of the same rows.
"""
import numpy as np
import pytest

import oracle
from decode_attention_paged_02_amd import workloads as W


def _pair(**kw):
    base = dict(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=16,
                context_lens=[37, 1, 100], q_dtype="f32", kv_dtype="f32", seed=9, extra_pages=3)
    base.update(kw)
    return W.make_gqa(kv_layout=0, **base), W.make_gqa(kv_layout=1, **base)


def _ref(c, **kw):
    return oracle.paged_attention(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens,
                                  scale=c.scale, q_dtype=c.q_dtype, kv_dtype=c.kv_dtype,
                                  k_scale=c.k_scale, v_scale=c.v_scale, causal=c.causal,
                                  kv_layout=c.kv_layout, **kw)


def test_generator_stores_the_same_elements():
    t, h = _pair()
    assert h.k_cache.shape == (t.k_cache.shape[0], 2, 16, 64)
    assert h.num_kv_heads == t.num_kv_heads == 2
    rng = np.random.default_rng(0)
    for _ in range(200):
        p, s, k = rng.integers(t.k_cache.shape[0]), rng.integers(16), rng.integers(2)
        assert np.array_equal(h.k_cache[p, k, s], t.k_cache[p, s, k], equal_nan=True)
        assert np.array_equal(h.v_cache[p, k, s], t.v_cache[p, s, k], equal_nan=True)
    assert np.array_equal(h.q, t.q) and np.array_equal(h.block_tables, t.block_tables)


@pytest.mark.parametrize("kw", [
    dict(),
    dict(q_len=3, causal=True, q_dtype="f16", kv_dtype="f16"),
    dict(q_len=2, causal=False, q_dtype="bf16", kv_dtype="bf16"),
    dict(q_dtype="f16", kv_dtype="e4m3", num_kv_heads=4, num_q_heads=16),
])
def test_oracle_does_not_depend_on_the_layout(kw):
    t, h = _pair(**kw)
    o_t, l_t = _ref(t)
    o_h, l_h = _ref(h)
    assert np.isfinite(o_t).all()
    assert np.array_equal(o_t, o_h) and np.array_equal(l_t, l_h)


def test_oracle_split_ranges_in_head_major_layout():
    t, h = _pair(context_lens=[300, 17, 64])
    tb = np.array([16, 0, 32], np.int32)
    te = np.array([160, 17, 48], np.int32)
    a = _ref(t, tok_begin=tb, tok_end=te)
    b = _ref(h, tok_begin=tb, tok_end=te)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_oracle_rejects_unknown_layout():
    t, _ = _pair()
    with pytest.raises(ValueError):
        oracle.paged_attention(t.q, t.k_cache, t.v_cache, t.block_tables, t.context_lens,
                               scale=t.scale, q_dtype="f32", kv_dtype="f32", kv_layout=2)


@pytest.mark.parametrize("cache_dtype", ["f16", "e4m3"])
def test_append_into_head_major_cache(cache_dtype):
    rng = np.random.default_rng(3)
    B, s_new, H, w, P, pages = 3, 2, 4, 16, 16, 6
    src = rng.standard_normal((B, s_new, H, w)).astype(np.float16)
    table = np.array([[4, 1], [0, 5], [2, 3]], np.int32)
    pos = np.array([15, -1, 3], np.int32)             # sequence 0 crosses a page boundary
    scale = 0.01 if cache_dtype == "e4m3" else 1.0
    npdt = np.uint8 if cache_dtype == "e4m3" else np.float16
    cache_h = np.zeros((pages, H, P, w), npdt)
    got = oracle.kv_append(src, cache_h, table, pos, src_dtype="f16", cache_dtype=cache_dtype,
                           scale=scale, kv_layout=1)
    tok = oracle.kv_append(src, np.zeros((pages, P, H, w), npdt), table, pos, src_dtype="f16",
                           cache_dtype=cache_dtype, scale=scale)
    assert np.array_equal(got, tok.transpose(0, 2, 1, 3))
    if cache_dtype == "f16":
        want = np.zeros_like(cache_h)
        for b in range(B):
            if pos[b] < 0:
                continue
            for t in range(s_new):
                p = pos[b] + t
                for h in range(H):
                    want[table[b, p // P], h, p % P] = src[b, t, h]
        assert np.array_equal(got, want)
