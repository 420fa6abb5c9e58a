"""Pins for the oracle's MLA path.

 - Weight absorption is an associativity identity ("From MHA to MLA" sec. 6;
   "Attention Kernel Variants", MLA section): attention over materialized
   per-head keys [W_UK_r c ; k_R] and values W_UV_r c (through the GQA oracle,
   MHA layout) equals W_UV_r applied to the latent output of the MLA oracle
   run with the absorbed query [W_UK_r^T q_C ; q_R].  Weights are synthetic.
 - The rope block only enters the score: with q_R = 0, randomizing the rope
   columns changes nothing; making them equal across tokens leaves the output
   unchanged and shifts the LSE by scale * q_R . k_R (softmax shift invariance).
 - ctx = 1 returns the latent of that token.
"""
import math

import numpy as np

import oracle
from decode_attention_paged_02_amd import workloads as W

DL, DR = 32, 8          # small latent / rope widths for fast fp64 checks


def _case(seed, lens, Hq=4, P=8, dtype="f32", kv_dtype=None):
    return W.make_mla(batch=len(lens), num_q_heads=Hq, d_latent=DL, d_rope=DR, page_size=P,
                      context_lens=lens, dtype=dtype, seed=seed, scale=1 / math.sqrt(24.0),
                      extra_pages=2, kv_dtype=kv_dtype)


def _mla(case, q=None, kv=None, qd=None, kd=None):
    return oracle.mla_attention(case.q if q is None else q,
                                case.k_cache if kv is None else kv, case.block_tables,
                                case.context_lens, scale=case.scale, d_latent=case.d_latent,
                                q_dtype=qd or case.q_dtype, kv_dtype=kd or case.kv_dtype,
                                kv_scale=case.k_scale)


def test_absorbed_equals_materialized_per_head():
    case = _case(1, [13, 40], Hq=3)
    rng = np.random.default_rng(2)
    dqk, dv = 12, 10                                   # per-head content-key / value widths
    W_UK = rng.standard_normal((3, dqk, DL)) / math.sqrt(DL)
    W_UV = rng.standard_normal((3, dv, DL)) / math.sqrt(DL)
    q_c = rng.standard_normal((2, 3, dqk))
    q_r = rng.standard_normal((2, 3, DR))
    lat = case.k_cache.astype(np.float64)              # [pages, P, DL + DR]
    c, k_r = lat[..., :DL], lat[..., DL:]
    # materialized MHA cache: per head r, K_r = [W_UK_r c ; k_R], V_r = W_UV_r c
    k_mat = np.concatenate([np.einsum("rkl,nsl->nsrk", W_UK, c),
                            np.broadcast_to(k_r[:, :, None, :], c.shape[:2] + (3, DR))], -1)
    v_mat = np.einsum("rvl,nsl->nsrv", W_UV, c)
    q_mat = np.concatenate([q_c, q_r], -1)
    o_mat, l_mat = oracle.paged_attention(q_mat, np.ascontiguousarray(k_mat),
                                          np.ascontiguousarray(v_mat), case.block_tables,
                                          case.context_lens, scale=case.scale,
                                          q_dtype="f64", kv_dtype="f64")
    # absorbed: q_hat = [W_UK_r^T q_C ; q_R] against the shared latent record
    q_hat = np.concatenate([np.einsum("rkl,brk->brl", W_UK, q_c), q_r], -1)
    o_lat, l_lat = _mla(case, q=q_hat, kv=lat, qd="f64", kd="f64")
    o_abs = np.einsum("rvl,brl->brv", W_UV, o_lat)
    np.testing.assert_allclose(o_abs, o_mat, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_lat, l_mat, rtol=0, atol=1e-12)


def test_rope_columns_only_enter_the_score():
    case = _case(3, [17, 64])
    q = case.q.copy()
    q[..., DL:] = 0
    o1, l1 = _mla(case, q=q)
    kv = case.k_cache.copy()
    kv[..., DL:] = np.random.default_rng(4).standard_normal(kv[..., DL:].shape)
    o2, l2 = _mla(case, q=q, kv=kv)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_constant_rope_shifts_lse_only():
    case = _case(5, [9, 33])
    kv = case.k_cache.copy()
    kv[..., DL:] = 0
    o1, l1 = _mla(case, kv=kv)
    k_r = np.random.default_rng(6).standard_normal(DR).astype(np.float32)
    kv[..., DL:] = k_r
    o2, l2 = _mla(case, kv=kv)
    shift = case.scale * (case.q[..., DL:].astype(np.float64) @ k_r.astype(np.float64))
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1 + shift, rtol=0, atol=1e-12)


def test_single_token_returns_its_latent():
    case = _case(7, [1, 1, 1], Hq=2)
    out, lse = _mla(case)
    for b in range(3):
        rec = case.k_cache[case.block_tables[b, 0], 0].astype(np.float64)
        for h in range(2):
            np.testing.assert_array_equal(out[b, h], rec[:DL])
            assert abs(lse[b, h] - case.scale * float(case.q[b, h].astype(np.float64) @ rec)) < 1e-12


def test_mla_matches_gqa_oracle_with_aliased_value():
    """MLA == the GQA oracle with Hkv = 1, K = the record, V = its first DL columns."""
    case = _case(8, [5, 50, 21], Hq=5, dtype="bf16")
    out, lse = _mla(case)
    kv = W.to_float32(case.k_cache, "bf16").astype(np.float64)
    k = kv[:, :, None, :]
    v = np.ascontiguousarray(kv[:, :, None, :DL])
    q = W.to_float32(case.q, "bf16").astype(np.float64)
    o2, l2 = oracle.paged_attention(q, k, v, case.block_tables, case.context_lens,
                                    scale=case.scale, q_dtype="f64", kv_dtype="f64")
    np.testing.assert_allclose(out, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, l2, rtol=0, atol=1e-12)


def test_mla_matches_torch_sdpa():
    import torch
    case = _case(9, [3, 70], Hq=4, dtype="bf16")
    out, lse = _mla(case)
    kv = W.to_float32(case.k_cache, "bf16").astype(np.float64)
    q = torch.from_numpy(W.to_float32(case.q, "bf16").astype(np.float64))
    P = case.page_size
    for b in range(case.batch):
        j = np.arange(int(case.context_lens[b]))
        rec = torch.from_numpy(kv[case.block_tables[b, j // P], j % P])   # [n, DL + DR]
        k = rec.unsqueeze(0).expand(case.num_q_heads, -1, -1).contiguous()
        v = rec[:, :DL].unsqueeze(0).expand(case.num_q_heads, -1, -1).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(q[b].unsqueeze(1), k, v,
                                                               scale=case.scale)
        np.testing.assert_allclose(out[b], ref[:, 0].numpy(), rtol=0, atol=1e-12)


def test_fp8_latent_matches_gqa_oracle_with_aliased_value_and_scales():
    """An fp8 latent with one dequantization scale: MLA == the GQA oracle on the
    same stored bytes with K = the record, V = its first DL columns and
    k_scale = v_scale = the latent scale (whose fp8 handling is pinned on its
    own)."""
    case = _case(12, [5, 50, 21], Hq=5, dtype="bf16", kv_dtype="e4m3")
    assert case.kv_dtype == "e4m3" and case.k_scale != 1.0
    out, lse = _mla(case)
    k = case.k_cache[:, :, None, :]
    v = np.ascontiguousarray(case.k_cache[:, :, None, :DL])
    o2, l2 = oracle.paged_attention(case.q, k, v, case.block_tables, case.context_lens,
                                    scale=case.scale, q_dtype="bf16", kv_dtype="e4m3",
                                    k_scale=case.k_scale, v_scale=case.k_scale)
    np.testing.assert_allclose(out, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, l2, rtol=0, atol=1e-12)


def test_fp8_latent_matches_torch_sdpa_on_decoded_values():
    import torch
    case = _case(13, [3, 70], Hq=4, dtype="bf16", kv_dtype="e4m3")
    out, lse = _mla(case)
    kv = torch.from_numpy(case.k_cache).view(torch.float8_e4m3fn).double().numpy() * case.k_scale
    q = torch.from_numpy(W.to_float32(case.q, "bf16").astype(np.float64))
    P = case.page_size
    for b in range(case.batch):
        j = np.arange(int(case.context_lens[b]))
        rec = torch.from_numpy(kv[case.block_tables[b, j // P], j % P])
        k = rec.unsqueeze(0).expand(case.num_q_heads, -1, -1).contiguous()
        v = rec[:, :DL].unsqueeze(0).expand(case.num_q_heads, -1, -1).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(q[b].unsqueeze(1), k, v,
                                                               scale=case.scale)
        np.testing.assert_allclose(out[b], ref[:, 0].numpy(), rtol=0, atol=1e-12)
