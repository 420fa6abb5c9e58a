"""GPU parity over a seeded sweep of configurations: the GQA and MLA entry
points with random shapes, dtypes, page sizes, query-token counts, causal
flags, split counts, thresholds and schedules, each against the fp64 oracle.
The cases are drawn once from a fixed seed (the same cases on every run)."""
import math
import random

import numpy as np
import pytest

from decode_attention_paged_02_amd import pda
from decode_attention_paged_02_amd import workloads as W
from gpu_util import check, need_gpu, oracle_ref, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _gqa_cases(n, seed=2024):
    r = random.Random(seed)
    out = []
    for i in range(n):
        q_dtype, kv_dtype = r.choice([("f16", "f16"), ("bf16", "bf16"), ("f32", "f32"),
                                      ("f16", "e4m3"), ("bf16", "e4m3")])
        d = r.choice([64, 128] + ([] if q_dtype == "f32" else [256]))
        Hkv = r.choice([1, 2, 4, 8])
        G = r.choice([1, 2, 3, 4, 6, 8, 16])
        q_len = 1 if q_dtype == "f32" else r.choice([1, 1, 1, 2, 3, 4])
        B = r.randint(1, 6)
        lens = [r.choice([0, 1, r.randint(2, 64), r.randint(65, 3000)]) for _ in range(B)]
        out.append(dict(idx=i, q_dtype=q_dtype, kv_dtype=kv_dtype, d=d, Hkv=Hkv, G=G,
                        P=r.choice([16, 32, 64]), q_len=q_len, causal=r.random() < 0.8,
                        lens=lens, splits=r.choice([0, 1, 2, 5, 16]),
                        thr=r.choice([0, 0, 256]), schedule=r.choice([0, 0, 1]),
                        variant=r.choice([pda.PDA_GQA_DEFAULT, pda.PDA_GQA_MFMA,
                                          pda.PDA_GQA_VALU])))
    return out


def _supported(c):
    if c["variant"] == pda.PDA_GQA_MFMA and c["q_dtype"] == "f32":
        return False
    if c["variant"] == pda.PDA_GQA_VALU and c["q_len"] > 1:
        return False
    return True


@pytest.mark.parametrize("c", [c for c in _gqa_cases(40) if _supported(c)],
                         ids=lambda c: "gqa%d" % c["idx"])
def test_gqa_sweep(c):
    case = W.make_gqa(batch=len(c["lens"]), num_q_heads=c["Hkv"] * c["G"],
                      num_kv_heads=c["Hkv"], head_dim=c["d"], page_size=c["P"],
                      context_lens=c["lens"], q_dtype=c["q_dtype"], kv_dtype=c["kv_dtype"],
                      seed=500 + c["idx"], extra_pages=2, q_len=c["q_len"], causal=c["causal"])
    say("sweep", c)
    ref_o, ref_l = oracle_ref(case)
    out, lse = pda.run_case(case, num_splits=c["splits"], split_min_tokens=c["thr"],
                            schedule=c["schedule"], variant=c["variant"])
    check(case, out, lse, ref_o, ref_l, label=str(c))


def _mla_cases(n, seed=77):
    r = random.Random(seed)
    out = []
    for i in range(n):
        d_latent = r.choice([512, 512, 256])
        q_len = r.choice([1, 1, 2, 3])
        variant = r.choice([pda.PDA_MLA_DEFAULT, pda.PDA_MLA_MFMA, pda.PDA_MLA_VALU])
        if d_latent != 512 or q_len > 1:
            variant = pda.PDA_MLA_MFMA
        B = r.randint(1, 4)
        out.append(dict(idx=i, d_latent=d_latent, q_len=q_len, variant=variant,
                        Hq=r.choice([1, 4, 16, 32, 48]), P=r.choice([64, 128]),
                        kv=r.choice(["bf16", "e4m3"]), causal=r.random() < 0.8,
                        lens=[r.choice([0, 1, r.randint(2, 200), r.randint(201, 4000)])
                              for _ in range(B)],
                        splits=r.choice([0, 1, 3, 8]), thr=r.choice([0, 500]),
                        schedule=r.choice([0, 1])))
    return out


@pytest.mark.parametrize("c", _mla_cases(16), ids=lambda c: "mla%d" % c["idx"])
def test_mla_sweep(c):
    case = W.make_mla(batch=len(c["lens"]), num_q_heads=c["Hq"], d_latent=c["d_latent"],
                      d_rope=64, page_size=c["P"], context_lens=c["lens"], dtype="bf16",
                      seed=700 + c["idx"], std=0.5, scale=1.0 / math.sqrt(192.0),
                      extra_pages=2, q_len=c["q_len"], causal=c["causal"], kv_dtype=c["kv"])
    say("sweep", c)
    ref_o, ref_l = oracle_ref(case)
    out, lse = pda.run_case(case, num_splits=c["splits"], split_min_tokens=c["thr"],
                            schedule=c["schedule"], variant=c["variant"])
    check(case, out, lse, ref_o, ref_l, label=str(c))
