"""GPU: the C-ABI example (HIP runtime + libpda, no Python in the call path)
runs a paged decode step with head-major pages and two splits; its inputs and
results, written to a file, match the fp64 oracle.  The example's code runs
in this process, loaded as a shared library (the same source builds the
standalone program)."""
import ctypes
import os

import numpy as np
import pytest

import oracle
from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "decode_attention_paged_02_amd", "examples", "libc_abi_decode.so")


def test_c_abi_example_matches_oracle(tmp_path):
    need_gpu()
    if not os.path.exists(LIB):
        pytest.fail("example library missing: run __graft_entry__.build()")
    out_file = str(tmp_path / "step.bin")
    say("c abi example")
    lib = ctypes.CDLL(LIB)
    lib.pda_example_decode_step.argtypes = [ctypes.c_char_p]
    lib.pda_example_decode_step.restype = ctypes.c_int
    assert lib.pda_example_decode_step(out_file.encode()) == 0
    raw = open(out_file, "rb").read()
    B, Hq, Hkv, D, P, max_pages, num_pages, splits = np.frombuffer(raw[:32], np.int32)
    off = 32

    def take(n, dt):
        nonlocal off
        a = np.frombuffer(raw, dt, n, off)
        off += a.nbytes
        return a

    table = take(B * max_pages, np.int32).reshape(B, max_pages)
    lens = take(B, np.int32)
    q = take(B * Hq * D, np.float16).reshape(B, Hq, D)
    k = take(num_pages * Hkv * P * D, np.float16).reshape(num_pages, Hkv, P, D)
    v = take(num_pages * Hkv * P * D, np.float16).reshape(num_pages, Hkv, P, D)
    out = take(B * Hq * D, np.float16).reshape(B, Hq, D).astype(np.float64)
    lse = take(B * Hq, np.float32).reshape(B, Hq).astype(np.float64)
    assert off == len(raw) and splits == 2
    ref_o, ref_l = oracle.paged_attention(q, k, v, table, lens, scale=1.0 / np.sqrt(D),
                                          q_dtype="f16", kv_dtype="f16", kv_layout=1)
    want = ref_o.astype(np.float16).astype(np.float64)   # the oracle rounded to the output type
    err = np.abs(out - want)
    assert err.max() <= 2e-3 and np.sqrt((err ** 2).mean()) <= 1e-4, err.max()
    assert np.abs(lse - ref_l).max() <= 1e-3
