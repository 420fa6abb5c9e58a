"""Pins of the parity checker itself (tests/gpu_util.py errors / check), on the
CPU: outputs with the kinds of mistakes a kernel can make are rejected, and
the one allowance the checker makes (a value that rounded to the other
neighbour of the exact result) is accepted only as far as it is justified.

The "GPU" outputs here are built on the host from the oracle's result or from
a plain numpy attention with one step deliberately changed."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_paged_02_amd import workloads as W
from gpu_util import check, errors, oracle_ref

TORCH = {"bf16": torch.bfloat16, "f16": torch.float16}


def _case(dt):
    # short contexts: outputs of magnitude up to ~3, where 16-bit rounding
    # and relative faults are largest in absolute terms
    lens = [int(x) for x in np.random.default_rng(1).integers(1, 40, 48)]
    return W.make_gqa(batch=48, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=16,
                      context_lens=lens, q_dtype=dt, kv_dtype=dt, seed=77)


def _attention(case, round_p):
    """softmax(scale q K^T) V per (b, h) in fp64 from the stored values, with
    the unnormalized weights p passed through round_p before the weighted
    sum (the denominator keeps the exact weights)."""
    q = oracle.decode(case.q, case.q_dtype)
    K = oracle.decode(case.k_cache, case.kv_dtype)
    V = oracle.decode(case.v_cache, case.kv_dtype)
    B, Hq, _ = q.shape
    P, G = case.page_size, Hq // case.num_kv_heads
    out = np.zeros((B, Hq, V.shape[-1]))
    for b in range(B):
        n = int(case.context_lens[b])
        pages = [int(case.block_tables[b][j // P]) for j in range(n)]
        for h in range(Hq):
            kv = h // G
            Kb = np.stack([K[pages[j], j % P, kv] for j in range(n)])
            Vb = np.stack([V[pages[j], j % P, kv] for j in range(n)])
            s = case.scale * (Kb @ q[b, h])
            p = np.exp(s - s.max())
            out[b, h] = round_p(p) @ Vb / p.sum()
    return out


def _as(x, dt):
    return torch.from_numpy(np.ascontiguousarray(x)).to(TORCH[dt])


@pytest.fixture(scope="module", params=["bf16", "f16"])
def ref(request):
    dt = request.param
    case = _case(dt)
    o, l = oracle_ref(case)
    return dt, case, o, l


def test_correctly_rounded_output_passes(ref):
    dt, case, o, l = ref
    assert errors(_as(o, dt), o) == (0.0, 0.0)
    check(case, _as(o, dt), torch.from_numpy(l).float(), o, l)
    # the numpy attention used to plant the faults below agrees with the oracle
    assert np.abs(_attention(case, lambda p: p) - o).max() < 1e-12


def test_relative_bias_of_2_pow_minus_9_is_rejected(ref):
    dt, case, o, l = ref
    with pytest.raises(AssertionError):
        check(case, _as(o * (1 + 2.0 ** -9), dt), None, o, l)


def test_probabilities_rounded_to_bf16_without_low_part_are_rejected(ref):
    """p rounded to bfloat16 with no p_lo correction (2^-9 relative error per
    weight) fails the bar; p rounded to binary16 (what the f16 kernels do) is
    within it."""
    dt, case, o, l = ref
    bad = _attention(case, lambda p: torch.from_numpy(p).to(torch.bfloat16).double().numpy())
    with pytest.raises(AssertionError):
        check(case, _as(bad, dt), None, o, l)
    ok = _attention(case, lambda p: torch.from_numpy(p).to(torch.float16).double().numpy())
    check(case, _as(ok, dt), None, o, l)


def test_one_ulp_shift_at_magnitudes_of_one_and_more_is_rejected(ref):
    dt, case, o, l = ref
    t = _as(o, dt)
    bits = t.view(torch.int16).clone()
    big = t.double().abs() >= 1
    assert big.any()
    bits[big] += 1          # one unit in the last place, away from zero
    with pytest.raises(AssertionError):
        check(case, bits.view(TORCH[dt]), None, o, l)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_a_rounding_tie_flip_is_accepted_and_nothing_more(dt):
    """Exact values on or next to the midpoint of two neighbours: the other
    neighbour counts as the distance to the midpoint (0 or 1e-9); a value two
    steps away, or the other neighbour of a value far from the midpoint,
    counts in full."""
    one = torch.tensor([1.0], dtype=TORCH[dt])
    up = (one.view(torch.int16) + 1).view(TORCH[dt])            # next value above 1
    mid = 0.5 * (1.0 + float(up))
    exact = np.array([mid, mid + 1e-9, mid - 1e-9])
    lo_hi = [one, up, one]                                       # the other neighbour each time
    for x, other in zip(exact, lo_hi):
        mx, _ = errors(other, np.array([x]))
        assert mx <= 1.01e-9
    step = float(up) - 1.0
    far = np.array([1.0 + 0.1 * step])                           # rounds to 1 with margin
    assert errors(up, far)[0] == pytest.approx(0.4 * step, rel=1e-6)
    two_up = (one.view(torch.int16) + 2).view(TORCH[dt])
    assert errors(two_up, np.array([mid]))[0] >= step
