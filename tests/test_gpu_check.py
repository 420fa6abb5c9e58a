"""GPU: the on-device precondition check (pda_check_inputs) counts exactly the
lengths, table entries and append positions that break the documented
preconditions, and nothing in valid inputs.  The checker only compares the
values it reads; none of them addresses memory."""
import numpy as np
import pytest
import torch

from decode_attention_paged_02_amd import pda
from decode_attention_paged_02_amd import workloads as W
from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


@pytest.mark.parametrize("make", [W.ragged_fp8, W.gqa_batch64, W.tiny_gqa])
def test_valid_workloads_have_no_violations(make):
    case = make()
    say("check", case.name)
    # poisoned tables hold -1 past the used pages: not followed, not counted
    got = pda.check_inputs(_dev(case.block_tables), _dev(case.context_lens),
                           page_size=case.page_size, num_pages=case.num_pages)
    assert got == (0, 0, 0)


def test_counts_each_kind_of_violation():
    P, max_pages, num_pages = 16, 4, 10
    lens = np.array([0, 1, 16, 17, 64, 65, -3, 40], np.int32)
    table = np.full((8, max_pages), 2 ** 30, np.int32)      # never followed unless used
    table[1, 0] = 9                                          # valid
    table[2, 0] = 10                                         # == num_pages: bad
    table[3, :2] = [0, -1]                                   # second page bad
    table[4, :] = [1, 2, 3, 4]                               # all valid (64 tokens)
    table[5, :] = [1, 2, 3, 4]                               # length 65 > 64: bad length
    table[7, :3] = [5, 6, 7]                                 # valid (40 tokens)
    say("check violations")
    got = pda.check_inputs(_dev(table), _dev(lens), page_size=P, num_pages=num_pages)
    assert got == (2, 2, 0)                                  # lens 65, -3; entries 10, -1
    # append positions: sequence 7 appends 3 tokens at 40..42 (page 2, valid);
    # sequence 1 at 63 + 3 > 64 (bad position); sequence 0 at 16..18 needs
    # table[0, 1] = 2^30 (bad entry); -1 skips
    pos = np.array([16, 63, -1, -1, -1, -1, -1, 40], np.int32)
    got = pda.check_inputs(_dev(table), _dev(lens), page_size=P, num_pages=num_pages,
                           positions=_dev(pos), s_new=3)
    assert got == (2, 3, 1)


def test_empty_batch():
    z = torch.zeros((0, 4), dtype=torch.int32, device="cuda")
    assert pda.check_inputs(z, torch.zeros(0, dtype=torch.int32, device="cuda"),
                            page_size=16, num_pages=1) == (0, 0, 0)
