"""kda_chunk_fwd_noalloc: the prefill without a workspace argument, its chunk
products in the library's per-GPU scratch.  Its results must equal those of
kda_chunk_fwd (same arithmetic, in time slabs that fit the scratch) bit for
bit, on two calls in a row, the second with a smaller input, and match the
fp64 oracle; a shape whose smallest workspace exceeds the scratch is refused
before any launch.
"""
import pytest
import torch

import kda_inputs
import oracle
from tests import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import gated_delta_rule_75_amd as m
    m.lib()
    return m


def _c(t):
    return None if t is None else t.cuda()


def _both(kda, inp, chunk):
    cu = inp.cu_seqlens.cuda() if inp.num_seqs > 1 else None
    args = (_c(inp.q), _c(inp.k), _c(inp.v), _c(inp.g), _c(inp.beta))
    kw = dict(cu_seqlens=cu, z=_c(inp.z), initial_state=_c(inp.S0), chunk=chunk)
    y0, s0 = kda.chunk_fwd(*args, **kw)
    y1, s1 = kda.chunk_fwd_noalloc(*args, **kw)
    torch.cuda.synchronize()
    return (y0.cpu(), s0.cpu()), (y1.cpu(), s1.cpu())


def test_noalloc_matches_chunk_fwd_twice_second_smaller(kda):
    scratch = kda.lib().kda_noalloc_scratch_bytes()
    assert scratch == 64 << 20
    # 1: the K3 layer shape at 2048 tokens, more chunk products than the scratch holds
    big = kda_inputs.make_workload(1, "chunk", lens=[2048])
    need = kda.chunk_fwd_workspace_size(kda.KDA_BF16, 96, 128, 128, 64, 1, 2048)
    assert need > scratch            # so the call really runs in several slabs
    ref, got = _both(kda, big, 64)
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])
    heads = [0, 41, 95]
    yo, so = oracle.recurrence(big.q, big.k, big.v, big.g, big.beta, big.cu_seqlens, z=big.z,
                               chains=[(0, h) for h in heads])
    parity.check("noalloc K3 layer 2048 tokens", "bf16", y=(got[0][:, heads], yo[:, heads]),
                 state=(got[1][0, heads], so))
    # 2: a smaller, packed input right after, in the same scratch
    small = kda_inputs.make_prefill([300, 17, 0, 129], 4, 128, 128, "bf16", True, 0.05, 700, 8.0, 4.0)
    ref, got = _both(kda, small, 32)
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])
    yo, so = oracle.recurrence(small.q, small.k, small.v, small.g, small.beta, small.cu_seqlens,
                               z=small.z, S_init=small.S0)
    parity.check("noalloc varlen after the big call", "bf16", y=(got[0], yo), state=(got[1], so))


def test_noalloc_fp32_and_refusal(kda):
    inp = kda_inputs.make_workload(0, "chunk", lens=[333], H=3, s0_std=0.1)
    ref, got = _both(kda, inp, 16)
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])
    yo, so = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, z=inp.z,
                               S_init=inp.S0)
    parity.check("noalloc fp32 d64", "f32", y=(got[0], yo), state=(got[1], so))
    # 16 sequences x 96 heads carry 100 MB of states: more than the scratch, refused
    L = kda.lib()
    st = L.kda_chunk_fwd_noalloc(kda.KDA_BF16, 96, 128, 128, 64, 1.0, 16, 16 * 512, None, None,
                                 None, None, None, None, None, None, None, None, None)
    assert st == 3       # KDA_ERR_WORKSPACE_TOO_SMALL, before any pointer is looked at
