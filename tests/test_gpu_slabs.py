"""Bounded workspaces: the prefill and the KCP scan given less than their full
workspace take the chunks in time slabs, carrying each chain's state between
slabs.  The arithmetic per chunk is the same, so the results must equal the
one-pass call's bit for bit; they are also checked against the fp64 oracle.
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


def _limits(kda, dt, H, d, chunk, N, T):
    """Workspace limits giving slabs of 1, 3 and 7 chunks."""
    least = kda.chunk_fwd_workspace_min(dt, H, d, d, chunk, N, T)
    block = (kda.chunk_fwd_workspace_size(dt, H, d, d, chunk, N, 2 * 64 * chunk) -
             kda.chunk_fwd_workspace_size(dt, H, d, d, chunk, N, 64 * chunk)) // 64
    assert least < kda.chunk_fwd_workspace_size(dt, H, d, d, chunk, N, T)
    return [least, least + 2 * block + 300, least + 6 * block + 300]


def _prefill(kda, inp, chunk, limit=None, fused=False):
    cu = inp.cu_seqlens.cuda() if inp.num_seqs > 1 else None
    y, fs = kda.chunk_fwd(_c(inp.q), _c(inp.k), _c(inp.v), _c(inp.g), _c(inp.beta), cu_seqlens=cu,
                          z=_c(inp.z), initial_state=_c(inp.S0), chunk=chunk,
                          max_workspace_bytes=limit)
    torch.cuda.synchronize()
    return y.cpu(), fs.cpu()


@pytest.mark.parametrize("dtype,d,chunk,lens", [
    ("bf16", 128, 64, [1000]),
    ("f32", 64, 16, [333]),
    ("bf16", 128, 32, [300, 17, 0, 129, 64, 1]),      # packed, ragged and empty sequences
    ("f32", 128, 64, [70, 200, 5]),
])
def test_prefill_slabs_equal_one_pass(kda, dtype, d, chunk, lens):
    inp = kda_inputs.make_prefill(lens, 3, d, d, dtype, True, 0.05, 600 + chunk, 8.0, 4.0)
    y1, s1 = _prefill(kda, inp, chunk)
    yo, so = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, z=inp.z,
                               S_init=inp.S0)
    dt = kda.KDA_BF16 if dtype == "bf16" else kda.KDA_F32
    for limit in _limits(kda, dt, 3, d, chunk, len(lens), inp.T):
        y, s = _prefill(kda, inp, chunk, limit)
        parity.check(f"prefill slabs {dtype} d{d} c{chunk} limit {limit}", dtype, y=(y, yo),
                     state=(s, so))
        assert torch.equal(y, y1) and torch.equal(s, s1), f"limit {limit}: differs from one pass"


def test_prefill_slabs_at_the_k3_layer(kda):
    """The K3 layer (H=96, T=8192) in a workspace of 256 MiB instead of 894 MB."""
    inp = kda_inputs.make_workload(1, "chunk")
    d = {n: getattr(inp, n).cuda() for n in ("q", "k", "v", "g", "beta", "z")}
    y1, s1 = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], z=d["z"])
    y2, s2 = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], z=d["z"],
                           max_workspace_bytes=256 << 20)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(s1, s2)
    heads = [0, 95]
    yo, so = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, z=inp.z,
                               chains=[(0, h) for h in heads])
    parity.check("k3 layer in 256 MiB (2 heads)", "bf16", y=(y2.cpu()[:, heads], yo[:, heads]),
                 state=(s2.cpu()[0, heads], so))


def test_checkpoints_with_slabs(kda):
    lens = [300, 40, 256, 129]
    inp = kda_inputs.make_prefill(lens, 2, 128, 128, "bf16", True, 0.05, 610, 8.0, 4.0)
    args = (inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.g.cuda(), inp.beta.cuda(), 64)
    kw = dict(cu_seqlens=inp.cu_seqlens.cuda(), z=inp.z.cuda(), initial_state=inp.S0.cuda(), chunk=32)
    y1, f1, c1, o1 = kda.chunk_fwd_checkpointed(*args, **kw)
    least = kda.chunk_fwd_workspace_min(kda.KDA_BF16, 2, 128, 128, 32, len(lens), inp.T)
    y2, f2, c2, o2 = kda.chunk_fwd_checkpointed(*args, **kw, max_workspace_bytes=least)
    torch.cuda.synchronize()
    n = int(o1[-1])
    assert torch.equal(o1, o2) and n > 0
    assert torch.equal(c1[:n], c2[:n]) and torch.equal(y1, y2) and torch.equal(f1, f2)
    co, _ = oracle.checkpoints(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, 64, S_init=inp.S0)
    parity.check("checkpoints in slabs of one chunk", "bf16", checkpoints=(c2[:n], co))


def test_fused_prefill_with_slabs(kda):
    raw = kda_inputs.make_raw_prefill([500, 77], 2, 128, 128, "bf16", True, 0.05, 620, 8.0, 4.0)
    args = (raw.q.cuda(), raw.k.cuda(), raw.v.cuda(), raw.a.cuda(), raw.b.cuda())
    kw = dict(cu_seqlens=raw.cu_seqlens.cuda(), z=raw.z.cuda(), initial_state=raw.S0.cuda())
    y1, s1 = kda.chunk_fwd_fused(*args, **kw)
    least = kda.chunk_fwd_workspace_min(kda.KDA_BF16, 2, 128, 128, 64, 2, raw.q.shape[0])
    y2, s2 = kda.chunk_fwd_fused(*args, **kw, max_workspace_bytes=least + 5000)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(s1, s2)


@pytest.mark.parametrize("dtype,d,chunk,T,nseg", [
    ("bf16", 128, 64, 4096, 8), ("f32", 64, 16, 1001, 7), ("bf16", 128, 32, 2000, 16),
    ("f32", 128, 64, 3000, 5), ("bf16", 64, 64, 2500, 3),
])
def test_kcp_slabs_equal_one_pass(kda, dtype, d, chunk, T, nseg):
    inp = kda_inputs.make_workload(3, "segment", lens=[T], H=2, dk=d, dv=d, dtype=dtype,
                                   s0_std=0.05, gated=True)
    x = [_c(t) for t in (inp.q, inp.k, inp.v, inp.g, inp.beta)]
    y1, s1 = kda.kcp_scan(*x, nseg, z=_c(inp.z), initial_state=_c(inp.S0), chunk=chunk)
    dt = kda.KDA_BF16 if dtype == "bf16" else kda.KDA_F32
    least = kda.kcp_workspace_min(dt, 2, d, d, chunk, T, nseg)
    full = kda.kcp_workspace_size(dt, 2, d, d, chunk, T, nseg)
    yo, so = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, z=inp.z,
                               S_init=inp.S0)
    for limit in (least, least + (full - least) // 3, full - 1):
        y2, s2 = kda.kcp_scan(*x, nseg, z=_c(inp.z), initial_state=_c(inp.S0), chunk=chunk,
                              max_workspace_bytes=limit)
        torch.cuda.synchronize()
        parity.check(f"kcp slabs {dtype} d{d} c{chunk} limit {limit}", dtype,
                     y=(y2.cpu(), yo), state=(s2.cpu(), so))
        assert torch.equal(y1, y2) and torch.equal(s1, s2), f"limit {limit}: differs from one pass"
