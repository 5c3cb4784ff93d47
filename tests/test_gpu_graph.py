"""Capture in a HIP graph.  A call makes no allocation, memset or host
synchronisation of its own (buffers come from the caller, the per-call
planning runs on the device), so the prefill, the KCP scan and the decode step
can be recorded once and replayed.  Each replay is checked bit for bit against
the eager call, with eager work and synchronisations between the replays."""
import pytest
import torch

import kda_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import gated_delta_rule_75_amd as m
    m.lib()
    return m


def _capture(fn):
    """fn() once on a side stream (first-call set-up outside the capture), then
    recorded into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replays(g, reset, outs, refs, noise):
    for r in range(4):
        reset()
        noise.mul_(1.0001).add_(1.0)      # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, refs):
            assert torch.equal(o, e), f"replay {r} differs from the eager call"


def test_prefill_varlen_in_a_graph(kda):
    inp = kda_inputs.make_workload(2, H=4, lmin=50, lmax=300, s0_std=0.02)
    x = [t.cuda() for t in (inp.q, inp.k, inp.v, inp.g, inp.beta)]
    z, s0, cu = inp.z.cuda(), inp.S0.cuda(), inp.cu_seqlens.cuda()
    y_e, s_e = kda.chunk_fwd(*x, cu_seqlens=cu, z=z, initial_state=s0)
    y, fs = torch.empty_like(y_e), torch.empty_like(s_e)
    T, H, d = inp.q.shape
    dt = kda.KDA_BF16 if inp.q.dtype == torch.bfloat16 else kda.KDA_F32
    ws = torch.empty(kda.chunk_fwd_workspace_size(dt, H, d, d, 64, inp.num_seqs, T),
                     dtype=torch.uint8, device="cuda")
    g = _capture(lambda: kda.chunk_fwd(*x, cu_seqlens=cu, z=z, initial_state=s0, y=y,
                                       final_state=fs, workspace=ws))
    noise = torch.zeros(1 << 20, device="cuda")

    def reset():
        y.zero_()
        fs.zero_()
    _replays(g, reset, (y, fs), (y_e, s_e), noise)


def test_kcp_scan_in_a_graph(kda):
    T, nseg = 3000, 8
    inp = kda_inputs.make_workload(3, "segment", lens=[T], H=2, dk=128, dv=128, dtype="bf16",
                                   s0_std=0.05, gated=True)
    x = [t.cuda() for t in (inp.q, inp.k, inp.v, inp.g, inp.beta)]
    z, s0 = inp.z.cuda(), inp.S0.cuda()
    y_e, s_e = kda.kcp_scan(*x, nseg, z=z, initial_state=s0)
    y, fs = torch.empty_like(y_e), torch.empty_like(s_e)
    ws = torch.empty(kda.kcp_workspace_size(kda.KDA_BF16, 2, 128, 128, 64, T, nseg),
                     dtype=torch.uint8, device="cuda")
    g = _capture(lambda: kda.kcp_scan(*x, nseg, z=z, initial_state=s0, y=y, final_state=fs,
                                      workspace=ws))
    noise = torch.zeros(1 << 20, device="cuda")

    def reset():
        y.zero_()
        fs.zero_()
    _replays(g, reset, (y, fs), (y_e, s_e), noise)


def test_decode_step_in_a_graph(kda):
    dec = kda_inputs.make_decode(N=32, H=8, dk=128, dv=128, dtype="bf16", gated=True, s0_std=0.02,
                                 pool=1, seed=21)
    x = [getattr(dec, n)[0].cuda() for n in ("q", "k", "v", "g", "beta", "z")]
    s_e = dec.S0.clone().cuda()
    y_e = kda.decode_step(*x[:5], s_e, z=x[5])
    state = dec.S0.clone().cuda()
    y = torch.empty_like(y_e)
    s0 = dec.S0.cuda()
    g = _capture(lambda: kda.decode_step(*x[:5], state, z=x[5], y=y))
    noise = torch.zeros(1 << 20, device="cuda")

    def reset():
        state.copy_(s0)
        y.zero_()
    _replays(g, reset, (y, state), (y_e, s_e), noise)
