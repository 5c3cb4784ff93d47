"""Parity at the full workload sizes, in the launch configuration the benchmark
times, on outputs the oracle can compute one chain at a time.

- K3-layer prefill (H=96, T=8192): every output and final state of 4 heads
  (plus the chunk-scale long-memory variant).
- The same layer through the fused-input entry point (raw q, k, gate
  pre-activations): every output and final state of 3 heads.
- Varlen prefill (16 sequences, lengths in [512, 8192], H=96): 3 sampled
  (sequence, head) chains, including the longest and the shortest sequence.
- KCP scan (T=2^20, H=4, 256 segments, segment-scale long-memory draw so the
  carried state matters): head 0's final state and the outputs of 3 segments.
- Decode (128 requests x 96 heads, 1000 steps): every state and output after
  step 1, 32 sampled chains after step 10, 8 after step 1000.
- Speculative replay (128 requests x 96 heads, 4 draft tokens, acceptance
  uniform in [0, 4]): every draft output of the verify call and every state
  after the commit call.
"""
import sys

import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from oracle import rel_l2

pytestmark = pytest.mark.gpu
BF16_TOL = 2e-2


def log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def kda():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import gated_delta_rule_75_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("stress", [None, "chunk"])
def test_k3_layer_prefill_full_size(kda, stress):
    inp = kda_inputs.make_workload(1, stress)
    dev = torch.device("cuda")
    y, fs = kda.chunk_fwd(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.g.to(dev),
                          inp.beta.to(dev), z=inp.z.to(dev), chunk=64)
    torch.cuda.synchronize()
    heads = [0, 31, 64, 95]
    yo, so = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, z=inp.z,
                               chains=[(0, h) for h in heads])
    ey = rel_l2(y.cpu()[:, heads].double().numpy(), yo[:, heads])
    es = rel_l2(fs.cpu()[0, heads].double().numpy(), so)
    log(f"[fullsize] k3 layer prefill {stress}: y={ey:.3e} state={es:.3e}")
    assert ey <= BF16_TOL and es <= BF16_TOL


def test_k3_layer_prefill_fused_full_size(kda):
    """kda_chunk_fwd_fused at the K3 layer shape from raw inputs (the draws of
    the plain workload before normalisation and squashing)."""
    w = kda_inputs.WORKLOADS[1]
    raw = kda_inputs.make_raw_prefill(w["lens"], w["H"], w["dk"], w["dv"], w["dtype"], True, 0.0,
                                      kda_inputs.workload_seed(1))
    dev = torch.device("cuda")
    y, fs = kda.chunk_fwd_fused(raw.q.to(dev), raw.k.to(dev), raw.v.to(dev), raw.a.to(dev),
                                raw.b.to(dev), z=raw.z.to(dev), chunk=64)
    torch.cuda.synchronize()
    heads = [0, 50, 95]
    pick = lambda t: t[:, heads].contiguous()
    yo, so = oracle.recurrence_fused(pick(raw.q), pick(raw.k), pick(raw.v), pick(raw.a),
                                     pick(raw.b), raw.cu_seqlens, z=pick(raw.z))
    ey = rel_l2(y.cpu()[:, heads].double().numpy(), yo)
    es = rel_l2(fs.cpu()[0, heads].double().numpy(), so)
    log(f"[fullsize] k3 layer fused prefill: y={ey:.3e} state={es:.3e}")
    assert ey <= BF16_TOL and es <= BF16_TOL


def _chain(inp, n, h):
    """Host copy of one (sequence, head) chain of device inputs."""
    cu = inp.cu_seqlens.tolist()
    sl = slice(cu[n], cu[n + 1])
    pick = lambda t: None if t is None else t[sl, h:h + 1].contiguous().cpu()
    s0 = None if inp.S0 is None else inp.S0[n:n + 1, h:h + 1].cpu()
    return pick(inp.q), pick(inp.k), pick(inp.v), pick(inp.z), pick(inp.g), pick(inp.beta), s0, sl


def test_varlen_prefill_full_size(kda):
    lens = kda_inputs.varlen_lengths()
    dev = torch.device("cuda")
    inp = kda_inputs.draw_on_device(lens, 96, 128, 128, True, 0.02, kda_inputs.workload_seed(2), dev)
    y, fs = kda.chunk_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta,
                          cu_seqlens=inp.cu_seqlens.to(dev), z=inp.z, initial_state=inp.S0,
                          chunk=64)
    torch.cuda.synchronize()
    order = sorted(range(len(lens)), key=lambda i: lens[i])
    for n, h in [(order[-1], 0), (order[0], 95), (order[len(order) // 2], 47)]:
        q, k, v, z, g, b, s0, sl = _chain(inp, n, h)
        yo, so = oracle.recurrence(q, k, v, g, b, [0, lens[n]], z=z, S_init=s0)
        ey = rel_l2(y[sl, h:h + 1].cpu().double().numpy(), yo)
        es = rel_l2(fs[n, h].cpu().double().numpy(), so[0])
        log(f"[fullsize] varlen seq {n} (len {lens[n]}) head {h}: y={ey:.3e} state={es:.3e}")
        assert ey <= BF16_TOL and es <= BF16_TOL


def test_kcp_full_size(kda):
    w = kda_inputs.WORKLOADS[3]
    T, H, S = w["lens"][0], w["H"], w["segments"]
    dev = torch.device("cuda")
    gs, bs = kda_inputs.STRESS["segment"]
    inp = kda_inputs.draw_on_device([T], H, 128, 128, False, 0.0,
                                    kda_inputs.workload_seed(3, "segment"), dev, gs, bs)
    y, fs = kda.kcp_scan(inp.q, inp.k, inp.v, inp.g, inp.beta, S, chunk=64)
    torch.cuda.synchronize()
    h = 0
    host = lambda t: t[:, h:h + 1].contiguous().cpu()
    q, k, v, g, b = host(inp.q), host(inp.k), host(inp.v), host(inp.g), host(inp.beta)
    seg = T // S
    bounds = [i * seg for i in range(S)] + [T]
    out = oracle.kcp(q, k, v, g, b, bounds, want_y=False)
    es = rel_l2(fs[0, h].cpu().double().numpy(), out["final"][0])
    log(f"[fullsize] kcp head {h}: final state rel_l2={es:.3e}")
    assert es <= BF16_TOL
    for s in (1, S // 2, S - 1):
        sl = slice(bounds[s], bounds[s + 1])
        yo, _ = oracle.recurrence(q[sl], k[sl], v[sl], g[sl], b[sl], [0, seg],
                                  chain_states=out["starts"][s])
        ey = rel_l2(y[sl, h:h + 1].cpu().double().numpy(), yo)
        log(f"[fullsize] kcp head {h} segment {s}: y rel_l2={ey:.3e}")
        assert ey <= BF16_TOL
    # the long-memory draw really carries state across segments
    assert np.abs(out["starts"][S - 1]).max() > 1e-3


def test_decode_full_size(kda):
    dec = kda_inputs.make_decode_workload()
    dev = torch.device("cuda")
    P = dec.q.shape[0]
    pool = [{n: getattr(dec, n)[p].to(dev) for n in ("q", "k", "v", "z", "g", "beta")}
            for p in range(P)]
    state = dec.S0.to(dev)
    y = None
    snaps = {}
    for s in range(1000):
        x = pool[s % P]
        y = kda.decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], state, z=x["z"], y=y)
        if s + 1 in (1, 10):
            torch.cuda.synchronize()
            snaps[s + 1] = (y.cpu(), state.cpu())
    torch.cuda.synchronize()
    snaps[1000] = (y.cpu(), state.cpu())
    # step 1: every chain
    yo, _, so = oracle.decode_steps(dec, 1)
    ey = rel_l2(snaps[1][0].double().numpy(), yo)
    es = rel_l2(snaps[1][1].double().numpy().reshape(so.shape), so)
    log(f"[fullsize] decode step 1 (all chains): y={ey:.3e} state={es:.3e}")
    assert ey <= BF16_TOL and es <= BF16_TOL
    rng = np.random.default_rng(0)
    for steps, nchains in ((10, 32), (1000, 8)):
        chains = [(int(rng.integers(dec.N)), int(rng.integers(dec.H))) for _ in range(nchains)]
        idx = [t % P for t in range(steps)]
        ys, yr, ss, sr = [], [], [], []
        for n, h in chains:
            seq = lambda t: t[idx, n, h:h + 1].contiguous()
            y_o, s_o = oracle.recurrence(seq(dec.q), seq(dec.k), seq(dec.v), seq(dec.g),
                                         seq(dec.beta), [0, steps], z=seq(dec.z),
                                         S_init=dec.S0[n:n + 1, h:h + 1])
            ys.append(snaps[steps][0][n, h].double().numpy())
            yr.append(y_o[-1, 0])
            ss.append(snaps[steps][1][n, h].double().numpy())
            sr.append(s_o[0])
        ey, es = rel_l2(np.stack(ys), np.stack(yr)), rel_l2(np.stack(ss), np.stack(sr))
        log(f"[fullsize] decode step {steps} ({nchains} chains): y={ey:.3e} state={es:.3e}")
        assert ey <= BF16_TOL and es <= BF16_TOL


def test_replay_full_size(kda):
    rep = kda_inputs.make_replay(128, 4, 96, 128, 128, "bf16", True, 0.02, 95)
    dev = torch.device("cuda")
    x = {n: getattr(rep, n).to(dev) for n in ("q", "k", "v", "z", "g", "beta")}
    state = rep.S0.to(dev)
    y = kda.decode_replay(x["q"], x["k"], x["v"], x["g"], x["beta"], state, z=x["z"])
    kda.decode_replay(x["q"], x["k"], x["v"], x["g"], x["beta"], state,
                      accepted=rep.accepted.to(dev), z=x["z"], want_y=False)
    torch.cuda.synchronize()
    yo, so = oracle.replay(rep)
    ey = rel_l2(y.cpu().double().numpy(), yo)
    es = rel_l2(state.cpu().double().numpy(), so)
    log(f"[fullsize] replay 128x96, 4 drafts: y={ey:.3e} committed={es:.3e}")
    assert ey <= BF16_TOL and es <= BF16_TOL
    untouched = (rep.accepted == 0).nonzero().flatten()
    assert torch.equal(state[untouched].cpu(), rep.S0[untouched])
