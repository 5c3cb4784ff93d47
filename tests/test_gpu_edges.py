"""Parity at the edges of the method's input ranges, through every entry point
that carries a state: kda_chunk_fwd, kda_kcp_scan and kda_decode_step.

- g at the lower bound g_min = -5 over whole 16-token tiles (page "Exercices",
  Niveau 2 Q8: a 16-token tile then accumulates a log-decay of -80, and its
  factor e^80 must still fit bf16; the prefill kernels split every exponent at
  16-token sub-tile references for exactly this).  Also mixed with g = 0 on
  half of the channels, so that the same tiles carry both e^80 factors and a
  state that is not forgotten, and slightly past the bound (-5.4) where the
  header states the kernels stay finite.
- g = 0 (alpha = 1: no forgetting at all).
- The delta rule's overwrite (page "Exercices", Niveau 2 Q7: erase, then
  write): alpha = beta = 1 with unit keys drawn from a small orthonormal set,
  each written several times with different values; a query equal to a key
  returns the value of that key's latest write.  Compared with the oracle, and
  in fp32 with that closed form too.

Each case runs at d = 128 in bf16 and fp32 with chunks 16, 32 and 64.
"""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from tests import parity

pytestmark = pytest.mark.gpu

T_EDGE = 300      # several 64-token chunks and a ragged tail
H_EDGE = 2


@pytest.fixture(scope="module")
def kda():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import gated_delta_rule_75_amd as m
    m.lib()
    return m


def edge_inputs(case, dtype, seed=500, T=T_EDGE, H=H_EDGE, d=128, gated=True, s0_std=0.05):
    """Inputs of one edge case; q, k, v, z, beta drawn by the usual recipe, then
    g (and for the overwrite case k, q, beta) replaced by the case's values."""
    inp = kda_inputs.make_prefill([T], H, d, d, dtype, gated, s0_std, seed)
    if case == "gmin":
        inp.g.fill_(kda_inputs.G_MIN)
    elif case == "gmin_half":
        inp.g.zero_()
        inp.g[..., 0::2] = kda_inputs.G_MIN
    elif case == "g_past_min":
        inp.g.fill_(-5.4)
        inp.g[..., 1::3] = 0.0
    elif case == "g0":
        inp.g.zero_()
    elif case == "overwrite":
        rng = np.random.default_rng(seed)
        basis, _ = np.linalg.qr(rng.standard_normal((d, d)))
        nkeys = 8                                     # few keys, each written ~T/8 times
        keys = torch.tensor(basis[:, :nkeys].T.copy(), dtype=torch.float32)
        kid = torch.tensor(rng.integers(0, nkeys, (T, H)))
        qid = torch.tensor(rng.integers(0, nkeys, (T, H)))
        td = inp.k.dtype
        inp.k = keys[kid].to(td).contiguous()
        inp.q = keys[qid].to(td).contiguous()
        inp.g.zero_()
        inp.beta.fill_(1.0)
        inp.S0 = None
        inp.kid, inp.qid = kid, qid
    else:
        raise ValueError(case)
    return inp


def _c(t):
    return None if t is None else t.cuda()


def oracle_of(inp):
    return oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, z=inp.z,
                             S_init=inp.S0)


CASES = ["gmin", "gmin_half", "g_past_min", "g0", "overwrite"]


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", CASES)
def test_chunk_fwd_edges(kda, case, dtype, chunk):
    inp = edge_inputs(case, dtype)
    y, fs = kda.chunk_fwd(_c(inp.q), _c(inp.k), _c(inp.v), _c(inp.g), _c(inp.beta), z=_c(inp.z),
                          initial_state=_c(inp.S0), chunk=chunk)
    torch.cuda.synchronize()
    yo, so = oracle_of(inp)
    parity.check(f"chunk_fwd {case} {dtype} c{chunk}", dtype, y=(y, yo), state=(fs, so))
    if case == "overwrite" and dtype == "f32":
        _check_retrieval(inp, y.cpu())


def _check_retrieval(inp, y):
    """Closed form of the overwrite case (fp32 keys exactly orthonormal up to
    rounding): o_t = sigma(z_t) * (value of q_t's latest write at or before t),
    or 0 when that key has not been written yet."""
    T, H = inp.kid.shape
    want = torch.zeros(T, H, inp.dv, dtype=torch.float64)
    last = {}
    for t in range(T):
        for h in range(H):
            last[(h, int(inp.kid[t, h]))] = inp.v[t, h].double()
            key = (h, int(inp.qid[t, h]))
            if key in last:
                want[t, h] = last[key]
    if inp.z is not None:
        want = want * torch.sigmoid(inp.z.double())
    err = (y.double() - want).abs().max().item()
    parity.log(f"[parity] overwrite closed form: max abs err {err:.3e}")
    assert err <= 1e-4


@pytest.mark.parametrize("dtype,chunk", [("bf16", 64), ("f32", 16), ("bf16", 32), ("f32", 64)])
@pytest.mark.parametrize("case", CASES)
def test_kcp_scan_edges(kda, case, dtype, chunk):
    inp = edge_inputs(case, dtype, seed=510, T=1000)
    y, fs = kda.kcp_scan(_c(inp.q), _c(inp.k), _c(inp.v), _c(inp.g), _c(inp.beta), 8, z=_c(inp.z),
                         initial_state=_c(inp.S0), chunk=chunk)
    torch.cuda.synchronize()
    yo, so = oracle_of(inp)
    parity.check(f"kcp_scan {case} {dtype} c{chunk}", dtype, y=(y, yo), state=(fs, so))
    if case == "overwrite" and dtype == "f32":
        _check_retrieval(inp, y.cpu())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", CASES)
def test_decode_step_edges(kda, case, dtype):
    """The same token stream, one token at a time, for 3 requests side by side
    (request n takes head n % H_EDGE of the prefill inputs)."""
    T = 40
    inp = edge_inputs(case, dtype, seed=520, T=T)
    N = 3
    pick = [n % H_EDGE for n in range(N)]
    sel = lambda t: None if t is None else t[:, pick].contiguous()   # [T, N, .] as N requests
    q, k, v, z, g, beta = (sel(x) for x in (inp.q, inp.k, inp.v, inp.z, inp.g, inp.beta))
    S0 = inp.S0[0, pick].contiguous() if inp.S0 is not None else torch.zeros(N, 128, 128)
    state = S0.clone().cuda().reshape(N, 1, 128, 128)
    ys = []
    for t in range(T):
        one = lambda x: None if x is None else x[t].reshape(N, 1, *x.shape[2:]).cuda()
        ys.append(kda.decode_step(one(q), one(k), one(v), one(g), one(beta), state, z=one(z)).cpu())
    torch.cuda.synchronize()
    y = torch.stack(ys)[:, :, 0]                     # [T, N, dv]
    # the oracle runs the N requests as N heads of one sequence
    yo, so = oracle.recurrence(q, k, v, g, beta, inp.cu_seqlens, z=z, S_init=S0[None])
    parity.check(f"decode {case} {dtype}", dtype, y=(y, yo), state=(state.reshape(1, N, 128, 128), so))
