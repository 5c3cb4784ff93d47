"""Parity of the fused-input entry points (kda_chunk_fwd_fused,
kda_decode_step_fused) with the fp64 oracle fed by the same raw inputs.

The oracle forms unit q, k, g = -5 sigmoid(a) and beta = sigmoid(b) in fp64
from the raw values and runs the sequential recurrence; the kernels do the
same in fp32.  Tolerances as for the plain entry points: rel-L2 <= 1e-4
(fp32 inputs) and <= 2e-2 (bf16 inputs) on y and on the final states.
"""
import sys

import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from oracle import rel_l2
from tests import parity
from tests.parity import TOL

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def kda():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import gated_delta_rule_75_amd as m
    m.lib()
    return m


def _c(t):
    return None if t is None else t.cuda()


def run_fused(kda, raw, chunk, scale=1.0):
    cu = raw.cu_seqlens.cuda() if raw.cu_seqlens.numel() > 2 else None
    y, fs = kda.chunk_fwd_fused(_c(raw.q), _c(raw.k), _c(raw.v), _c(raw.a), _c(raw.b),
                                cu_seqlens=cu, z=_c(raw.z), initial_state=_c(raw.S0),
                                chunk=chunk, scale=scale)
    torch.cuda.synchronize()
    return y.cpu(), fs.cpu()


def check(name, y, fs, yo, so, tol):
    parity.check(name, "f32" if tol <= TOL["f32"] else "bf16", y=(y, yo), state=(fs, so))


@pytest.mark.parametrize("dtype,d,chunk,stress", [
    ("bf16", 128, 64, None), ("bf16", 128, 16, "chunk"), ("bf16", 64, 64, "chunk"),
    ("f32", 64, 16, None), ("f32", 128, 64, "chunk"), ("f32", 64, 64, None), ("bf16", 128, 32, None),
    ("f32", 128, 32, "chunk"),
])
def test_fused_prefill_matches_oracle(kda, dtype, d, chunk, stress):
    gs, bs = kda_inputs.STRESS[stress]
    raw = kda_inputs.make_raw_prefill([555], 3, d, d, dtype, True, 0.05, 71, gs, bs)
    y, fs = run_fused(kda, raw, chunk, scale=0.9)
    yo, so = oracle.recurrence_fused(raw.q, raw.k, raw.v, raw.a, raw.b, raw.cu_seqlens, z=raw.z,
                                     S_init=raw.S0, scale=0.9)
    check(f"fused {dtype} d{d} c{chunk} {stress}", y, fs, yo, so, TOL[dtype])


def test_fused_prefill_varlen_ragged_and_empty(kda):
    raw = kda_inputs.make_raw_prefill([300, 1, 0, 77, 129, 64], 2, 128, 128, "bf16", True, 0.02,
                                      72, *kda_inputs.STRESS["chunk"])
    y, fs = run_fused(kda, raw, 64)
    yo, so = oracle.recurrence_fused(raw.q, raw.k, raw.v, raw.a, raw.b, raw.cu_seqlens, z=raw.z,
                                     S_init=raw.S0)
    check("fused varlen ragged", y, fs, yo, so, TOL["bf16"])


def test_fused_prefill_zero_vectors(kda):
    """Degenerate inputs: zero keys (nothing erased or written, pure decay) and
    zero queries (zero output) stay finite and match the oracle."""
    raw = kda_inputs.make_raw_prefill([200], 2, 64, 64, "f32", False, 0.3, 73,
                                      *kda_inputs.STRESS["chunk"])
    raw.k[50:90] = 0
    raw.q[10:20] = 0
    y, fs = run_fused(kda, raw, 16)
    yo, so = oracle.recurrence_fused(raw.q, raw.k, raw.v, raw.a, raw.b, raw.cu_seqlens,
                                     S_init=raw.S0)
    check("fused zero vectors", y, fs, yo, so, TOL["f32"])
    assert float(y[10:20].abs().max()) == 0.0


def test_fused_prefill_ignores_the_scale_of_q_and_k(kda):
    raw = kda_inputs.make_raw_prefill([130], 2, 128, 128, "f32", True, 0.05, 74)
    y1, s1 = run_fused(kda, raw, 64)
    raw.q *= 4
    raw.k *= 0.5
    y2, s2 = run_fused(kda, raw, 64)
    assert rel_l2(y2.double().numpy(), y1.double().numpy()) <= 1e-5
    assert rel_l2(s2.double().numpy(), s1.double().numpy()) <= 1e-5


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("f32", 128), ("bf16", 64)])
def test_fused_decode_matches_oracle(kda, dtype, d):
    steps = 5
    raw = kda_inputs.make_raw_decode(4, 3, d, d, dtype, True, 0.02, steps, 75)
    N, H = 4, 3
    state = raw.S0.clone().cuda()
    st = None
    cu = np.arange(N + 1, dtype=np.int32)
    for s in range(steps):
        y = kda.decode_step_fused(raw.q[s].cuda(), raw.k[s].cuda(), raw.v[s].cuda(),
                                  raw.a[s].cuda(), raw.b[s].cuda(), state, z=raw.z[s].cuda(),
                                  scale=1.1)
        yo, st = oracle.recurrence_fused(raw.q[s], raw.k[s], raw.v[s], raw.a[s], raw.b[s], cu,
                                         z=raw.z[s], scale=1.1,
                                         chain_states=(raw.S0.double().numpy().reshape(N * H, d, d)
                                                       if st is None else st))
    torch.cuda.synchronize()
    ey = rel_l2(y.cpu().double().numpy(), yo)
    es = rel_l2(state.cpu().double().numpy().reshape(st.shape), st)
    log(f"[parity] fused decode {dtype} d={d}: y={ey:.3e} state={es:.3e}")
    assert ey <= TOL[dtype] and es <= TOL[dtype]


def test_fused_decode_equals_fused_prefill_token_by_token(kda):
    """Decode steps on one request equal a prefill over the same tokens."""
    raw = kda_inputs.make_raw_prefill([24], 2, 64, 64, "f32", True, 0.1, 76)
    y_p, s_p = run_fused(kda, raw, 16)
    state = raw.S0.clone().cuda()
    ys = []
    for t in range(24):
        sl = slice(t, t + 1)
        ys.append(kda.decode_step_fused(raw.q[sl].cuda(), raw.k[sl].cuda(), raw.v[sl].cuda(),
                                        raw.a[sl].cuda(), raw.b[sl].cuda(), state,
                                        z=raw.z[sl].cuda()).cpu())
    torch.cuda.synchronize()
    assert rel_l2(torch.cat(ys).double().numpy(), y_p.double().numpy()) <= 1e-4
    assert rel_l2(state.cpu().double().numpy(), s_p.double().numpy()) <= 1e-4
