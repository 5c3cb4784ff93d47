"""The blocked algorithm of the HIP prefill, modelled in fp64 numpy, equals the
sequential oracle (CPU only).  Covers chunk 16 and 64, ragged tails, an
initial state, the gate, and the long-memory stress draws."""
import numpy as np
import pytest

import kda_inputs
from tests.chunk_model import chunk_forward


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("stress", [None, "chunk"])
def test_chunk_model_equals_sequential_oracle(oracle_mod, C, stress):
    gs, bs = kda_inputs.STRESS[stress]
    inp = kda_inputs.make_prefill([150, 64, 7], 2, 32, 16, "f32", True, 0.3, 21, gs, bs)
    y, st = oracle_mod.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens,
                                  z=inp.z, S_init=inp.S0, scale=0.5)
    cu = inp.cu_seqlens.tolist()
    for n in range(inp.num_seqs):
        for h in range(inp.H):
            sl = slice(cu[n], cu[n + 1])
            ym, Sm = chunk_forward(inp.q[sl, h], inp.k[sl, h], inp.v[sl, h], inp.g[sl, h],
                                   inp.beta[sl, h], inp.z[sl, h], inp.S0[n, h], C=C, scale=0.5)
            np.testing.assert_allclose(ym, y[sl, h], rtol=0, atol=1e-11)
            np.testing.assert_allclose(Sm, st[n * inp.H + h], rtol=0, atol=1e-11)


def test_chunk_model_at_the_decay_bound(oracle_mod):
    """g = g_min everywhere: the largest in-tile factor is e^{16*5} = e^80."""
    inp = kda_inputs.make_prefill([128], 1, 16, 8, "f32", False, 0.0, 3)
    inp.g.fill_(kda_inputs.G_MIN)
    y, st = oracle_mod.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens)
    ym, Sm = chunk_forward(inp.q[:, 0], inp.k[:, 0], inp.v[:, 0], inp.g[:, 0], inp.beta[:, 0], C=64)
    np.testing.assert_allclose(ym, y[:, 0], rtol=0, atol=1e-11)
    np.testing.assert_allclose(Sm, st[0], rtol=0, atol=1e-11)


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("stress", [None, "chunk"])
def test_two_pass_model_equals_sequential_oracle(oracle_mod, C, stress):
    from tests.chunk_model import chunk_prep, state_scan
    gs, bs = kda_inputs.STRESS[stress]
    inp = kda_inputs.make_prefill([150, 64, 7], 2, 32, 16, "f32", True, 0.3, 22, gs, bs)
    y, st = oracle_mod.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens,
                                  z=inp.z, S_init=inp.S0, scale=0.5)
    cu = inp.cu_seqlens.tolist()
    for n in range(inp.num_seqs):
        for h in range(inp.H):
            sl = slice(cu[n], cu[n + 1])
            prep = chunk_prep(inp.q[sl, h], inp.k[sl, h], inp.v[sl, h], inp.g[sl, h],
                              inp.beta[sl, h], C=C, scale=0.5)
            ym, Sm = state_scan(prep, 16, inp.z[sl, h], inp.S0[n, h])
            np.testing.assert_allclose(ym, y[sl, h], rtol=0, atol=1e-11)
            np.testing.assert_allclose(Sm, st[n * inp.H + h], rtol=0, atol=1e-11)


def test_two_pass_model_at_the_decay_bound(oracle_mod):
    from tests.chunk_model import chunk_prep, state_scan
    inp = kda_inputs.make_prefill([128], 1, 16, 8, "f32", False, 0.0, 3)
    inp.g.fill_(kda_inputs.G_MIN)
    y, st = oracle_mod.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens)
    prep = chunk_prep(inp.q[:, 0], inp.k[:, 0], inp.v[:, 0], inp.g[:, 0], inp.beta[:, 0], C=64)
    ym, Sm = state_scan(prep, 8)
    np.testing.assert_allclose(ym, y[:, 0], rtol=0, atol=1e-11)
    np.testing.assert_allclose(Sm, st[0], rtol=0, atol=1e-11)
