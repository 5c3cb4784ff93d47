"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: an
explicit-matrix brute force, closed forms of special cases, invariants of the
recurrence, a hand-worked example, and the KCP identities whose error class
the pages print.  None needs a GPU.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import kda_inputs
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny(lens, H=2, dk=8, dv=6, dtype="f32", gated=True, s0_std=0.3, seed=7, gs=0.0, bs=0.0):
    return kda_inputs.make_prefill(lens, H, dk, dv, dtype, gated, s0_std, seed, gs, bs)


def _run(oracle_mod, inp, scale=1.0, **kw):
    return oracle_mod.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, z=inp.z,
                                 S_init=inp.S0, scale=scale, **kw)


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gated", [False, True])
def test_oracle_matches_explicit_matrix_products(oracle_mod, dtype, gated):
    inp = _tiny([5, 17, 1, 30], H=3, dk=8, dv=5, dtype=dtype, gated=gated, gs=-1.0)
    scale = 0.75
    y, st = _run(oracle_mod, inp, scale=scale)
    cu = inp.cu_seqlens.tolist()
    for n in range(inp.num_seqs):
        for h in range(inp.H):
            sl = slice(cu[n], cu[n + 1])
            yb, Sb = brute.sequence(inp.q[sl, h], inp.k[sl, h], inp.v[sl, h], inp.g[sl, h],
                                    inp.beta[sl, h], None if inp.z is None else inp.z[sl, h],
                                    inp.S0[n, h], scale)
            np.testing.assert_allclose(y[sl, h], yb, rtol=0, atol=1e-13)
            np.testing.assert_allclose(st[n * inp.H + h], Sb, rtol=0, atol=1e-13)


def test_oracle_hand_worked_example(oracle_mod):
    fx = json.load(open(os.path.join(GOLDEN, "hand_worked_2x2.json")))
    i = fx["inputs"]
    f = lambda a: torch.tensor(a, dtype=torch.float32)
    T = 3
    q = f(i["q"]).reshape(T, 1, 2)
    k = f(i["k"]).reshape(T, 1, 2)
    v = f(i["v"]).reshape(T, 1, 2)
    g = torch.log(torch.tensor(i["alpha"], dtype=torch.float64)).float().reshape(T, 1, 2)
    beta = f(i["beta"]).reshape(T, 1)
    cu = [0, T]
    y, st = oracle_mod.recurrence(q, k, v, g, beta, cu)
    tol = fx["tolerance"]
    np.testing.assert_allclose(y[:, 0], np.array(fx["expected"]["o"]), rtol=0, atol=tol)
    np.testing.assert_allclose(st[0], np.array(fx["expected"]["S_final"]), rtol=0, atol=tol)
    z = torch.zeros(T, 1, 2)
    z[:2] = 50.0  # sigmoid(50) == 1 in fp64 to ~2e-22
    z[2] = f(i["z_last"])
    yg, _ = oracle_mod.recurrence(q, k, v, g, beta, cu, z=z)
    np.testing.assert_allclose(yg[2, 0], np.array(fx["expected"]["y_last_gated"]), rtol=0, atol=tol)
    np.testing.assert_allclose(yg[:2, 0], np.array(fx["expected"]["o"][:2]), rtol=0, atol=tol)


# ---------------------------------------------------------------- closed forms
def test_oracle_beta_zero_is_pure_channel_decay(oracle_mod):
    """beta = 0: S_t = Diag(exp(G_t)) S_0 with G_t the running sum of g."""
    inp = _tiny([40], H=2, dk=8, dv=6, s0_std=1.0, gated=False)
    inp.beta.zero_()
    y, st = _run(oracle_mod, inp)
    G = torch.cumsum(inp.g.double(), 0)                       # [T, H, dk]
    S0 = inp.S0[0].double()                                   # [H, dk, dv]
    for h in range(inp.H):
        St = torch.exp(G[:, h, :, None]) * S0[h][None]        # [T, dk, dv]
        o = torch.einsum("tcv,tc->tv", St, inp.q[:, h].double())
        np.testing.assert_allclose(y[:, h], o.numpy(), rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(st[h], St[-1].numpy(), rtol=1e-12, atol=1e-15)


def test_oracle_exact_retrieval_with_orthonormal_keys(oracle_mod):
    """alpha = 1, beta = 1, orthonormal keys, S_0 = 0: querying with key j returns v_j."""
    dk, dv, T = 16, 5, 12
    rng = np.random.default_rng(3)
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = torch.tensor(Qm[:, :T].T.copy(), dtype=torch.float32)   # T orthonormal rows
    v = torch.tensor(rng.standard_normal((T, dv)), dtype=torch.float32)
    pick = [rng.integers(0, t + 1) for t in range(T)]               # any j <= t
    q = keys[pick]
    g = torch.zeros(T, 1, dk)
    beta = torch.ones(T, 1)
    y, st = oracle_mod.recurrence(q[:, None], keys[:, None], v[:, None], g, beta, [0, T])
    kd = keys.double().numpy()
    expect = v.double().numpy()[pick]
    np.testing.assert_allclose(y[:, 0], expect, rtol=0, atol=2e-6)  # keys are fp32-rounded
    # the final state holds every pair: S^T k_j = v_j
    np.testing.assert_allclose(kd @ st[0], v.double().numpy(), rtol=0, atol=2e-6)


def test_oracle_overwrite_same_key(oracle_mod):
    """beta = alpha = 1 and the same unit key twice: the later value replaces the earlier."""
    dk, dv = 8, 4
    k1 = torch.zeros(dk)
    k1[3] = 1.0
    k = torch.stack([k1, k1])[:, None]
    v = torch.tensor([[1.0, 2.0, 3.0, 4.0], [-5.0, 6.0, 0.5, 0.25]])[:, None]
    y, st = oracle_mod.recurrence(k, k, v, torch.zeros(2, 1, dk), torch.ones(2, 1), [0, 2])
    np.testing.assert_array_equal(y[1, 0], v[1, 0].double().numpy())
    np.testing.assert_array_equal(st[0], np.outer(k1.double().numpy(), v[1, 0].double().numpy()))


def test_oracle_scalar_case_is_an_ema(oracle_mod):
    """dk = dv = 1, k = +-1: S_t = (1 - beta_t) alpha_t S_{t-1} + beta_t k_t v_t."""
    T = 50
    gen = torch.Generator().manual_seed(11)
    k = (torch.randint(0, 2, (T, 1, 1), generator=gen) * 2 - 1).float()
    v = torch.randn(T, 1, 1, generator=gen)
    q = torch.randn(T, 1, 1, generator=gen)
    beta = torch.rand(T, 1, generator=gen)
    g = -5.0 * torch.rand(T, 1, 1, generator=gen)
    S0 = torch.tensor([[[[0.7]]]])
    y, st = oracle_mod.recurrence(q, k, v, g, beta, [0, T], S_init=S0)
    S = float(S0[0, 0, 0, 0])
    for t in range(T):
        b = float(beta[t, 0])
        S = (1 - b) * math.exp(float(g[t, 0, 0])) * S + b * float(k[t, 0, 0]) * float(v[t, 0, 0])
        assert abs(y[t, 0, 0] - S * float(q[t, 0, 0])) <= 1e-14 * (1 + abs(S))
    assert abs(st[0, 0, 0] - S) <= 1e-14


def test_oracle_zero_values_never_expand_the_state(oracle_mod):
    """v = 0 with unit keys, beta in [0,1], alpha <= 1: ||S_t||_2 <= ||S_{t-1}||_2."""
    inp = _tiny([60], H=1, dk=8, dv=8, s0_std=1.0, gated=False)
    inp.v.zero_()
    state = inp.S0[0, 0].double().numpy()[None]
    prev = np.linalg.norm(state[0], 2)
    for t in range(60):
        sl = slice(t, t + 1)
        _, state = oracle_mod.recurrence(inp.q[sl], inp.k[sl], inp.v[sl], inp.g[sl],
                                         inp.beta[sl], [0, 1], chain_states=state, want_y=False)
        cur = np.linalg.norm(state[0], 2)
        assert cur <= prev * (1 + 1e-12)
        prev = cur
    assert prev < np.linalg.norm(inp.S0[0, 0].double().numpy(), 2)


def test_oracle_gate_limits(oracle_mod):
    inp = _tiny([20], H=2, dk=8, dv=6, gated=True)
    y_plain, _ = oracle_mod.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens,
                                       S_init=inp.S0)
    y_half, _ = oracle_mod.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens,
                                      z=torch.zeros_like(inp.z), S_init=inp.S0)
    y_one, _ = oracle_mod.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens,
                                     z=torch.full_like(inp.z, 60.0), S_init=inp.S0)
    np.testing.assert_allclose(y_half, y_plain / 2, rtol=1e-15, atol=0)
    np.testing.assert_allclose(y_one, y_plain, rtol=1e-15, atol=0)


def test_oracle_scale_is_linear_in_output_only(oracle_mod):
    inp = _tiny([25], H=1, gated=True)
    y1, s1 = _run(oracle_mod, inp, scale=1.0)
    y2, s2 = _run(oracle_mod, inp, scale=0.125)
    np.testing.assert_allclose(y2, 0.125 * y1, rtol=1e-15)
    np.testing.assert_array_equal(s1, s2)


# ---------------------------------------------------------------- sequences
def test_oracle_resume_equals_single_call(oracle_mod):
    """Splitting a sequence and passing the state on gives the same result."""
    inp = _tiny([70], H=2, gated=True)
    y, st = _run(oracle_mod, inp)
    a = slice(0, 33)
    b = slice(33, 70)
    ya, sa = oracle_mod.recurrence(inp.q[a], inp.k[a], inp.v[a], inp.g[a], inp.beta[a], [0, 33],
                                   z=inp.z[a], S_init=inp.S0)
    yb, sb = oracle_mod.recurrence(inp.q[b], inp.k[b], inp.v[b], inp.g[b], inp.beta[b], [0, 37],
                                   z=inp.z[b], chain_states=sa)
    np.testing.assert_array_equal(np.concatenate([ya, yb]), y)
    np.testing.assert_array_equal(sb, st)


def test_oracle_decode_steps_equal_recurrence(oracle_mod):
    """Decode applied T times = the recurrence over those T tokens (same fp64 loop)."""
    dec = kda_inputs.make_decode(N=3, H=2, dk=8, dv=6, dtype="bf16", gated=True, s0_std=0.02,
                                 pool=4, seed=5)
    steps = 7
    y, snaps, fin = oracle_mod.decode_steps(dec, steps, record=(1, steps))
    P = dec.q.shape[0]
    idx = [s % P for s in range(steps)]
    for n in range(dec.N):
        seq = lambda t: t[idx, n]
        y_seq, s_seq = oracle_mod.recurrence(seq(dec.q), seq(dec.k), seq(dec.v), seq(dec.g),
                                             seq(dec.beta), [0, steps], z=seq(dec.z),
                                             S_init=dec.S0[n:n + 1])
        for h in range(dec.H):
            np.testing.assert_array_equal(fin[n * dec.H + h], s_seq[h])
            np.testing.assert_array_equal(y[n, h], y_seq[-1, h])


def test_oracle_sampled_chains_equal_full_run(oracle_mod):
    inp = _tiny([9, 21, 14], H=3, gated=True)
    y, st = _run(oracle_mod, inp)
    chains = [(2, 1), (0, 2), (1, 0)]
    ys, ss = _run(oracle_mod, inp, chains=chains)
    cu = inp.cu_seqlens.tolist()
    for i, (n, h) in enumerate(chains):
        np.testing.assert_array_equal(ss[i], st[n * inp.H + h])
        np.testing.assert_array_equal(ys[cu[n]:cu[n + 1], h], y[cu[n]:cu[n + 1], h])


# ---------------------------------------------------------------- KCP
def _err_scale(*arrs):
    return max(float(np.abs(a).max()) for a in arrs)


def test_oracle_kcp_pair_matches_explicit_products(oracle_mod):
    inp = _tiny([48], H=2, dk=8, dv=6, gated=False, s0_std=0.0)
    out = oracle_mod.kcp(inp.q, inp.k, inp.v, inp.g, inp.beta, [0, 20, 48], want_pairs=True)
    for s, (a, b) in enumerate([(0, 20), (20, 48)]):
        for h in range(inp.H):
            M, L = brute.pair(inp.k[a:b, h], inp.v[a:b, h], inp.g[a:b, h], inp.beta[a:b, h])
            np.testing.assert_allclose(out["M"][s, h], M, rtol=0, atol=1e-14)
            np.testing.assert_allclose(out["Sloc"][s, h], L, rtol=0, atol=1e-14)


def test_oracle_kcp_composition_identity(oracle_mod):
    """(M2, S2) o (M1, S1) equals the pair of the concatenated segment.

    Page 'Reproduire Kimi K3' prints 6.94e-18 for this check (sizes unstated);
    the bound here is machine precision relative to the magnitudes involved.
    """
    fx = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))
    dk = 16
    inp = _tiny([64], H=1, dk=dk, dv=12, gated=False, s0_std=0.0, gs=6.0, bs=2.0)
    out = oracle_mod.kcp(inp.q, inp.k, inp.v, inp.g, inp.beta, [0, 25, 64], want_pairs=True)
    whole = oracle_mod.kcp(inp.q, inp.k, inp.v, inp.g, inp.beta, [0, 64], want_pairs=True)
    Mc, Sc = oracle_mod.compose(out["M"][1, 0], out["Sloc"][1, 0], out["M"][0, 0],
                                out["Sloc"][0, 0])
    err = max(np.abs(Mc - whole["M"][0, 0]).max(), np.abs(Sc - whole["Sloc"][0, 0]).max())
    bound = 8 * dk * np.finfo(np.float64).eps * _err_scale(Mc, Sc)
    assert err <= bound, (err, bound)
    # the pages' figure belongs to the same machine-precision class
    assert fx["kcp_composition_max_error"]["value"] < 1e-15
    # a composition in the wrong order is far off (the identity is not symmetric)
    Mw, Sw = oracle_mod.compose(out["M"][0, 0], out["Sloc"][0, 0], out["M"][1, 0],
                                out["Sloc"][1, 0])
    assert np.abs(Sw - whole["Sloc"][0, 0]).max() > 1e3 * bound


def test_oracle_kcp_four_segment_scan_equals_sequential(oracle_mod):
    """Prefix scan of 4 segments (page 'Exercices', Niveau 3 Q22; 1.39e-17 printed)."""
    dk = 16
    inp = _tiny([200], H=2, dk=dk, dv=12, gated=True, s0_std=0.05, gs=6.0, bs=2.0)
    y, st = _run(oracle_mod, inp)
    S0 = inp.S0[0]
    out = oracle_mod.kcp(inp.q, inp.k, inp.v, inp.g, inp.beta, [0, 50, 100, 150, 200], z=inp.z,
                         S0=S0)
    err_s = np.abs(out["final"] - st).max()
    err_y = np.nanmax(np.abs(out["y"] - y))
    bound = 64 * dk * np.finfo(np.float64).eps * max(_err_scale(st), _err_scale(y))
    assert err_s <= bound and err_y <= bound, (err_s, err_y, bound)
    # entering states equal the sequential state at each boundary
    for s, t in enumerate([50, 100, 150]):
        _, sb = oracle_mod.recurrence(inp.q[:t], inp.k[:t], inp.v[:t], inp.g[:t], inp.beta[:t],
                                      [0, t], S_init=inp.S0, want_y=False)
        np.testing.assert_allclose(out["starts"][s + 1], sb, rtol=0, atol=bound)


def test_oracle_kcp_needs_the_transition(oracle_mod):
    """Page 'Exercices', Niveau 3 Q21: summing local states alone is wrong."""
    inp = _tiny([96], H=1, dk=8, dv=6, gated=False, s0_std=0.0, gs=6.0, bs=2.0)
    out = oracle_mod.kcp(inp.q, inp.k, inp.v, inp.g, inp.beta, [0, 32, 64, 96], want_pairs=True)
    naive = out["Sloc"].sum(axis=0)
    assert np.abs(naive - out["final"]).max() > 1e-3


# ---------------------------------------------------------------- page figures
def test_page_figures_are_consistent():
    fx = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))
    gm = fx["g_min"]
    bf16_max = float(torch.finfo(torch.bfloat16).max)
    e = math.exp(-gm["tile_tokens"] * gm["value"])
    assert abs(e - gm["exp_bound"]) / gm["exp_bound"] < 0.01
    assert e < bf16_max and abs(bf16_max - gm["bf16_max_quoted"]) / bf16_max < 0.15
    assert math.exp(-gm["tile_tokens"] * gm["g_min_rejected"]) > bf16_max
    # bf16 holds e^80 as a finite number and overflows at e^160
    assert torch.isfinite(torch.tensor(e).to(torch.bfloat16))
    assert not torch.isfinite(torch.tensor(math.exp(160.0)).to(torch.float32).to(torch.bfloat16))
    L = fx["kda_layer"]
    bytes_2b = L["kda_layers"] * L["num_heads"] * L["head_dim"] ** 2 * 2
    assert abs(bytes_2b / 1e6 - fx["state_per_request"]["value_mib_quoted"]) < 0.5


def test_generator_recipe():
    """The synthetic inputs respect the method's preconditions."""
    inp = kda_inputs.make_workload(0)
    assert inp.q.dtype == torch.float32 and inp.T == 256 and inp.H == 2 and inp.dk == 64
    nk = inp.k.double().norm(dim=-1)
    assert torch.allclose(nk, torch.ones_like(nk), atol=1e-6)
    assert float(inp.g.min()) > kda_inputs.G_MIN and float(inp.g.max()) < 0
    assert 0 < float(inp.beta.min()) and float(inp.beta.max()) < 1
    again = kda_inputs.make_workload(0)
    assert torch.equal(inp.q, again.q) and torch.equal(inp.g, again.g)
    small2 = kda_inputs.make_workload(2, H=2, lmin=3, lmax=40)
    assert small2.num_seqs == 16 and all(3 <= n <= 40 for n in small2.lengths())
    assert small2.q.dtype == torch.bfloat16 and small2.S0.shape == (16, 2, 128, 128)


# ---------------------------------------------------------------- prefix-cache checkpoints
def test_oracle_checkpoints_are_brute_force_prefix_states(oracle_mod):
    """Checkpoint j = the state after (j+1)*interval tokens, by explicit transition
    matrices on each prefix (page "Exercices", Niveau 3 Q26)."""
    from oracle import brute
    inp = kda_inputs.make_prefill([37, 20, 8], 2, 6, 5, "f32", False, 0.4, 31)
    ck, offs = oracle_mod.checkpoints(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, 8,
                                      S_init=inp.S0)
    assert offs.tolist() == [0, 4, 6, 7]
    cu = inp.cu_seqlens.tolist()
    for n in range(3):
        for j in range(offs[n + 1] - offs[n]):
            for h in range(2):
                sl = slice(cu[n], cu[n] + 8 * (j + 1))
                _, S = brute.sequence(inp.q[sl, h], inp.k[sl, h], inp.v[sl, h], inp.g[sl, h],
                                      inp.beta[sl, h], S0=inp.S0[n, h])
                np.testing.assert_allclose(ck[offs[n] + j, h], S, rtol=0, atol=1e-12)


def test_oracle_checkpoint_at_the_end_is_the_final_state(oracle_mod):
    inp = kda_inputs.make_prefill([64, 128], 2, 8, 8, "f32", True, 0.2, 32)
    ck, offs = oracle_mod.checkpoints(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, 32,
                                      S_init=inp.S0)
    _, st = oracle_mod.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens,
                                  S_init=inp.S0)
    np.testing.assert_allclose(ck[offs[1] - 1], st[0:2], rtol=0, atol=1e-13)
    np.testing.assert_allclose(ck[offs[2] - 1], st[2:4], rtol=0, atol=1e-13)


def test_oracle_resume_from_a_checkpoint(oracle_mod):
    """Running the rest of a sequence from a checkpoint reproduces the uncut run."""
    inp = kda_inputs.make_prefill([96], 1, 8, 8, "f32", True, 0.0, 33)
    ck, _ = oracle_mod.checkpoints(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, 32)
    y_full, s_full = oracle_mod.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens,
                                           z=inp.z)
    sl = slice(32, 96)
    y_rest, s_rest = oracle_mod.recurrence(inp.q[sl], inp.k[sl], inp.v[sl], inp.g[sl],
                                           inp.beta[sl], [0, 64], z=inp.z[sl],
                                           chain_states=ck[0])
    np.testing.assert_allclose(y_rest, y_full[32:], rtol=0, atol=1e-13)
    np.testing.assert_allclose(s_rest, s_full, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- speculative-decoding replay
def test_oracle_replay_matches_brute_force(oracle_mod):
    """Replay outputs and the committed state after the accepted prefix, by
    explicit transition matrices (page "Exercices", Niveau 3 Q27)."""
    from oracle import brute
    rep = kda_inputs.make_replay(3, 5, 2, 6, 4, "f32", True, 0.3, 41)
    rep.accepted[:] = torch.tensor([0, 2, 5], dtype=torch.int32)
    y, committed = oracle_mod.replay(rep, scale=0.7)
    for n in range(3):
        for h in range(2):
            yb, _ = brute.sequence(rep.q[n, :, h], rep.k[n, :, h], rep.v[n, :, h], rep.g[n, :, h],
                                   rep.beta[n, :, h], rep.z[n, :, h], S0=rep.S0[n, h], scale=0.7)
            np.testing.assert_allclose(y[n, :, h], yb, rtol=0, atol=1e-12)
            a = int(rep.accepted[n])
            _, Sb = brute.sequence(rep.q[n, :a, h], rep.k[n, :a, h], rep.v[n, :a, h],
                                   rep.g[n, :a, h], rep.beta[n, :a, h], S0=rep.S0[n, h])
            np.testing.assert_allclose(committed[n, h], Sb, rtol=0, atol=1e-12)
    # nothing accepted: the resident state is kept
    np.testing.assert_array_equal(committed[0], rep.S0[0].double().numpy())


def test_oracle_full_acceptance_equals_decode_steps(oracle_mod):
    """Accepting every draft token equals Td single-token decode steps."""
    rep = kda_inputs.make_replay(4, 3, 2, 8, 8, "f32", True, 0.1, 42)
    rep.accepted[:] = 3
    y, committed = oracle_mod.replay(rep)
    dec = kda_inputs.DecodeInputs(rep.q.transpose(0, 1).contiguous(), rep.k.transpose(0, 1).contiguous(),
                                  rep.v.transpose(0, 1).contiguous(), rep.z.transpose(0, 1).contiguous(),
                                  rep.g.transpose(0, 1).contiguous(), rep.beta.transpose(0, 1).contiguous(),
                                  rep.S0, 4, 2, 8, 8, "f32")
    y_last, _, st = oracle_mod.decode_steps(dec, 3)
    np.testing.assert_allclose(y[:, 2], y_last, rtol=0, atol=1e-13)
    np.testing.assert_allclose(committed.reshape(8, 8, 8), st, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- fused input step
def _raw_tiny(lens, H=2, dk=8, dv=5, dtype="f32", gated=True, s0_std=0.3, seed=51, gs=0.0, bs=0.0):
    return kda_inputs.make_raw_prefill(lens, H, dk, dv, dtype, gated, s0_std, seed, gs, bs)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_oracle_fused_matches_brute_force(oracle_mod, dtype):
    """Raw inputs through the fused step (norms, g = g_min sigmoid(a), beta =
    sigmoid(b)) then the recurrence, against explicit matrices fed by an
    independently written gate step (sigmoid through tanh, norm through hypot)."""
    raw = _raw_tiny([9, 1, 23], H=3, dtype=dtype, gs=-1.0)
    y, st = oracle_mod.recurrence_fused(raw.q, raw.k, raw.v, raw.a, raw.b, raw.cu_seqlens, z=raw.z,
                                        S_init=raw.S0, scale=0.8)
    cu = raw.cu_seqlens.tolist()
    for n in range(3):
        for h in range(3):
            sl = slice(cu[n], cu[n + 1])
            yb, Sb = brute.fused_sequence(raw.q[sl, h], raw.k[sl, h], raw.v[sl, h], raw.a[sl, h],
                                          raw.b[sl, h], raw.z[sl, h], raw.S0[n, h], 0.8)
            np.testing.assert_allclose(y[sl, h], yb, rtol=0, atol=1e-13)
            np.testing.assert_allclose(st[n * 3 + h], Sb, rtol=0, atol=1e-13)


def test_oracle_gates_special_values(oracle_mod):
    """sigmoid(0) = 1/2 gives g = g_min / 2 = -2.5 and beta = 1/2 exactly; the
    decay stays inside (g_min, 0) and beta inside (0, 1); a unit vector keeps its
    direction and a zero vector stays zero (no division by zero)."""
    q = torch.zeros(4, 1, 3)
    q[0, 0] = torch.tensor([3.0, 0.0, 4.0])
    q[1, 0, 1] = -2.0
    a = torch.tensor([[[0.0, 30.0, -30.0]]]).repeat(4, 1, 1)
    b = torch.tensor([[0.0], [30.0], [-30.0], [1.0]])
    qh, kh, g, beta = oracle_mod.gates(q, q, a, b)
    assert g[0, 0, 0].item() == -2.5 and beta[0, 0].item() == 0.5
    assert -5.0 < g.min().item() and g.max().item() < 0.0
    assert 0.0 < beta.min().item() and beta.max().item() < 1.0
    assert abs(g[0, 0, 1].item() + 5.0) < 1e-12 and abs(g[0, 0, 2].item()) < 1e-12
    eps = oracle_mod.NORM_EPS
    np.testing.assert_allclose(qh[0, 0].numpy(), np.array([3.0, 0.0, 4.0]) / math.sqrt(25.0 + eps),
                               rtol=1e-15)
    assert qh[1, 0, 1].item() == pytest.approx(-2.0 / math.sqrt(4.0 + eps), rel=1e-15)
    assert torch.equal(qh[2], torch.zeros(1, 3, dtype=torch.float64))
    assert torch.equal(kh, qh)


def test_oracle_gates_match_library_routines(oracle_mod):
    """Against torch's own normalize (x / max(||x||, eps)) and sigmoid: the two
    norms differ only by eps / (2 ||x||^2), below 1e-8 relative here."""
    gen = torch.Generator().manual_seed(52)
    q = torch.randn(40, 3, 16, generator=gen, dtype=torch.float64) * 3
    k = torch.randn(40, 3, 16, generator=gen, dtype=torch.float64)
    a = torch.randn(40, 3, 16, generator=gen, dtype=torch.float64) * 4
    b = torch.randn(40, 3, generator=gen, dtype=torch.float64) * 4
    qh, kh, g, beta = oracle_mod.gates(q, k, a, b)
    eps = oracle_mod.NORM_EPS
    for x, xh in ((q, qh), (k, kh)):
        ref = torch.nn.functional.normalize(x, dim=-1)
        bound = ref.abs() * (eps / (2 * (x * x).sum(-1, keepdim=True))) * 1.001 + 1e-16
        assert bool(((xh - ref).abs() <= bound).all())
        assert float(((xh - ref).abs() / bound).max()) > 0.5      # the eps term is really there
    np.testing.assert_allclose(g, -5.0 * torch.sigmoid(a), rtol=1e-14, atol=0)
    np.testing.assert_allclose(beta, torch.sigmoid(b), rtol=1e-14, atol=0)


def test_oracle_fused_is_invariant_to_the_scale_of_q_and_k(oracle_mod):
    """Only the directions of q and k matter (up to the eps of the norm)."""
    raw = _raw_tiny([40], H=2, dk=8, dv=6, s0_std=0.2)
    y1, s1 = oracle_mod.recurrence_fused(raw.q, raw.k, raw.v, raw.a, raw.b, raw.cu_seqlens,
                                         z=raw.z, S_init=raw.S0)
    y2, s2 = oracle_mod.recurrence_fused(raw.q * 8, raw.k * 2, raw.v, raw.a, raw.b,
                                         raw.cu_seqlens, z=raw.z, S_init=raw.S0)
    assert oracle_mod.rel_l2(y2, y1) < 1e-6 and oracle_mod.rel_l2(s2, s1) < 1e-6
    assert oracle_mod.rel_l2(y2, y1) > 0          # eps does enter


def test_oracle_fused_zero_keys_leave_only_the_decay(oracle_mod):
    """k = 0 gives k_hat = 0: nothing is erased or written, so S_t =
    Diag(exp(g_t)) S_{t-1} in closed form and o_t = scale S_t^T q_hat_t."""
    raw = _raw_tiny([12], H=1, dk=4, dv=3, s0_std=0.5, gated=False)
    k0 = torch.zeros_like(raw.k)
    y, st = oracle_mod.recurrence_fused(raw.q, k0, raw.v, raw.a, raw.b, raw.cu_seqlens,
                                        S_init=raw.S0, scale=1.5)
    S = raw.S0[0, 0].double().numpy().copy()
    for t in range(12):
        at = raw.a[t, 0].double().numpy()
        S = np.diag(np.exp(-5.0 / (1.0 + np.exp(-at)))) @ S
        qt = raw.q[t, 0].double().numpy()
        qh = qt / math.sqrt(float(qt @ qt) + 1e-6)
        np.testing.assert_allclose(y[t, 0], 1.5 * S.T @ qh, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(st[0], S, rtol=1e-13, atol=1e-16)


def test_raw_generator_shares_the_processed_draws():
    """make_raw_prefill draws the very numbers make_prefill processes: normalising
    its q, k and squashing its a, b in fp32 gives make_prefill's inputs."""
    raw = kda_inputs.make_raw_prefill([30, 7], 2, 16, 8, "f32", True, 0.1, 53, 8.0, 4.0)
    ref = kda_inputs.make_prefill([30, 7], 2, 16, 8, "f32", True, 0.1, 53, 8.0, 4.0)
    assert torch.allclose(raw.q / raw.q.norm(dim=-1, keepdim=True), ref.q, atol=1e-6)
    assert torch.equal(raw.v, ref.v) and torch.equal(raw.z, ref.z) and torch.equal(raw.S0, ref.S0)
    assert torch.allclose(kda_inputs.G_MIN * torch.sigmoid(raw.a), ref.g, atol=1e-6)
    assert torch.allclose(torch.sigmoid(raw.b), ref.beta, atol=1e-6)
    dec = kda_inputs.make_raw_decode(3, 2, 8, 8, "bf16", True, 0.02, 2, 54)
    assert dec.q.shape == (2, 3, 2, 8) and dec.b.shape == (2, 3, 2) and dec.a.dtype == torch.bfloat16
