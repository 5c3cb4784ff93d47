"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerances: relative L2 error (over the whole flattened tensor, oracle as the
reference) <= 1e-4 for fp32 inputs and <= 2e-2 for bf16 inputs, on outputs y
and on final states.  Sizes span several chunks and a ragged tail; the
long-memory stress draws make the carried state matter across chunks and
segments.
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


def _dev(t):
    return None if t is None else t.cuda()


def run_prefill(kda, inp, chunk, scale=1.0, S0=None):
    cu = inp.cu_seqlens.cuda() if inp.num_seqs > 1 else None
    s0 = inp.S0 if S0 is None else S0
    y, fs = kda.chunk_fwd(_dev(inp.q), _dev(inp.k), _dev(inp.v), _dev(inp.g), _dev(inp.beta),
                          cu_seqlens=cu, z=_dev(inp.z), initial_state=_dev(s0), chunk=chunk,
                          scale=scale)
    torch.cuda.synchronize()
    return y.cpu(), fs.cpu()


def oracle_prefill(inp, scale=1.0):
    return oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, z=inp.z,
                             S_init=inp.S0, scale=scale)


def assert_parity(name, inp, y, fs, yo, so, tol):
    """Whole-tensor rel-L2 <= tol (the dtype's tolerance) and every (token,
    head) row and state row within the dtype's row bound (tests/parity.py)."""
    dt = "f32" if tol <= TOL["f32"] else "bf16"
    out = parity.check(name, dt, y=(y, yo), state=(fs, so))
    return out["y"][0], out["state"][0]


# ---------------------------------------------------------------- decode
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("f32", 128), ("bf16", 64)])
def test_decode_matches_oracle(kda, dtype, d):
    dec = kda_inputs.make_decode(N=5, H=3, dk=d, dv=d, dtype=dtype, gated=True, s0_std=0.02,
                                 pool=3, seed=31)
    state = dec.S0.clone().cuda()
    steps = 6
    for s in range(steps):
        p = s % 3
        y = kda.decode_step(dec.q[p].cuda(), dec.k[p].cuda(), dec.v[p].cuda(), dec.g[p].cuda(),
                            dec.beta[p].cuda(), state, z=dec.z[p].cuda())
    torch.cuda.synchronize()
    yo, _, so = oracle.decode_steps(dec, steps)
    parity.check(f"decode {dtype} d={d}", dtype, y=(y, yo), state=(state, so))


def test_decode_and_replay_are_deterministic(kda):
    """The same step from two copies of one state gives the same bits, as do
    two replay calls (no atomics or order-dependent reductions)."""
    dec = kda_inputs.make_decode(N=16, H=8, dk=128, dv=128, dtype="bf16", gated=True, s0_std=0.02,
                                 pool=1, seed=12)
    x = [getattr(dec, n)[0].cuda() for n in ("q", "k", "v", "g", "beta", "z")]
    sa, sb = dec.S0.clone().cuda(), dec.S0.clone().cuda()
    ya = kda.decode_step(*x[:5], sa, z=x[5])
    yb = kda.decode_step(*x[:5], sb, z=x[5])
    torch.cuda.synchronize()
    assert torch.equal(ya, yb) and torch.equal(sa, sb)
    rep = kda_inputs.make_replay(8, 3, 4, 128, 128, "bf16", True, 0.02, 13)
    r = [getattr(rep, n).cuda() for n in ("q", "k", "v", "g", "beta", "z")]
    ra, rb = rep.S0.clone().cuda(), rep.S0.clone().cuda()
    acc = rep.accepted.cuda()
    y1 = kda.decode_replay(*r[:5], ra, z=r[5], accepted=acc)
    y2 = kda.decode_replay(*r[:5], rb, z=r[5], accepted=acc)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(ra, rb)


def test_decode_ungated_and_scaled(kda):
    dec = kda_inputs.make_decode(N=2, H=2, dk=128, dv=128, dtype="f32", gated=False,
                                 s0_std=0.5, pool=1, seed=8)
    state = dec.S0.clone().cuda()
    y = kda.decode_step(dec.q[0].cuda(), dec.k[0].cuda(), dec.v[0].cuda(), dec.g[0].cuda(),
                        dec.beta[0].cuda(), state, scale=0.25)
    torch.cuda.synchronize()
    yo, _, so = oracle.decode_steps(dec, 1, scale=0.25)
    assert rel_l2(y.cpu().double().numpy(), yo) <= 1e-5
    assert rel_l2(state.cpu().double().numpy().reshape(so.shape), so) <= 1e-5


# ---------------------------------------------------------------- prefill
@pytest.mark.parametrize("dtype,d,tol", [("f32", 64, 1e-4), ("bf16", 128, 2e-2)])
def test_decode_steps_equal_prefill(kda, dtype, d, tol):
    """T decode steps of one request equal one prefill over the same T tokens
    (two different kernels: the one-pass step and the two-pass chunked form),
    with the tokens laid out [T, H, d] for the prefill and [1, H, d] per step."""
    T, H = 70, 3
    inp = kda_inputs.make_prefill([T], H, d, d, dtype, True, 0.05, 81, 8.0, 4.0)
    y_p, s_p = run_prefill(kda, inp, chunk=64, scale=0.8)
    state = inp.S0.clone().cuda()
    ys = []
    for t in range(T):
        sl = slice(t, t + 1)
        ys.append(kda.decode_step(inp.q[sl].cuda(), inp.k[sl].cuda(), inp.v[sl].cuda(),
                                  inp.g[sl].cuda(), inp.beta[sl].cuda(), state,
                                  z=inp.z[sl].cuda(), scale=0.8).cpu())
    torch.cuda.synchronize()
    ey = rel_l2(torch.cat(ys).double().numpy(), y_p.double().numpy())
    es = rel_l2(state.cpu().double().numpy(), s_p.double().numpy())
    log(f"[parity] decode x{T} vs prefill {dtype} d{d}: y={ey:.3e} state={es:.3e}")
    assert ey <= tol and es <= tol


def test_prefill_tiny_fp32_workload(kda):
    """B=1, H=2, T=256, dk=dv=64, chunk 16, fp32, ungated, S0 = 0."""
    inp = kda_inputs.make_workload(0)
    y, fs = run_prefill(kda, inp, chunk=16)
    yo, so = oracle_prefill(inp)
    assert_parity("tiny fp32 c16", inp, y, fs, yo, so, TOL["f32"])


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("stress", [None, "chunk"])
def test_prefill_fp32_d64(kda, chunk, stress):
    inp = kda_inputs.make_workload(0, stress, lens=[333], H=3, gated=True, s0_std=0.1)
    y, fs = run_prefill(kda, inp, chunk=chunk, scale=0.5)
    yo, so = oracle_prefill(inp, scale=0.5)
    assert_parity(f"fp32 d64 c{chunk} {stress}", inp, y, fs, yo, so, TOL["f32"])


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("stress", [None, "chunk"])
def test_prefill_fp32_d128(kda, chunk, stress):
    inp = kda_inputs.make_workload(1, stress, lens=[197], H=2, dtype="f32", s0_std=0.05)
    y, fs = run_prefill(kda, inp, chunk=chunk)
    yo, so = oracle_prefill(inp)
    assert_parity(f"fp32 d128 c{chunk} {stress}", inp, y, fs, yo, so, TOL["f32"])


@pytest.mark.parametrize("chunk", [64, 32, 16])
@pytest.mark.parametrize("stress", [None, "chunk"])
def test_prefill_bf16_d128(kda, chunk, stress):
    inp = kda_inputs.make_workload(1, stress, lens=[1000], H=4, s0_std=0.02)
    y, fs = run_prefill(kda, inp, chunk=chunk)
    yo, so = oracle_prefill(inp)
    assert_parity(f"bf16 d128 c{chunk} {stress}", inp, y, fs, yo, so, TOL["bf16"])


@pytest.mark.parametrize("chunk", [64, 32, 16])
def test_prefill_bf16_d64(kda, chunk):
    inp = kda_inputs.make_workload(1, "chunk", lens=[517], H=3, dk=64, dv=64, s0_std=0.05)
    y, fs = run_prefill(kda, inp, chunk=chunk)
    yo, so = oracle_prefill(inp)
    assert_parity(f"bf16 d64 c{chunk}", inp, y, fs, yo, so, TOL["bf16"])


def test_prefill_varlen_with_ragged_and_empty_sequences(kda):
    lens = [1, 17, 64, 65, 0, 200, 127, 3]
    inp = kda_inputs.make_prefill(lens, 5, 128, 128, "bf16", True, 0.02, 77, 8.0, 4.0)
    y, fs = run_prefill(kda, inp, chunk=64)
    yo, so = oracle_prefill(inp)
    assert_parity("varlen ragged", inp, y, fs, yo, so, TOL["bf16"])
    # the empty sequence passes its initial state through unchanged
    np.testing.assert_array_equal(fs[4].numpy(), inp.S0[4].numpy())


@pytest.mark.parametrize("lens", [[0], [0, 0, 0]])
def test_prefill_zero_tokens(kda, lens):
    """No tokens at all: y is empty and every final state is its initial state."""
    inp = kda_inputs.make_prefill(lens, 3, 64, 64, "bf16", True, 0.05, 79, 0.0, 0.0)
    y, fs = run_prefill(kda, inp, chunk=64)
    assert y.shape == (0, 3, 64)
    np.testing.assert_array_equal(fs.numpy(), inp.S0.numpy())


def test_prefill_varlen_many_short_sequences(kda):
    """More than 1024 packed sequences (no longest-first reordering), lengths 0..40."""
    rng = np.random.default_rng(5)
    lens = rng.integers(0, 41, 1100).tolist()
    inp = kda_inputs.make_prefill(lens, 1, 64, 64, "bf16", True, 0.05, 78, 8.0, 4.0)
    y, fs = run_prefill(kda, inp, chunk=16)
    yo, so = oracle_prefill(inp)
    assert_parity("varlen 1100 short", inp, y, fs, yo, so, TOL["bf16"])


def test_prefill_many_chains_wide_scan_waves(kda):
    """Enough (sequence, head) chains that each scan wave takes 32 state columns."""
    rng = np.random.default_rng(6)
    lens = rng.integers(1, 200, 16).tolist()
    inp = kda_inputs.make_prefill(lens, 64, 64, 64, "bf16", True, 0.05, 79, 8.0, 4.0)
    y, fs = run_prefill(kda, inp, chunk=64)
    yo, so = oracle_prefill(inp)
    assert_parity("varlen 1024 chains", inp, y, fs, yo, so, TOL["bf16"])


def test_prefill_many_chains_two_value_tiles(kda):
    """fp32, dk = dv = 128 and 1024 (sequence, head) chains: each scan wave takes
    two 16-column value tiles and stages its own share of the chunk operands
    (the operands of one chunk do not fit twice in LDS beside loader waves)."""
    rng = np.random.default_rng(8)
    lens = rng.integers(1, 61, 16).tolist()
    inp = kda_inputs.make_prefill(lens, 64, 128, 128, "f32", True, 0.05, 80, 8.0, 4.0)
    y, fs = run_prefill(kda, inp, chunk=64)
    yo, so = oracle_prefill(inp)
    assert_parity("fp32 1024 chains", inp, y, fs, yo, so, TOL["f32"])


def test_prefill_varlen_workload_shape_reduced(kda):
    """Varlen workload recipe (16 sequences, lengths uniform) at reduced lengths and heads."""
    inp = kda_inputs.make_workload(2, H=6, lmin=20, lmax=700)
    y, fs = run_prefill(kda, inp, chunk=64)
    yo, so = oracle_prefill(inp)
    assert_parity("varlen workload reduced", inp, y, fs, yo, so, TOL["bf16"])


def test_prefill_beta_zero_is_pure_decay(kda):
    """beta = 0 and S0 != 0: y_t = scale (e^{G_t} * S0)^T q_t exactly (GPU invariant run)."""
    inp = kda_inputs.make_workload(0, "chunk", lens=[300], H=2, s0_std=1.0)
    inp.beta.zero_()
    y, fs = run_prefill(kda, inp, chunk=64)
    yo, so = oracle_prefill(inp)
    assert_parity("beta=0", inp, y, fs, yo, so, TOL["f32"])


def test_prefill_exact_retrieval_orthonormal_keys(kda):
    """alpha = 1, beta = 1, orthonormal keys, S0 = 0: query k_j returns v_j."""
    T, d = 100, 128
    rng = np.random.default_rng(5)
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = torch.tensor(Qm[:, :T].T.copy(), dtype=torch.float32)
    v = torch.tensor(rng.standard_normal((T, d)), dtype=torch.float32)
    pick = torch.tensor([int(rng.integers(0, t + 1)) for t in range(T)])
    inp = kda_inputs.KDAInputs(q=keys[pick][:, None].contiguous(), k=keys[:, None].contiguous(),
                               v=v[:, None].contiguous(), z=None,
                               g=torch.zeros(T, 1, d), beta=torch.ones(T, 1),
                               cu_seqlens=torch.tensor([0, T], dtype=torch.int32), S0=None,
                               H=1, dk=d, dv=d, dtype="f32")
    y, fs = run_prefill(kda, inp, chunk=16)
    err = (y[:, 0].double() - v[pick].double()).abs().max().item()
    log(f"[parity] exact retrieval max abs err {err:.3e}")
    assert err <= 1e-4


@pytest.mark.parametrize("small", [16, 32])
def test_prefill_chunk_size_changes_rounding_only(kda, small):
    inp = kda_inputs.make_workload(1, "chunk", lens=[700], H=2, s0_std=0.02)
    ys, ss = run_prefill(kda, inp, chunk=small)
    y64, s64 = run_prefill(kda, inp, chunk=64)
    ey = rel_l2(ys.double().numpy(), y64.double().numpy())
    es = rel_l2(ss.double().numpy(), s64.double().numpy())
    assert ey <= TOL["bf16"] and es <= TOL["bf16"], (ey, es)


def test_prefill_resume_equals_single_call(kda):
    inp = kda_inputs.make_workload(1, "chunk", lens=[600], H=2, s0_std=0.02)
    y, fs = run_prefill(kda, inp, chunk=64)
    a = kda_inputs.KDAInputs(inp.q[:250], inp.k[:250], inp.v[:250], inp.z[:250], inp.g[:250],
                             inp.beta[:250], torch.tensor([0, 250], dtype=torch.int32), inp.S0,
                             inp.H, inp.dk, inp.dv, inp.dtype)
    b = kda_inputs.KDAInputs(inp.q[250:], inp.k[250:], inp.v[250:], inp.z[250:], inp.g[250:],
                             inp.beta[250:], torch.tensor([0, 350], dtype=torch.int32), None,
                             inp.H, inp.dk, inp.dv, inp.dtype)
    ya, sa = run_prefill(kda, a, chunk=64)
    yb, sb = run_prefill(kda, b, chunk=64, S0=sa)
    assert rel_l2(torch.cat([ya, yb]).double().numpy(), y.double().numpy()) <= 1e-2
    assert rel_l2(sb.double().numpy(), fs.double().numpy()) <= 1e-2


def test_prefill_is_deterministic(kda):
    inp = kda_inputs.make_workload(2, H=4, lmin=50, lmax=300)
    y1, s1 = run_prefill(kda, inp, chunk=64)
    y2, s2 = run_prefill(kda, inp, chunk=64)
    assert torch.equal(y1, y2) and torch.equal(s1, s2)


def test_prefill_final_state_may_alias_initial_state(kda):
    inp = kda_inputs.make_workload(1, "chunk", lens=[300], H=2, s0_std=0.02)
    st = inp.S0.clone().cuda()
    y, _ = kda.chunk_fwd(inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.g.cuda(),
                         inp.beta.cuda(), z=inp.z.cuda(), initial_state=st, final_state=st)
    torch.cuda.synchronize()
    yo, so = oracle_prefill(inp)
    assert_parity("aliased state", inp, y.cpu(), st.cpu(), yo, so, TOL["bf16"])


# ---------------------------------------------------------------- speculative-decoding replay
def _replay_dev(rep):
    d = {n: getattr(rep, n).cuda() for n in ("q", "k", "v", "g", "beta")}
    d["z"] = None if rep.z is None else rep.z.cuda()
    return d


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_replay_verify_then_commit(kda, dtype, d):
    rep = kda_inputs.make_replay(8, 5, 4, d, d, dtype, True, 0.05, 91, 8.0, 4.0)
    rep.accepted[:2] = torch.tensor([0, 5], dtype=torch.int32)   # none and all accepted
    x = _replay_dev(rep)
    state = rep.S0.cuda()
    y = kda.decode_replay(x["q"], x["k"], x["v"], x["g"], x["beta"], state, z=x["z"], scale=0.5)
    torch.cuda.synchronize()
    # the verify pass only reads the states
    assert torch.equal(state.cpu(), rep.S0)
    kda.decode_replay(x["q"], x["k"], x["v"], x["g"], x["beta"], state,
                      accepted=rep.accepted.cuda(), z=x["z"], scale=0.5, want_y=False)
    torch.cuda.synchronize()
    yo, so = oracle.replay(rep, scale=0.5)
    parity.check(f"replay {dtype} d{d}", dtype, y=(y, yo), committed=(state, so))
    # nothing accepted: bit-identical state
    assert torch.equal(state[0].cpu(), rep.S0[0])


def test_replay_outputs_and_commit_in_one_call(kda):
    rep = kda_inputs.make_replay(6, 4, 3, 128, 128, "bf16", True, 0.05, 92)
    x = _replay_dev(rep)
    state = rep.S0.cuda()
    y = kda.decode_replay(x["q"], x["k"], x["v"], x["g"], x["beta"], state,
                          accepted=rep.accepted.cuda(), z=x["z"])
    torch.cuda.synchronize()
    yo, so = oracle.replay(rep)
    parity.check("replay outputs and commit", "bf16", y=(y, yo), committed=(state, so))


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_replay_long_drafts_across_input_groups(kda, dtype, d):
    """Nine draft tokens: the inputs are staged a few tokens at a time, and the
    accepted prefixes end inside, at the end of, and past the first groups."""
    rep = kda_inputs.make_replay(10, 9, 3, d, d, dtype, True, 0.05, 94, 8.0, 4.0)
    rep.accepted[:] = torch.tensor([0, 1, 3, 4, 5, 7, 8, 9, 2, 6], dtype=torch.int32)
    x = _replay_dev(rep)
    yo, so = oracle.replay(rep)
    # outputs and commit in one call
    state = rep.S0.cuda()
    y = kda.decode_replay(x["q"], x["k"], x["v"], x["g"], x["beta"], state,
                          accepted=rep.accepted.cuda(), z=x["z"])
    torch.cuda.synchronize()
    parity.check(f"replay Td=9 {dtype} d{d}", dtype, y=(y, yo), committed=(state, so))
    # the commit alone gives the same states
    state2 = rep.S0.cuda()
    kda.decode_replay(x["q"], x["k"], x["v"], x["g"], x["beta"], state2,
                      accepted=rep.accepted.cuda(), z=x["z"], want_y=False)
    torch.cuda.synchronize()
    assert rel_l2(state2.cpu().double().numpy(), so) <= TOL[dtype]
    assert torch.equal(state2[0].cpu(), rep.S0[0])


def test_replay_full_acceptance_equals_decode_steps(kda):
    """Accepting every draft token = Td calls of kda_decode_step (same kernels'
    arithmetic per token, so the results agree to rounding)."""
    rep = kda_inputs.make_replay(5, 3, 2, 128, 128, "bf16", True, 0.05, 93)
    rep.accepted[:] = 3
    x = _replay_dev(rep)
    s_rep = rep.S0.cuda()
    y_rep = kda.decode_replay(x["q"], x["k"], x["v"], x["g"], x["beta"], s_rep,
                              accepted=rep.accepted.cuda(), z=x["z"])
    s_dec = rep.S0.cuda()
    for t in range(3):
        y_t = kda.decode_step(x["q"][:, t].contiguous(), x["k"][:, t].contiguous(),
                              x["v"][:, t].contiguous(), x["g"][:, t].contiguous(),
                              x["beta"][:, t].contiguous(), s_dec, z=x["z"][:, t].contiguous())
        torch.cuda.synchronize()
        assert rel_l2(y_rep[:, t].cpu().double().numpy(), y_t.cpu().double().numpy()) <= 1e-5
    assert rel_l2(s_rep.cpu().double().numpy(), s_dec.cpu().double().numpy()) <= 1e-6


# ---------------------------------------------------------------- prefix-cache checkpoints
@pytest.mark.parametrize("chunk,interval", [(64, 128), (16, 48), (64, 64)])
def test_prefill_checkpoints_match_oracle(kda, chunk, interval):
    """States every `interval` tokens of ragged packed sequences (one shorter than
    the interval, one an exact multiple) against the oracle's checkpoints."""
    lens = [300, 40, 256, 129, 0, 1]
    inp = kda_inputs.make_prefill(lens, 3, 128, 128, "bf16", True, 0.05, 81, 8.0, 4.0)
    y, fs, ck, offs = kda.chunk_fwd_checkpointed(
        inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.g.cuda(), inp.beta.cuda(), interval,
        cu_seqlens=inp.cu_seqlens.cuda(), z=inp.z.cuda(), initial_state=inp.S0.cuda(), chunk=chunk)
    torch.cuda.synchronize()
    co, oo = oracle.checkpoints(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, interval,
                                S_init=inp.S0)
    assert offs.cpu().tolist() == oo.tolist()      # integer offsets: exact
    n = int(oo[-1])
    parity.check(f"checkpoints c{chunk} every {interval} ({n} states)", "bf16", checkpoints=(ck[:n], co))
    yo, so = oracle_prefill(inp)
    assert_parity(f"checkpointed prefill c{chunk}", inp, y.cpu(), fs.cpu(), yo, so, TOL["bf16"])


def test_prefill_checkpoints_single_sequence_fp32(kda):
    inp = kda_inputs.make_workload(0, "chunk", lens=[256], s0_std=0.3)
    y, fs, ck, offs = kda.chunk_fwd_checkpointed(
        inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.g.cuda(), inp.beta.cuda(), 32,
        initial_state=inp.S0.cuda(), chunk=16)
    torch.cuda.synchronize()
    co, oo = oracle.checkpoints(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, 32,
                                S_init=inp.S0)
    assert offs.cpu().tolist() == oo.tolist() == [0, 8]
    parity.check("checkpoints fp32 single sequence", "f32", checkpoints=(ck, co))


# ---------------------------------------------------------------- KCP
@pytest.mark.parametrize("dtype,d,chunk", [("bf16", 128, 64), ("f32", 64, 16), ("bf16", 64, 64),
                                           ("f32", 128, 64), ("bf16", 128, 16), ("bf16", 128, 32)])
def test_kcp_scan_matches_sequential_oracle(kda, dtype, d, chunk):
    inp = kda_inputs.make_workload(3, "segment", lens=[4096], H=2, dk=d, dv=d, dtype=dtype,
                                   s0_std=0.05, gated=True)
    nseg = 8
    y, fs = kda.kcp_scan(inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.g.cuda(),
                         inp.beta.cuda(), nseg, z=inp.z.cuda(), initial_state=inp.S0.cuda(),
                         chunk=chunk)
    torch.cuda.synchronize()
    yo, so = oracle_prefill(inp)
    assert_parity(f"kcp {dtype} d{d} c{chunk}", inp, y.cpu(), fs.cpu(), yo, so, TOL[dtype])


@pytest.mark.parametrize("dtype,d,chunk,H,T", [("bf16", 128, 64, 2, 10000), ("f32", 128, 64, 2, 9000),
                                                 ("bf16", 64, 16, 4, 7000), ("f32", 64, 32, 4, 8192)])
def test_kcp_many_segments_two_value_tiles(kda, dtype, d, chunk, H, T):
    """256 segments a head: enough (transition, local state) chains for the
    pair pass to take two value tiles a wave, whose workgroups split their
    waves between transition and value columns; ragged last segments."""
    inp = kda_inputs.make_workload(3, "segment", lens=[T], H=H, dk=d, dv=d, dtype=dtype,
                                   s0_std=0.05, gated=True)
    y, fs = kda.kcp_scan(inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.g.cuda(),
                         inp.beta.cuda(), 256, z=inp.z.cuda(), initial_state=inp.S0.cuda(),
                         chunk=chunk)
    torch.cuda.synchronize()
    yo, so = oracle_prefill(inp)
    assert_parity(f"kcp 256 segments {dtype} d{d} c{chunk}", inp, y.cpu(), fs.cpu(), yo, so, TOL[dtype])


def test_kcp_ragged_segments(kda):
    """T not a multiple of the segment count (trailing segments shorter or empty)."""
    inp = kda_inputs.make_workload(3, "segment", lens=[1001], H=2, s0_std=0.05)
    y, fs = kda.kcp_scan(inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.g.cuda(),
                         inp.beta.cuda(), 7, initial_state=inp.S0.cuda())
    torch.cuda.synchronize()
    yo, so = oracle_prefill(inp)
    assert_parity("kcp ragged", inp, y.cpu(), fs.cpu(), yo, so, TOL["bf16"])


@pytest.mark.parametrize("dtype,d,T,nseg", [("f32", 64, 512, 1), ("f32", 64, 130, 130), ("bf16", 128, 1000, 64)])
def test_kcp_degenerate_segment_counts(kda, dtype, d, T, nseg):
    """One segment (no scan at all), one token a segment, and segments shorter
    than a chunk with the trailing ones empty."""
    inp = kda_inputs.make_workload(3, "segment", lens=[T], H=2, dk=d, dv=d, dtype=dtype,
                                   s0_std=0.05, gated=True)
    y, fs = kda.kcp_scan(inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.g.cuda(),
                         inp.beta.cuda(), nseg, z=inp.z.cuda(), initial_state=inp.S0.cuda())
    torch.cuda.synchronize()
    yo, so = oracle_prefill(inp)
    assert_parity(f"kcp T={T} nseg={nseg}", inp, y.cpu(), fs.cpu(), yo, so, TOL[dtype])


def test_kcp_equals_chunk_fwd(kda):
    inp = kda_inputs.make_workload(3, "segment", lens=[2048], H=2)
    yk, sk = kda.kcp_scan(inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.g.cuda(),
                          inp.beta.cuda(), 16)
    yc, sc = run_prefill(kda, inp, chunk=64)
    torch.cuda.synchronize()
    assert rel_l2(yk.cpu().double().numpy(), yc.double().numpy()) <= 1e-2
    assert rel_l2(sk.cpu().double().numpy(), sc.double().numpy()) <= 1e-2
