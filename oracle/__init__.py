"""fp64 CPU oracle of the KDA recurrence -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library: the arithmetic
lives in `kda_oracle.c` (plain C, fp64, OpenMP over independent chains) and,
for tiny inputs, in `brute.py` (explicit dk x dk transition matrices in numpy).

Definition followed (page "Exercices", Niveau 2 Q7 for the three operations,
Q8 for the bounded log-decay, Q9 for unit keys; page "Ce qui est public et ce
qui ne l'est pas" for the output gate; page "Exercices", Niveau 3 Q21-Q22 for
the KCP pair and its composition):

    S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
    o_t = scale * S_t^T q_t,     y_t = o_t * sigmoid(z_t)  (gated)

The fused input step (`gates`, `recurrence_fused`) forms the recurrence's
inputs from raw ones in fp64: q and k scaled to unit length as
x / sqrt(sum x^2 + eps), the log-decay g = g_min * sigmoid(a), beta =
sigmoid(b); it then runs the same fp64 loop (dtype code F64: every input double).

Every function here is pinned by the CPU tests (brute force, closed forms,
invariants, the KCP identities); see the tests named test_oracle_*.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None

BF16, F32, F64 = 0, 1, 2
G_MIN = -5.0          # lower bound of the log-decay (page "Exercices", Niveau 2 Q8)
NORM_EPS = 1e-6       # x / sqrt(sum x^2 + eps) in the fused input step


def build() -> str:
    """Compile the C oracle with the host compiler (no HIP involved)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-std=c11",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    vp, dp, ip = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    lib.kdao_recurrence.argtypes = [ctypes.c_int, ctypes.c_int, ip, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_double, vp, vp, vp, vp, vp, vp,
                                    ctypes.c_int, ip, dp, dp, ctypes.c_int]
    lib.kdao_recurrence.restype = ctypes.c_int
    lib.kdao_kcp.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                             ctypes.c_double, vp, vp, vp, vp, vp, vp, ctypes.c_int, ip, dp, dp, dp,
                             dp, dp, dp, ctypes.c_int]
    lib.kdao_kcp.restype = ctypes.c_int
    lib.kdao_compose.argtypes = [ctypes.c_int, ctypes.c_int, dp, dp, dp, dp, dp, dp]
    lib.kdao_compose.restype = None
    lib.kdao_max_threads.argtypes = []
    lib.kdao_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def default_threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _raw(t: Optional[torch.Tensor]):
    """CPU contiguous tensor -> (dtype code, numpy array holding its bits)."""
    if t is None:
        return None, None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return BF16, t.view(torch.int16).numpy()
    if t.dtype == torch.float32:
        return F32, t.numpy()
    if t.dtype == torch.float64:
        return F64, t.numpy()
    raise TypeError(f"oracle inputs must be bf16, fp32 or fp64, got {t.dtype}")


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().to(torch.float32).numpy()


def _gate(t: torch.Tensor, dt: int) -> np.ndarray:
    """g or beta as the C oracle reads them: fp32, or fp64 when every input is fp64."""
    if dt == F64:
        return t.detach().cpu().contiguous().to(torch.float64).numpy()
    return _f32(t)


def recurrence(q, k, v, g, beta, cu_seqlens, z=None, S_init=None, scale: float = 1.0,
               chains: Optional[Sequence[Tuple[int, int]]] = None, want_y: bool = True,
               chain_states: Optional[np.ndarray] = None, nthreads: Optional[int] = None):
    """Sequential fp64 recurrence over packed sequences.

    q, k: [T, H, dk]; v, z: [T, H, dv] (bf16, fp32 or fp64, same dtype);
    g: [T, H, dk], beta: [T, H]: fp32 (fp64 when q..z are fp64);
    cu_seqlens: [N+1] int.
    S_init: [N, H, dk, dv] (any float dtype; widened to fp64) or None (zeros).
    chains: list of (seq, head) to run; None runs all of them.
    chain_states: fp64 [nchains, dk, dv] initial states in chain order
      (overrides S_init).
    Returns (y [T, H, dv] fp64 -- NaN where no chain wrote -- or None,
             states [nchains, dk, dv] fp64 in chain order).
    """
    lib = _load()
    dt, qn = _raw(q)
    dtk, kn = _raw(k)
    dtv, vn = _raw(v)
    dtz, zn = _raw(z)
    if len({dt, dtk, dtv} | ({dtz} if z is not None else set())) != 1:
        raise TypeError("q, k, v, z must share one dtype")
    T, H, dk = q.shape
    dv = v.shape[-1]
    gn = _gate(g, dt)
    bn = _gate(beta, dt)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    N = cu.size - 1
    if chains is None:
        ch = None
        nch = N * H
        pairs = [(n, h) for n in range(N) for h in range(H)]
    else:
        pairs = [(int(a), int(b)) for a, b in chains]
        ch = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
        nch = len(pairs)
    state = np.zeros((nch, dk, dv), dtype=np.float64)
    if chain_states is not None:
        state[...] = np.asarray(chain_states, dtype=np.float64).reshape(nch, dk, dv)
    elif S_init is not None:
        S_np = (S_init.detach().cpu().to(torch.float64).numpy()
                if isinstance(S_init, torch.Tensor) else np.asarray(S_init, dtype=np.float64))
        for i, (n, h) in enumerate(pairs):
            state[i] = S_np[n, h]
    y = np.full((T, H, dv), np.nan, dtype=np.float64) if want_y else None
    rc = lib.kdao_recurrence(dt, N, _ptr(cu), H, dk, dv, float(scale), _ptr(qn), _ptr(kn),
                             _ptr(vn), _ptr(gn), _ptr(bn), _ptr(zn), nch, _ptr(ch), _ptr(state),
                             _ptr(y), nthreads or default_threads())
    if rc != 0:
        raise ValueError("kdao_recurrence rejected its arguments")
    return y, state


def kcp(q, k, v, g, beta, seg_bounds, z=None, S0=None, scale: float = 1.0, want_y: bool = True,
        want_pairs: bool = False, nthreads: Optional[int] = None):
    """KCP over one sequence (all tokens of q..beta) split at seg_bounds.

    Returns a dict with 'final' [H, dk, dv], 'starts' [nseg, H, dk, dv], and,
    if asked, 'y' [T, H, dv] and the pairs 'M' [nseg, H, dk, dk], 'Sloc'.
    """
    lib = _load()
    dt, qn = _raw(q)
    _, kn = _raw(k)
    _, vn = _raw(v)
    _, zn = _raw(z)
    T, H, dk = q.shape
    dv = v.shape[-1]
    gn = _gate(g, dt)
    bn = _gate(beta, dt)
    sb = np.ascontiguousarray(np.asarray(seg_bounds, dtype=np.int64))
    nseg = sb.size - 1
    s0 = None
    if S0 is not None:
        s0 = np.ascontiguousarray(
            S0.detach().cpu().to(torch.float64).numpy() if isinstance(S0, torch.Tensor)
            else np.asarray(S0, dtype=np.float64)).reshape(H, dk, dv)
    M = np.zeros((nseg, H, dk, dk)) if want_pairs else None
    L = np.zeros((nseg, H, dk, dv)) if want_pairs else None
    starts = np.zeros((nseg, H, dk, dv))
    final = np.zeros((H, dk, dv))
    y = np.full((T, H, dv), np.nan) if want_y else None
    rc = lib.kdao_kcp(dt, T, H, dk, dv, float(scale), _ptr(qn), _ptr(kn), _ptr(vn), _ptr(gn),
                      _ptr(bn), _ptr(zn), nseg, _ptr(sb), _ptr(s0), _ptr(M), _ptr(L),
                      _ptr(starts), _ptr(final), _ptr(y), nthreads or default_threads())
    if rc != 0:
        raise ValueError("kdao_kcp rejected its arguments")
    out = {"final": final, "starts": starts}
    if want_y:
        out["y"] = y
    if want_pairs:
        out["M"], out["Sloc"] = M, L
    return out


def checkpoints(q, k, v, g, beta, cu_seqlens, interval: int, S_init=None, scale: float = 1.0,
                nthreads: Optional[int] = None):
    """States after every `interval` tokens of each packed sequence: the state a
    prefix cache saves at a boundary (page "Exercices", Niveau 3 Q26).

    Checkpoint j of sequence n is the state after its first (j + 1) interval
    tokens, for j < floor(len_n / interval).  The sequential recurrence runs
    span by span, each span starting from the previous one's fp64 state.
    Returns (ckpt [sum_n floor(len_n / interval), H, dk, dv] fp64,
             offsets [N + 1] int64: sequence n's checkpoints start at offsets[n]).
    """
    cu = [int(x) for x in np.asarray(cu_seqlens).tolist()]
    N = len(cu) - 1
    T, H, dk = q.shape
    dv = v.shape[-1]
    counts = [max(cu[n + 1] - cu[n], 0) // interval for n in range(N)]
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    out = np.zeros((int(offs[-1]), H, dk, dv))
    heads = [(0, h) for h in range(H)]
    for n in range(N):
        state = np.zeros((H, dk, dv))
        if S_init is not None:
            S_np = (S_init.detach().cpu().to(torch.float64).numpy()
                    if isinstance(S_init, torch.Tensor) else np.asarray(S_init, dtype=np.float64))
            state[...] = S_np[n]
        for j in range(counts[n]):
            sl = slice(cu[n] + j * interval, cu[n] + (j + 1) * interval)
            pick = lambda t: None if t is None else t[sl]
            _, state = recurrence(pick(q), pick(k), pick(v), pick(g), pick(beta), [0, interval],
                                  chains=heads, chain_states=state, scale=scale, want_y=False,
                                  nthreads=nthreads)
            out[offs[n] + j] = state
    return out, offs


def replay(rep, scale: float = 1.0, nthreads: Optional[int] = None):
    """Speculative-decoding replay (page "Exercices", Niveau 3 Q27: the state
    after any accepted prefix is fixed by the draft tokens' inputs, so only
    those are kept and the recurrence is replayed).

    rep: kda_inputs.ReplayInputs.  Each request's Td draft tokens run as one
    sequence from its resident state.  Returns (y [N, Td, H, dv]: the outputs of
    every draft token, committed [N, H, dk, dv]: the state after the first
    accepted[n] tokens (the resident state where accepted[n] = 0)).
    """
    N, Td, H, dk, dv = rep.N, rep.Td, rep.H, rep.dk, rep.dv
    flat = lambda t: None if t is None else t.reshape(N * Td, *t.shape[2:])
    cu = np.arange(0, (N + 1) * Td, Td, dtype=np.int32)
    y, _ = recurrence(flat(rep.q), flat(rep.k), flat(rep.v), flat(rep.g), flat(rep.beta), cu,
                      z=flat(rep.z), S_init=rep.S0, scale=scale, nthreads=nthreads)
    acc = [int(a) for a in rep.accepted.tolist()]
    committed = rep.S0.to(torch.float64).numpy().copy()
    for n in range(N):
        if acc[n] == 0:
            continue
        sl = slice(n * Td, n * Td + acc[n])
        pick = lambda t: None if t is None else flat(t)[sl]
        _, st = recurrence(pick(rep.q), pick(rep.k), pick(rep.v), pick(rep.g), pick(rep.beta),
                           [0, acc[n]], chains=[(0, h) for h in range(H)],
                           chain_states=committed[n], scale=scale, want_y=False,
                           nthreads=nthreads)
        committed[n] = st
    return y.reshape(N, Td, H, dv), committed


def gates(q_raw, k_raw, a, b, eps: float = NORM_EPS):
    """The fused input step in fp64, from raw (unnormalised, pre-activation) inputs.

    q_hat = q / sqrt(sum_c q_c^2 + eps), k_hat likewise (unit keys: page
    "Exercices", Niveau 2 Q9; q is normalised the same way);
    g = g_min * sigmoid(a) per key channel, in (g_min, 0) (bounded decay with
    g_min = -5: same page, Q8, and the decay row of page "Ce qui est public et
    ce qui ne l'est pas");
    beta = sigmoid(b) per (token, head), in (0, 1) (the beta of the KDA
    parametrisation, same table; W_beta, W_alpha are the low-rank projections
    of page "Retrouver les 2,8 T de paramètres", Bloc 4).
    Inputs are widened exactly; returns fp64 tensors (q_hat, k_hat, g, beta).
    """
    qd = q_raw.detach().cpu().to(torch.float64)
    kd = k_raw.detach().cpu().to(torch.float64)
    ad = a.detach().cpu().to(torch.float64)
    bd = b.detach().cpu().to(torch.float64)
    sig = lambda x: 1.0 / (1.0 + torch.exp(-x))
    qh = qd / torch.sqrt((qd * qd).sum(-1, keepdim=True) + eps)
    kh = kd / torch.sqrt((kd * kd).sum(-1, keepdim=True) + eps)
    return qh.contiguous(), kh.contiguous(), (G_MIN * sig(ad)).contiguous(), sig(bd).contiguous()


def _f64(t):
    return None if t is None else t.detach().cpu().to(torch.float64).contiguous()


def recurrence_fused(q_raw, k_raw, v, a, b, cu_seqlens, z=None, S_init=None, scale: float = 1.0,
                     chains=None, want_y: bool = True, chain_states=None, nthreads=None):
    """The recurrence fed by the fused input step: `gates` turns the raw inputs
    into (q_hat, k_hat, g, beta) in fp64, v and z are widened exactly, and the
    fp64 loop of `recurrence` runs on them.  Same arguments and returns as
    `recurrence`, with q_raw, k_raw, a ([T, H, dk]) and b ([T, H]) in place of
    q, k, g, beta."""
    qh, kh, g, beta = gates(q_raw, k_raw, a, b)
    return recurrence(qh, kh, _f64(v), g, beta, cu_seqlens, z=_f64(z), S_init=S_init, scale=scale,
                      chains=chains, want_y=want_y, chain_states=chain_states, nthreads=nthreads)


def compose(M2, S2, M1, S1):
    """(M2, S2) o (M1, S1) = (M2 M1, M2 S1 + S2) in fp64, via the C oracle."""
    lib = _load()
    M2 = np.ascontiguousarray(M2, dtype=np.float64)
    S2 = np.ascontiguousarray(S2, dtype=np.float64)
    M1 = np.ascontiguousarray(M1, dtype=np.float64)
    S1 = np.ascontiguousarray(S1, dtype=np.float64)
    dk, dv = S1.shape
    Mo = np.zeros((dk, dk))
    So = np.zeros((dk, dv))
    lib.kdao_compose(dk, dv, _ptr(M2), _ptr(S2), _ptr(M1), _ptr(S1), _ptr(Mo), _ptr(So))
    return Mo, So


def decode_steps(dec, steps: int, chains: Optional[Sequence[Tuple[int, int]]] = None,
                 scale: float = 1.0, record=(), nthreads: Optional[int] = None):
    """Decode: `steps` single-token recurrence steps on resident states.

    dec: kda_inputs.DecodeInputs; step s uses pooled set s % P.
    chains: (request, head) pairs to follow (None: all).  The state is kept in
    fp64 between steps.  Returns (y of the last step [N, H, dv] (NaN for
    chains not followed), {step: states [nchains, dk, dv]} for the steps in
    `record` (1-based step counts), final states).
    """
    N, H, dk, dv = dec.N, dec.H, dec.dk, dec.dv
    P = dec.q.shape[0]
    if chains is None:
        chains = [(n, h) for n in range(N) for h in range(H)]
    chains = [(int(a), int(b)) for a, b in chains]
    cu = np.arange(N + 1, dtype=np.int32)
    state = np.stack([dec.S0[n, h].to(torch.float64).numpy() for n, h in chains])
    snaps = {}
    y = None
    for s in range(steps):
        p = s % P
        y, state = recurrence(dec.q[p], dec.k[p], dec.v[p], dec.g[p], dec.beta[p], cu,
                              z=None if dec.z is None else dec.z[p],
                              chain_states=state, scale=scale, chains=chains,
                              nthreads=nthreads)
        if (s + 1) in record:
            snaps[s + 1] = state.copy()
    return y, snaps, state


def rel_l2(a, b) -> float:
    """||a - b||_2 / ||b||_2 in fp64 over the flattened arrays (b = reference);
    the absolute L2 norm of the difference when ||b||_2 == 0."""
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    d = np.linalg.norm(a - b)
    nb = np.linalg.norm(b)
    return float(d / nb) if nb > 0 else float(d)


def row_err(a, b) -> float:
    """Worst row of the difference, relative to the reference's typical row:
    max_r ||a_r - b_r||_2 / sqrt(mean_r ||b_r||_2^2) in fp64, rows along the
    last axis (one (token, head) output vector, or one row of a state), b the
    reference.  Measured against the root-mean-square row norm rather than each
    row's own norm, so a row whose reference is near zero does not dominate,
    while an error confined to a few rows (one token of every chunk, say) is
    not averaged away as it is in rel_l2.  The absolute worst row norm when b
    is all zero; 0.0 for empty arrays."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        raise ValueError(f"row_err: shapes differ {a.shape} vs {b.shape}")
    if a.size == 0:
        return 0.0
    n = b.shape[-1] if b.ndim else 1
    a = a.reshape(-1, n)
    b = b.reshape(-1, n)
    d = np.sqrt(((a - b) ** 2).sum(axis=1)).max()
    typ = np.sqrt((b ** 2).sum(axis=1).mean())
    return float(d / typ) if typ > 0 else float(d)
