"""fp64 numpy model of the blocked (chunkwise) algorithm the HIP prefill runs.

Test infrastructure: it documents the kernel's algebra and is checked against
the sequential oracle on the CPU; it shares no code with the HIP library.

Per chunk of C tokens entering with state S (dk x dv), with G_t the in-chunk
running sum of g (G_0 = 0) and R_a the value of G at the start of 16-token
sub-tile a:
    A[t, j] = sum_c k_tc k_jc exp(G_tc - G_jc)     j < t     (gated Gram)
    P[t, j] = sum_c q_tc k_jc exp(G_tc - G_jc)     j <= t
    Delta   = (I + diag(beta) A)^{-1} diag(beta) (V - (K * e^G) S)
    O       = (Q * e^G) S + P Delta
    S_next  = Diag(e^{G_C}) S + (K * e^{G_C - G})^T Delta
The exponential factors are formed from references inside the chunk so no
factor exceeds e^{16 |g_min|} (page "Exercices", Niveau 2 Q8): a diagonal
block uses R_a for both sides, an off-diagonal block (a, b) uses the end of
sub-tile b for both sides (each factor <= 1).  The unit lower-triangular
inverse is blocked: 16 x 16 diagonal inverses by forward substitution, then
off-diagonal blocks level by level, X_ab = -L_aa^{-1} sum_{b<=c<a} L_ac X_cb.
"""
import numpy as np


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def _blocked_unit_lower_inverse(L, tile=16):
    n = L.shape[0]
    nt = n // tile
    X = np.zeros_like(L)
    sl = lambda i: slice(i * tile, (i + 1) * tile)
    for a in range(nt):                                   # diagonal blocks
        Laa = L[sl(a), sl(a)]
        Xa = np.zeros((tile, tile))
        for j in range(tile):
            x = np.zeros(tile)
            x[j] = 1.0
            for i in range(j + 1, tile):
                x[i] = -Laa[i, :i] @ x[:i]
            Xa[:, j] = x
        X[sl(a), sl(a)] = Xa
    for d in range(1, nt):                                # off-diagonal levels
        for a in range(d, nt):
            b = a - d
            Y = sum(L[sl(a), sl(c)] @ X[sl(c), sl(b)] for c in range(b, a))
            X[sl(a), sl(b)] = -X[sl(a), sl(a)] @ Y
    return X


def chunk_forward(q, k, v, g, beta, z=None, S0=None, C=64, scale=1.0):
    """One head.  q, k, g: [T, dk]; v, z: [T, dv]; beta: [T].  Returns (y, S_T)."""
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else _f64(S0).copy()
    y = np.zeros((T, dv))
    nt = C // 16
    for c0 in range(0, T, C):
        n = min(C, T - c0)
        # masked (zero) tail rows: k = q = v = 0, g = 0, beta = 0
        pad = lambda x: np.concatenate([x[c0:c0 + n], np.zeros((C - n,) + x.shape[1:])])
        qc, kc, vc, gc, bc = pad(q), pad(k), pad(v), pad(g), pad(beta)
        G = np.cumsum(gc, axis=0)                          # [C, dk]
        R = np.array([G[16 * a - 1] if a > 0 else np.zeros(dk) for a in range(nt)])
        E = np.array([G[16 * a + 15] for a in range(nt)])  # end of each sub-tile
        A = np.zeros((C, C))
        P = np.zeros((C, C))
        for a in range(nt):
            ta = slice(16 * a, 16 * a + 16)
            for b in range(a + 1):
                tb = slice(16 * b, 16 * b + 16)
                ref = R[a] if b == a else E[b]
                row = np.exp(G[ta] - ref)                  # <= 1
                col = np.exp(ref - G[tb])                  # <= e^80 (diag) or <= 1
                assert row.max() <= 1.0 + 1e-12
                if b < a:
                    assert col.max() <= 1.0 + 1e-12
                A[ta, tb] = (kc[ta] * row) @ (kc[tb] * col).T
                P[ta, tb] = (qc[ta] * row) @ (kc[tb] * col).T
        A = np.tril(A, -1)
        P = np.tril(P, 0)
        L = np.eye(C) + bc[:, None] * A
        Tinv = _blocked_unit_lower_inverse(L)
        eG = np.exp(G)
        Rhs = bc[:, None] * (vc - (kc * eG) @ S)
        Delta = Tinv @ Rhs
        O = (qc * eG) @ S + P @ Delta
        if z is not None:
            O = O * (1.0 / (1.0 + np.exp(-pad(_f64(z)))))
        y[c0:c0 + n] = scale * O[:n]
        S = np.exp(G[-1])[:, None] * S + (kc * np.exp(G[-1] - G)).T @ Delta
    return y, S


# ---------------------------------------------------------------------------
# Two-pass form.  Everything in a chunk that does not involve the entering
# state is formed first, for every chunk at once ("prep"); a sequential pass
# then carries the state through the chunks with three products each.
#   W  = (I + diag(beta) A)^{-1} diag(beta) (K * e^G)      [C, dk]
#   U  = (I + diag(beta) A)^{-1} diag(beta) V              [C, dv]
#   Qt = scale (Q * e^G)     Pm = scale P                  [C, dk], [C, C]
#   Kh = K * e^{G_C - G]     gam = e^{G_C}                 [C, dk], [dk]
# and per chunk, with S the entering state:
#   Delta = U - W S,  O = Qt S + Pm Delta,  S <- gam * S + Kh^T Delta.
# The prep side forms the gated Gram products with one reference per
# 16-token sub-tile: row operand X_t e^{G_t - R_a(t)} (<= 1), column operand
# K_j e^{R_b(j) - G_j} (<= e^80), and for an off-diagonal block (a, b) the
# column factor e^{R_a - R_b} (<= 1).
# ---------------------------------------------------------------------------
def chunk_prep(q, k, v, g, beta, C=64, scale=1.0):
    """Per-chunk products of one head; returns a list of dicts (one per chunk)."""
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    T, dk = k.shape
    nt = C // 16
    out = []
    for c0 in range(0, T, C):
        n = min(C, T - c0)
        pad = lambda x: np.concatenate([x[c0:c0 + n], np.zeros((C - n,) + x.shape[1:])])
        qc, kc, vc, gc, bc = pad(q), pad(k), pad(v), pad(g), pad(beta)
        G = np.cumsum(gc, axis=0)
        R = np.array([G[16 * a - 1] if a > 0 else np.zeros(dk) for a in range(nt)])
        sub = np.arange(C) // 16
        er = np.exp(G - R[sub])                      # <= 1
        ec = np.exp(R[sub] - G)                      # <= e^{16 |g_min|}
        Kr, Qr, Kc = kc * er, qc * er, kc * ec
        A = np.zeros((C, C))
        P = np.zeros((C, C))
        for a in range(nt):
            ta = slice(16 * a, 16 * a + 16)
            for b in range(a + 1):
                tb = slice(16 * b, 16 * b + 16)
                col = Kc[tb] * np.exp(R[a] - R[b])   # factor <= 1 (1 on the diagonal)
                A[ta, tb] = Kr[ta] @ col.T
                P[ta, tb] = Qr[ta] @ col.T
        A = np.tril(A, -1)
        P = np.tril(P, 0)
        Linv = _blocked_unit_lower_inverse(np.eye(C) + bc[:, None] * A)
        LB = Linv * bc[None, :]
        eG = np.exp(G)
        out.append(dict(W=LB @ (kc * eG), U=LB @ vc, Qt=scale * qc * eG, Pm=scale * P,
                        Kh=kc * np.exp(G[-1] - G), gam=np.exp(G[-1]), n=n))
    return out


def state_scan(prep, dv, z=None, S0=None):
    """Sequential pass over prep's chunks; returns (y, S_T)."""
    dk = prep[0]["W"].shape[1] if prep else 0
    S = np.zeros((dk, dv)) if S0 is None else _f64(S0).copy()
    ys = []
    for ch in prep:
        Delta = ch["U"] - ch["W"] @ S
        O = ch["Qt"] @ S + ch["Pm"] @ Delta
        S = ch["gam"][:, None] * S + ch["Kh"].T @ Delta
        ys.append(O[:ch["n"]])
    y = np.concatenate(ys) if ys else np.zeros((0, dv))
    if z is not None:
        y = y / (1.0 + np.exp(-_f64(z)))
    return y, S
