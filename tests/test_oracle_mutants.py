"""The oracle's pins have teeth: plausible mistakes planted in a copy of the C
oracle (a dropped term, a wrong sign, a swapped operation order, a transposed
operand) each make at least one pin fail.  Mutants are built on the CPU in a
temporary directory; the committed oracle is never modified.
"""
import ctypes
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from oracle import brute

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

MUTANTS = {
    "erase_sign": ("u[j] = beta * (vj - u[j]);", "u[j] = beta * (vj + u[j]);"),
    "no_forget": ("for (int j = 0; j < ncol; ++j) row[j] *= a;", "(void)a;"),
    "decay_sign": ("double a = exp(load_elt(gate_dtype(dtype), g, goff + c));",
                   "double a = exp(-load_elt(gate_dtype(dtype), g, goff + c));"),
    "no_scale": ("double o = scale * yrow[j];", "double o = yrow[j];"),
    "gate_sign": ("if (z) o *= sigmoid(load_elt(dtype, z, zoff + j));",
                  "if (z) o *= sigmoid(-load_elt(dtype, z, zoff + j));"),
    "output_before_write": (
        "        token_step(dtype, dk, dv, S, k, th * dk, v, th * dv, g, th * dk,\n"
        "                   load_elt(gate_dtype(dtype), beta, th), u);\n"
        "        if (y) token_output(dtype, dk, dv, S, q, th * dk, z, th * dv, scale, y + th * dv);",
        "        if (y) token_output(dtype, dk, dv, S, q, th * dk, z, th * dv, scale, y + th * dv);\n"
        "        token_step(dtype, dk, dv, S, k, th * dk, v, th * dv, g, th * dk,\n"
        "                   load_elt(gate_dtype(dtype), beta, th), u);"),
    "f64_read_as_f32": ("    if (dtype == KDAO_F64) return ((const double*)base)[i];\n", ""),
    "compose_transposed": ("acc += M2[(int64_t)i * dk + c] * S1[(int64_t)c * dv + j];",
                           "acc += M2[(int64_t)c * dk + i] * S1[(int64_t)c * dv + j];"),
    "scan_drops_local": ("nxt[(int64_t)r * dv + j] = acc + Li[(int64_t)r * dv + j];",
                         "nxt[(int64_t)r * dv + j] = acc;"),
    "bf16_widen": ("uint32_t u = ((uint32_t)((const uint16_t*)base)[i]) << 16;",
                   "uint32_t u = ((uint32_t)((const uint16_t*)base)[i]) << 15;"),
    "erase_uses_query": ("        double kc = load_elt(dtype, k, koff + c);\n        const double* row = X + (int64_t)c * ncol;\n        for (int j = 0; j < ncol; ++j) u[j] += kc * row[j];",
                         "        double kc = load_elt(dtype, k, koff + (c + 1) % dk);\n        const double* row = X + (int64_t)c * ncol;\n        for (int j = 0; j < ncol; ++j) u[j] += kc * row[j];"),
}


def _pins_pass() -> bool:
    """A compact run of the pins against whatever library oracle._lib holds."""
    try:
        for dtype in ("f32", "bf16"):
            inp = kda_inputs.make_prefill([23, 9], 2, 8, 5, dtype, True, 0.3, 7, -1.0, 0.0)
            y, st = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens,
                                      z=inp.z, S_init=inp.S0, scale=0.5)
            cu = inp.cu_seqlens.tolist()
            for n in range(2):
                for h in range(2):
                    sl = slice(cu[n], cu[n + 1])
                    yb, Sb = brute.sequence(inp.q[sl, h], inp.k[sl, h], inp.v[sl, h],
                                            inp.g[sl, h], inp.beta[sl, h], inp.z[sl, h],
                                            inp.S0[n, h], 0.5)
                    if not (np.allclose(y[sl, h], yb, rtol=0, atol=1e-12)
                            and np.allclose(st[n * 2 + h], Sb, rtol=0, atol=1e-12)):
                        return False
        inp = kda_inputs.make_prefill([64], 1, 8, 6, "f32", False, 0.0, 9, 6.0, 2.0)
        parts = oracle.kcp(inp.q, inp.k, inp.v, inp.g, inp.beta, [0, 25, 64], want_pairs=True)
        whole = oracle.kcp(inp.q, inp.k, inp.v, inp.g, inp.beta, [0, 64], want_pairs=True)
        Mc, Sc = oracle.compose(parts["M"][1, 0], parts["Sloc"][1, 0], parts["M"][0, 0],
                                parts["Sloc"][0, 0])
        if not (np.allclose(Mc, whole["M"][0, 0], atol=1e-13)
                and np.allclose(Sc, whole["Sloc"][0, 0], atol=1e-13)):
            return False
        _, st = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, [0, 64], want_y=False)
        if not np.allclose(parts["final"], st, atol=1e-13):
            return False
        return _fused_pins_pass()
    except ValueError:
        return False


def _fused_pins_pass() -> bool:
    """The fused input step: against brute force with its own gate step, and
    sigmoid(0) = 1/2."""
    raw = kda_inputs.make_raw_prefill([11, 6], 2, 6, 4, "bf16", True, 0.3, 61, -1.0, 0.0)
    y, st = oracle.recurrence_fused(raw.q, raw.k, raw.v, raw.a, raw.b, raw.cu_seqlens, z=raw.z,
                                    S_init=raw.S0, scale=0.6)
    cu = raw.cu_seqlens.tolist()
    for n in range(2):
        for h in range(2):
            sl = slice(cu[n], cu[n + 1])
            yb, Sb = brute.fused_sequence(raw.q[sl, h], raw.k[sl, h], raw.v[sl, h], raw.a[sl, h],
                                          raw.b[sl, h], raw.z[sl, h], raw.S0[n, h], 0.6)
            if not (np.allclose(y[sl, h], yb, rtol=0, atol=1e-12)
                    and np.allclose(st[n * 2 + h], Sb, rtol=0, atol=1e-12)):
                return False
    z1 = torch.zeros(1, 1, 2)
    _, _, g, beta = oracle.gates(z1 + 1, z1 + 1, z1, torch.zeros(1, 1))
    return bool((g == -2.5).all()) and bool((beta == 0.5).all())


# mistakes planted in the fused input step (oracle.gates, Python)
GATE_MUTANTS = {
    "norm_without_sqrt": ("qh = qd / torch.sqrt((qd * qd).sum(-1, keepdim=True) + eps)",
                          "qh = qd / ((qd * qd).sum(-1, keepdim=True) + eps)"),
    "norm_over_heads": ("kh = kd / torch.sqrt((kd * kd).sum(-1, keepdim=True) + eps)",
                        "kh = kd / torch.sqrt((kd * kd).sum(-2, keepdim=True) + eps)"),
    "q_left_raw": ("qh = qd / torch.sqrt((qd * qd).sum(-1, keepdim=True) + eps)", "qh = qd"),
    "decay_gate_flipped": ("(G_MIN * sig(ad))", "(G_MIN * sig(-ad))"),
    "decay_bound_sign": ("(G_MIN * sig(ad))", "(-G_MIN * sig(ad))"),
    "beta_unsquashed": ("sig(bd).contiguous()", "bd.contiguous()"),
}


@pytest.mark.parametrize("name", sorted(GATE_MUTANTS))
def test_planted_gate_mistake_is_caught(name, oracle_mod, monkeypatch):
    import inspect
    import textwrap
    src = textwrap.dedent(inspect.getsource(oracle.gates))
    old, new = GATE_MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    ns = dict(vars(oracle))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    monkeypatch.setattr(oracle, "gates", ns["gates"])
    assert not _fused_pins_pass(), f"mutant {name} slipped through the pins"


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="kdao_mut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_unmutated_oracle_passes_the_compact_pins(oracle_mod):
    assert _pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, workdir, oracle_mod, monkeypatch):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path_c = os.path.join(workdir, f"{name}.c")
    path_so = os.path.join(workdir, f"{name}.so")
    open(path_c, "w").write(src.replace(old, new))
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", path_so,
                    path_c, "-lm"], check=True)
    real = oracle._load()
    mut = ctypes.CDLL(path_so)
    for fn in ("kdao_recurrence", "kdao_kcp", "kdao_compose", "kdao_max_threads"):
        getattr(mut, fn).argtypes = getattr(real, fn).argtypes
        getattr(mut, fn).restype = getattr(real, fn).restype
    monkeypatch.setattr(oracle, "_lib", mut)
    assert not _pins_pass(), f"mutant {name} slipped through the pins"
