"""Seeded synthetic inputs for the KDA recurrence.

This module is shared by the fp64 oracle tests, the HIP parity tests and the
benchmark.  It holds no arithmetic of the recurrence itself: it only draws
random tensors, L2-normalises q and k (a precondition of the method, page
"Exercices", Niveau 2 Q9), squashes the gate pre-activations into their
ranges (beta in (0,1); log-decay g = g_min * sigmoid(x) in (g_min, 0), with
g_min = -5 from page "Exercices", Niveau 2 Q8 and the "gate_lower_bound"
entry of page "Ce qui est public et ce qui ne l'est pas") and casts to the
storage dtype.

Recipe (fixed draw order, one torch CPU generator per workload):
    lengths (varlen only), q, k, v, z (gated only), beta pre-activation,
    g pre-activation, initial state (if any).
All draws are i.i.d. N(0, 1) except the initial state (N(0, std)) and the
accepted draft lengths of a replay (uniform integers).  q and k are
normalised per (token, head) in fp32, then q, k, v, z are rounded to the
storage dtype (bf16 by round-to-nearest-even, or kept fp32).  beta and g stay
fp32.  Decode pools draw P independent token sets after the state.

Raw inputs of the fused input step (make_raw_prefill, make_raw_decode) are the
same draws, in the same order, left unprocessed: q and k not normalised, and
the pre-activations a = x - g_shift (decay) and b = x - beta_shift (beta),
all rounded to the storage dtype.

Shapes (token-major, channel fastest):
    q, k: [T, H, dk]   v, z: [T, H, dv]   g: [T, H, dk] fp32   beta: [T, H] fp32
    cu_seqlens: [N + 1] int32   S0: [N, H, dk, dv] fp32
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import torch

G_MIN = -5.0

# The five workloads: the K3 KDA layer shape is 96 heads of dimension 128
# (page "Retrouver les 2,8 T de paramètres", "Les constantes de départ":
# kda_H = 96, kda_hd = 128).
WORKLOADS = {
    0: dict(name="tiny_prefill_fp32", kind="prefill", H=2, dk=64, dv=64, lens=[256],
            dtype="f32", chunk=16, gated=False, s0_std=0.0),
    1: dict(name="k3_layer_prefill", kind="prefill", H=96, dk=128, dv=128, lens=[8192],
            dtype="bf16", chunk=64, gated=True, s0_std=0.0),
    2: dict(name="varlen_prefill", kind="prefill", H=96, dk=128, dv=128, lens="uniform",
            nseq=16, lmin=512, lmax=8192, dtype="bf16", chunk=64, gated=True, s0_std=0.02),
    3: dict(name="kcp_long_sequence", kind="kcp", H=4, dk=128, dv=128, lens=[1 << 20],
            segments=256, dtype="bf16", chunk=64, gated=False, s0_std=0.0),
    4: dict(name="decode", kind="decode", H=96, dk=128, dv=128, N=128, pool=16, steps=1000,
            dtype="bf16", gated=True, s0_std=0.02),
}

# Pre-activation shifts of the long-memory stress variants: g = g_min *
# sigmoid(x - g_shift), beta = sigmoid(x - beta_shift).  "chunk" keeps about
# 84 % of the state over 64 tokens; "segment" keeps most of it over thousands.
STRESS = {
    None: (0.0, 0.0),
    "chunk": (8.0, 4.0),
    "segment": (12.0, 8.0),
}


@dataclasses.dataclass
class KDAInputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    z: Optional[torch.Tensor]
    g: torch.Tensor
    beta: torch.Tensor
    cu_seqlens: torch.Tensor
    S0: Optional[torch.Tensor]
    H: int
    dk: int
    dv: int
    dtype: str

    @property
    def T(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_seqs(self) -> int:
        return int(self.cu_seqlens.numel() - 1)

    def lengths(self) -> List[int]:
        c = self.cu_seqlens.tolist()
        return [c[i + 1] - c[i] for i in range(len(c) - 1)]


def _tdtype(dtype: str) -> torch.dtype:
    if dtype == "bf16":
        return torch.bfloat16
    if dtype == "f32":
        return torch.float32
    raise ValueError(f"unknown dtype {dtype!r}")


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


def draw_tokens(gen: torch.Generator, shape_prefix, H: int, dk: int, dv: int, dtype: str,
                gated: bool, g_shift: float = 0.0, beta_shift: float = 0.0):
    """Draw q, k, v, z, beta, g for a block of tokens of shape shape_prefix + [H, .]."""
    sp = tuple(shape_prefix)
    td = _tdtype(dtype)
    q = _unit(torch.randn(*sp, H, dk, generator=gen)).to(td)
    k = _unit(torch.randn(*sp, H, dk, generator=gen)).to(td)
    v = torch.randn(*sp, H, dv, generator=gen).to(td)
    z = torch.randn(*sp, H, dv, generator=gen).to(td) if gated else None
    beta = torch.sigmoid(torch.randn(*sp, H, generator=gen) - beta_shift)
    g = G_MIN * torch.sigmoid(torch.randn(*sp, H, dk, generator=gen) - g_shift)
    return q, k, v, z, beta.contiguous(), g.contiguous()


def make_prefill(lens: List[int], H: int, dk: int, dv: int, dtype: str, gated: bool,
                 s0_std: float, seed: int, g_shift: float = 0.0,
                 beta_shift: float = 0.0, gen: Optional[torch.Generator] = None) -> KDAInputs:
    """Packed varlen prefill inputs for sequences of the given lengths."""
    if gen is None:
        gen = torch.Generator().manual_seed(seed)
    lens = [int(x) for x in lens]
    cu = torch.zeros(len(lens) + 1, dtype=torch.int32)
    if lens:
        cu[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0).to(torch.int32)
    T = int(cu[-1])
    q, k, v, z, beta, g = draw_tokens(gen, [T], H, dk, dv, dtype, gated, g_shift, beta_shift)
    S0 = None
    if s0_std > 0:
        S0 = (torch.randn(len(lens), H, dk, dv, generator=gen) * s0_std).contiguous()
    return KDAInputs(q, k, v, z, g, beta, cu, S0, H, dk, dv, dtype)


def workload_seed(wid: int, stress: Optional[str] = None) -> int:
    return (2000 if stress else 1000) + wid


def make_workload(wid: int, stress: Optional[str] = None, **override) -> KDAInputs:
    """Inputs of prefill/KCP workload `wid` (optionally a stress variant).

    `override` may shrink sizes (e.g. T, H, lens) for fast tests; it keeps the
    distributions.
    """
    w = dict(WORKLOADS[wid])
    w.update(override)
    if w["kind"] == "decode":
        raise ValueError("use make_decode for the decode workload")
    g_shift, beta_shift = STRESS[stress]
    seed = override.get("seed", workload_seed(wid, stress))
    gen = torch.Generator().manual_seed(seed)
    if w["lens"] == "uniform":
        lens = torch.randint(w["lmin"], w["lmax"] + 1, (w["nseq"],), generator=gen).tolist()
    else:
        lens = list(w["lens"])
    return make_prefill(lens, w["H"], w["dk"], w["dv"], w["dtype"], w["gated"], w["s0_std"],
                        seed, g_shift, beta_shift, gen=gen)


@dataclasses.dataclass
class DecodeInputs:
    """P pooled single-token input sets for N requests; step s uses set s % P."""
    q: torch.Tensor      # [P, N, H, dk]
    k: torch.Tensor
    v: torch.Tensor      # [P, N, H, dv]
    z: Optional[torch.Tensor]
    g: torch.Tensor      # [P, N, H, dk] fp32
    beta: torch.Tensor   # [P, N, H] fp32
    S0: torch.Tensor     # [N, H, dk, dv] fp32
    N: int
    H: int
    dk: int
    dv: int
    dtype: str


def make_decode(N: int, H: int, dk: int, dv: int, dtype: str, gated: bool, s0_std: float,
                pool: int, seed: int, g_shift: float = 0.0, beta_shift: float = 0.0) -> DecodeInputs:
    gen = torch.Generator().manual_seed(seed)
    S0 = (torch.randn(N, H, dk, dv, generator=gen) * s0_std).contiguous()
    q, k, v, z, beta, g = draw_tokens(gen, [pool, N], H, dk, dv, dtype, gated, g_shift, beta_shift)
    return DecodeInputs(q, k, v, z, g, beta, S0, N, H, dk, dv, dtype)


def make_decode_workload(stress: Optional[str] = None, **override) -> DecodeInputs:
    w = dict(WORKLOADS[4])
    w.update(override)
    g_shift, beta_shift = STRESS[stress]
    seed = override.get("seed", workload_seed(4, stress))
    return make_decode(w["N"], w["H"], w["dk"], w["dv"], w["dtype"], w["gated"], w["s0_std"],
                       w["pool"], seed, g_shift, beta_shift)


@dataclasses.dataclass
class ReplayInputs:
    """Draft tokens of speculative decoding: Td tokens per request against the
    resident states, plus the accepted prefix length of each request."""
    q: torch.Tensor        # [N, Td, H, dk]
    k: torch.Tensor
    v: torch.Tensor        # [N, Td, H, dv]
    z: Optional[torch.Tensor]
    g: torch.Tensor        # [N, Td, H, dk] fp32
    beta: torch.Tensor     # [N, Td, H] fp32
    S0: torch.Tensor       # [N, H, dk, dv] fp32
    accepted: torch.Tensor  # [N] int32 in [0, Td]
    N: int
    Td: int
    H: int
    dk: int
    dv: int
    dtype: str


def make_replay(N: int, Td: int, H: int, dk: int, dv: int, dtype: str, gated: bool,
                s0_std: float, seed: int, g_shift: float = 0.0,
                beta_shift: float = 0.0) -> ReplayInputs:
    """Draw order: state, draft tokens ([N, Td] prefix), accepted lengths
    (uniform integers in [0, Td])."""
    gen = torch.Generator().manual_seed(seed)
    S0 = (torch.randn(N, H, dk, dv, generator=gen) * s0_std).contiguous()
    q, k, v, z, beta, g = draw_tokens(gen, [N, Td], H, dk, dv, dtype, gated, g_shift, beta_shift)
    acc = torch.randint(0, Td + 1, (N,), generator=gen).to(torch.int32)
    return ReplayInputs(q, k, v, z, g, beta, S0, acc, N, Td, H, dk, dv, dtype)


def draw_on_device(lens: List[int], H: int, dk: int, dv: int, gated: bool, s0_std: float,
                   seed: int, device, g_shift: float = 0.0, beta_shift: float = 0.0) -> KDAInputs:
    """The same recipe (distributions, draw order) drawn by a torch generator on
    `device`, for workloads too large to draw on the host quickly.  bf16 storage.
    Not bit-identical to make_prefill (different generator); tests copy the
    sampled chains back to the host for the oracle."""
    gen = torch.Generator(device=device).manual_seed(seed)
    T = int(sum(lens))
    dt = torch.bfloat16

    def unit(x):
        return x / x.norm(dim=-1, keepdim=True)

    q = unit(torch.randn(T, H, dk, generator=gen, device=device)).to(dt)
    k = unit(torch.randn(T, H, dk, generator=gen, device=device)).to(dt)
    v = torch.randn(T, H, dv, generator=gen, device=device).to(dt)
    z = torch.randn(T, H, dv, generator=gen, device=device).to(dt) if gated else None
    beta = torch.sigmoid(torch.randn(T, H, generator=gen, device=device) - beta_shift)
    g = G_MIN * torch.sigmoid(torch.randn(T, H, dk, generator=gen, device=device) - g_shift)
    S0 = None
    if s0_std > 0:
        S0 = torch.randn(len(lens), H, dk, dv, generator=gen, device=device) * s0_std
    cu = torch.zeros(len(lens) + 1, dtype=torch.int32)
    if lens:
        cu[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0).to(torch.int32)
    return KDAInputs(q, k, v, z, g, beta, cu, S0, H, dk, dv, "bf16")


@dataclasses.dataclass
class RawInputs:
    """Inputs of the fused input step, in the storage dtype: q, k before
    normalisation, a the decay pre-activation (per key channel), b the beta
    pre-activation (per token and head).  Token shapes as in KDAInputs, with a
    leading [P] (decode steps) or a packed [T] token axis."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    z: Optional[torch.Tensor]
    a: torch.Tensor
    b: torch.Tensor
    cu_seqlens: Optional[torch.Tensor]
    S0: Optional[torch.Tensor]
    H: int
    dk: int
    dv: int
    dtype: str


def draw_raw_tokens(gen: torch.Generator, shape_prefix, H: int, dk: int, dv: int, dtype: str,
                    gated: bool, g_shift: float = 0.0, beta_shift: float = 0.0):
    """The draws of draw_tokens, unprocessed: (q, k, v, z, b, a) in the storage dtype."""
    sp = tuple(shape_prefix)
    td = _tdtype(dtype)
    q = torch.randn(*sp, H, dk, generator=gen).to(td)
    k = torch.randn(*sp, H, dk, generator=gen).to(td)
    v = torch.randn(*sp, H, dv, generator=gen).to(td)
    z = torch.randn(*sp, H, dv, generator=gen).to(td) if gated else None
    b = (torch.randn(*sp, H, generator=gen) - beta_shift).to(td)
    a = (torch.randn(*sp, H, dk, generator=gen) - g_shift).to(td)
    return q, k, v, z, b.contiguous(), a.contiguous()


def make_raw_prefill(lens: List[int], H: int, dk: int, dv: int, dtype: str, gated: bool,
                     s0_std: float, seed: int, g_shift: float = 0.0,
                     beta_shift: float = 0.0) -> RawInputs:
    """Packed prefill inputs for the fused input step (draw order of make_prefill)."""
    gen = torch.Generator().manual_seed(seed)
    lens = [int(x) for x in lens]
    cu = torch.zeros(len(lens) + 1, dtype=torch.int32)
    if lens:
        cu[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0).to(torch.int32)
    T = int(cu[-1])
    q, k, v, z, b, a = draw_raw_tokens(gen, [T], H, dk, dv, dtype, gated, g_shift, beta_shift)
    S0 = None
    if s0_std > 0:
        S0 = (torch.randn(len(lens), H, dk, dv, generator=gen) * s0_std).contiguous()
    return RawInputs(q, k, v, z, a, b, cu, S0, H, dk, dv, dtype)


def make_raw_decode(N: int, H: int, dk: int, dv: int, dtype: str, gated: bool, s0_std: float,
                    steps: int, seed: int, g_shift: float = 0.0,
                    beta_shift: float = 0.0) -> RawInputs:
    """`steps` single-token input sets [steps, N, H, .] for the fused decode
    step, after the state (draw order of make_decode)."""
    gen = torch.Generator().manual_seed(seed)
    S0 = (torch.randn(N, H, dk, dv, generator=gen) * s0_std).contiguous()
    q, k, v, z, b, a = draw_raw_tokens(gen, [steps, N], H, dk, dv, dtype, gated, g_shift, beta_shift)
    return RawInputs(q, k, v, z, a, b, None, S0, H, dk, dv, dtype)


def varlen_lengths(seed: Optional[int] = None) -> List[int]:
    """The varlen workload's sequence lengths (first draw of its generator)."""
    w = WORKLOADS[2]
    gen = torch.Generator().manual_seed(workload_seed(2) if seed is None else seed)
    return torch.randint(w["lmin"], w["lmax"] + 1, (w["nseq"],), generator=gen).tolist()
