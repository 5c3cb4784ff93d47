"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and rejects bad arguments before launching anything."""
import ctypes
import math
import os
import re

import pytest

import gated_delta_rule_75_amd as kda

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "kda.h")
OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3
BF16, F32 = kda.KDA_BF16, kda.KDA_F32
P = ctypes.c_void_p(1 << 20)          # a fake, aligned, never dereferenced address


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return kda.lib()


def test_header_declares_what_the_binding_knows():
    assert declared_symbols() == sorted(kda.SYMBOLS)


def test_library_exports_every_declared_symbol(L):
    for name in declared_symbols():
        assert hasattr(L, name), name
    assert L.kda_version() == 10100
    assert kda.kda_status_string(0) == "KDA_OK"
    assert kda.kda_status_string(3) == "KDA_ERR_WORKSPACE_TOO_SMALL"
    assert kda.kda_status_string(99) == "KDA_ERR_UNKNOWN"


def _fwd(L, dt=BF16, H=2, dk=128, dv=128, chunk=64, N=1, T=64, cu=None, q=P, k=P, v=P, g=P,
         beta=P, z=None, s0=None, sf=None, y=P, ws=P, wsb=1 << 40):
    return L.kda_chunk_fwd(dt, H, dk, dv, chunk, 1.0, N, T, cu, q, k, v, g, beta, z, s0, sf, y,
                           ws, wsb, None)


def test_chunk_fwd_rejects_bad_arguments(L):
    assert _fwd(L, dt=7) == INVALID
    assert _fwd(L, H=0) == INVALID
    assert _fwd(L, N=0) == INVALID
    assert _fwd(L, T=-1) == INVALID
    assert _fwd(L, N=2, cu=None) == INVALID                      # several sequences need offsets
    assert _fwd(L, q=None) == INVALID
    assert _fwd(L, y=None) == INVALID
    assert _fwd(L, beta=None) == INVALID
    assert _fwd(L, q=ctypes.c_void_p((1 << 20) + 4)) == INVALID  # bf16 runs of 4 need 8-byte alignment
    assert _fwd(L, dt=F32, v=ctypes.c_void_p((1 << 20) + 8)) == INVALID  # fp32 runs of 4: 16 bytes
    assert _fwd(L, g=ctypes.c_void_p((1 << 20) + 8)) == INVALID  # g in runs of 4: 16 bytes
    assert _fwd(L, s0=ctypes.c_void_p((1 << 20) + 8)) == INVALID # states need 16-byte alignment
    assert _fwd(L, ws=None) == INVALID
    assert _fwd(L, ws=ctypes.c_void_p((1 << 20) + 128)) == INVALID  # workspace: 256 bytes
    least = L.kda_chunk_fwd_workspace_min(BF16, 2, 128, 128, 64, 1, 64)
    assert 0 < least <= L.kda_chunk_fwd_workspace_size(BF16, 2, 128, 128, 64, 1, 64)
    assert _fwd(L, wsb=least - 1) == WS_SMALL


def test_chunk_fwd_checkpointed_rejects_bad_arguments(L):
    def ck(interval=128, cap=64, ckpt=P, offs=P, chunk=64, T=8192):
        return L.kda_chunk_fwd_checkpointed(BF16, 2, 128, 128, chunk, 1.0, 1, T, None, P, P, P, P,
                                            P, None, None, None, P, interval, ckpt, offs, cap, P,
                                            1 << 40, None)
    assert ck(interval=0) == INVALID
    assert ck(interval=-64) == INVALID
    assert ck(interval=96) == INVALID              # not a multiple of the chunk
    assert ck(cap=63) == INVALID                   # fewer rows than T / interval
    assert ck(offs=None) == INVALID
    assert ck(ckpt=None) == INVALID
    assert ck(ckpt=ctypes.c_void_p((1 << 20) + 8)) == INVALID


def test_chunk_fwd_rejects_unsupported_shapes(L):
    assert _fwd(L, dk=96, dv=96) == UNSUPPORTED
    assert _fwd(L, dk=128, dv=64) == UNSUPPORTED
    assert _fwd(L, chunk=48) == UNSUPPORTED
    assert _fwd(L, chunk=128) == UNSUPPORTED


def _pm_frags(C, kb):
    """Fragments (16 tokens x one k-block of kb tokens) of P on or below its diagonal."""
    return sum(1 for ta in range(C // 16) for u in range(-(-C // kb)) if u * kb <= 16 * ta + 15)


def _chunk_block_bytes(elt, dk, dv, C, CP):
    """Bytes of the chunk products of one (chunk, head): Wn, Qt [C, dk], Kh^T [dk, CP]
    in the input dtype, the 1 KiB fragments of Pm and of L^-1 diag(beta) on or
    below the diagonal, and gam [dk] fp32 (no C x dv product: U is formed from v
    by the state pass)."""
    kb = 32 if elt == 2 else 16
    return (2 * C * dk + dk * CP) * elt + 2 * _pm_frags(C, kb) * 1024 + dk * 4


def _rnd(x):
    return (x + 255) // 256 * 256


def test_chunk_fwd_workspace_size(L):
    H, dk, dv, C, N, T = 96, 128, 128, 64, 1, 8192
    nb = (T // C + N) * H
    parts = [N + 1, N]   # chunk offsets and order, int32
    parts = [_rnd(4 * x) for x in parts]
    for n in (C * dk, C * dk, dk * C, _pm_frags(C, 32) * 512, _pm_frags(C, 32) * 512):
        parts.append(_rnd(nb * n * 2))
    parts.append(_rnd(nb * dk * 4))
    assert L.kda_chunk_fwd_workspace_size(BF16, H, dk, dv, C, N, T) == sum(parts)
    # per (chunk, head) 60.5 KiB at this shape: 6 of the 8 fragments of P (and of
    # L^-1 diag(beta)) are stored
    assert _pm_frags(64, 32) == 6
    assert _chunk_block_bytes(2, dk, dv, C, C) == 61952
    # bf16 k-blocks are 32 tokens: chunk 16 pads K^T and P to 32 columns
    small = L.kda_chunk_fwd_workspace_size(BF16, 1, 64, 64, 16, 1, 16)
    assert small >= 2 * _chunk_block_bytes(2, 64, 64, 16, 32)
    assert L.kda_chunk_fwd_workspace_size(BF16, H, 96, 96, C, N, T) == 0
    assert L.kda_chunk_fwd_workspace_size(BF16, 0, dk, dv, C, N, T) == 0
    assert L.kda_chunk_fwd_workspace_size(BF16, H, dk, dv, 48, N, T) == 0


def test_kcp_workspace_size(L):
    H, dk, dv, S, T, C = 4, 128, 128, 256, 1 << 20, 64
    pairs = S * H * dk * (dk + dv) * 4
    starts = S * H * dk * dv * 4
    # the scan of the pairs goes through G groups of ceil(sqrt(S)) segments
    Lg = math.isqrt(S - 1) + 1
    G = -(-S // Lg)
    assert (Lg, G) == (16, 16)
    groups = G * H * dk * (dk + dv) * 4 + G * H * dk * dv * 4
    need = L.kda_kcp_workspace_size(BF16, H, dk, dv, C, T, S)
    nb = S * (T // S // C) * H
    base = pairs + starts + groups + nb * _chunk_block_bytes(2, dk, dv, C, C)
    assert base <= need <= base + 16 * 256 + 8 * S
    assert L.kda_kcp_workspace_size(BF16, H, 96, 96, C, T, S) == 0
    assert L.kda_kcp_workspace_size(BF16, 0, dk, dv, C, T, S) == 0
    assert L.kda_kcp_workspace_size(BF16, H, dk, dv, C, T, 0) == 0


def test_workspace_minimum_does_not_grow_with_T(L):
    """The smallest workspaces hold one chunk per head beside what does not
    depend on the length: the carried states (prefill) or the segment pairs and
    entering states (KCP)."""
    H, dk, dv, C = 96, 128, 128, 64
    one = _chunk_block_bytes(2, dk, dv, C, C) * H
    for N, T in ((1, 8192), (1, 1 << 20), (16, 89000)):
        least = L.kda_chunk_fwd_workspace_min(BF16, H, dk, dv, C, N, T)
        carry = N * H * dk * dv * 4
        assert carry + one <= least <= carry + one + 8 * 256 + 8 * N
        assert least < L.kda_chunk_fwd_workspace_size(BF16, H, dk, dv, C, N, T)
    # a call whose full workspace is one chunk per head needs no carry
    assert L.kda_chunk_fwd_workspace_min(BF16, 2, 64, 64, 64, 1, 10) == \
        L.kda_chunk_fwd_workspace_size(BF16, 2, 64, 64, 64, 1, 10)
    assert L.kda_chunk_fwd_workspace_min(BF16, 0, dk, dv, C, 1, 64) == 0
    # KCP at one 1M-token sequence, 4 heads, 256 segments: about 201 MB + one chunk per head
    S, T = 256, 1 << 20
    fixed = S * 4 * dk * (dk + dv) * 4 + S * 4 * dk * dv * 4 + 16 * 4 * dk * (dk + dv) * 4 + 16 * 4 * dk * dv * 4
    least = L.kda_kcp_workspace_min(BF16, 4, dk, dv, C, T, S)
    assert fixed + 4 * _chunk_block_bytes(2, dk, dv, C, C) <= least <= fixed + 4 * _chunk_block_bytes(2, dk, dv, C, C) + 4096
    assert least == L.kda_kcp_workspace_min(BF16, 4, dk, dv, C, 4 * T, S)
    assert L.kda_kcp_workspace_min(BF16, 4, dk, dv, C, T, 0) == 0


def _kcp(L, T=4096, S=4, ws=P, wsb=1 << 40, dk=128, chunk=64, dt=BF16, y=P):
    return L.kda_kcp_scan(dt, 2, dk, dk, chunk, 1.0, T, S, P, P, P, P, P, None, None, None, y,
                          ws, wsb, None)


def test_kcp_rejects_bad_arguments(L):
    assert _kcp(L, S=0) == INVALID
    assert _kcp(L, T=3, S=4) == INVALID
    assert _kcp(L, ws=None) == INVALID
    assert _kcp(L, ws=ctypes.c_void_p((1 << 20) + 128)) == INVALID   # 256-byte alignment
    assert _kcp(L, y=None) == INVALID
    assert _kcp(L, dk=96) == UNSUPPORTED
    assert _kcp(L, chunk=8) == UNSUPPORTED
    least = L.kda_kcp_workspace_min(BF16, 2, 128, 128, 64, 4096, 4)
    assert 0 < least < L.kda_kcp_workspace_size(BF16, 2, 128, 128, 64, 4096, 4)
    assert _kcp(L, wsb=least - 1) == WS_SMALL


def test_decode_rejects_bad_arguments(L):
    def dec(dt=BF16, N=4, H=2, dk=128, dv=128, state=P, y=P, q=P):
        return L.kda_decode_step(dt, N, H, dk, dv, 1.0, q, P, P, P, P, None, state, y, None)
    assert dec(N=-1) == INVALID
    assert dec(H=0) == INVALID
    assert dec(dt=5) == INVALID
    assert dec(state=None) == INVALID
    assert dec(q=None) == INVALID
    assert dec(state=ctypes.c_void_p((1 << 20) + 4)) == INVALID
    assert dec(dk=128, dv=64) == UNSUPPORTED


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(4, 1, 64)
    with pytest.raises(ValueError):
        kda.chunk_fwd(q, q, q, q, torch.zeros(4, 1))


def test_decode_replay_rejects_bad_arguments(L):
    def rp(dt=BF16, N=4, Td=3, H=2, dk=128, dv=128, acc=P, state=P, y=P, q=P):
        return L.kda_decode_replay(dt, N, Td, H, dk, dv, 1.0, q, P, P, P, P, None, acc, state, y,
                                   None)
    assert rp(Td=0) == INVALID
    assert rp(N=-1) == INVALID
    assert rp(acc=None, y=None) == INVALID        # nothing to produce
    assert rp(state=None) == INVALID
    assert rp(q=None) == INVALID
    assert rp(acc=ctypes.c_void_p((1 << 20) + 2)) == INVALID
    assert rp(dk=96, dv=96) == UNSUPPORTED
    assert rp(N=0) == OK                          # no requests: nothing launched


def test_fused_entry_points_reject_bad_arguments(L):
    def fw(dt=BF16, a=P, b=P, q=P, dk=128, chunk=64, ws=P):
        return L.kda_chunk_fwd_fused(dt, 2, dk, dk, chunk, 1.0, 1, 64, None, q, P, P, a, b, None,
                                     None, None, P, ws, 1 << 40, None)
    assert fw(dt=9) == INVALID
    assert fw(a=None) == INVALID
    assert fw(b=None) == INVALID
    assert fw(a=ctypes.c_void_p((1 << 20) + 4)) == INVALID            # a in runs of 4 bf16: 8 bytes
    assert fw(dt=F32, a=ctypes.c_void_p((1 << 20) + 8)) == INVALID    # fp32 runs of 4: 16 bytes
    assert fw(b=ctypes.c_void_p((1 << 20) + 1)) == INVALID            # b: one element
    assert fw(dt=F32, b=ctypes.c_void_p((1 << 20) + 2)) == INVALID
    assert fw(ws=None) == INVALID
    assert fw(dk=96) == UNSUPPORTED
    assert fw(chunk=48) == UNSUPPORTED

    def dec(dt=BF16, a=P, b=P, N=4, dk=128):
        return L.kda_decode_step_fused(dt, N, 2, dk, dk, 1.0, P, P, P, a, b, None, P, P, None)
    assert dec(a=None) == INVALID
    assert dec(b=ctypes.c_void_p((1 << 20) + 1)) == INVALID
    assert dec(dt=F32, a=ctypes.c_void_p((1 << 20) + 2)) == INVALID
    assert dec(N=-1) == INVALID
    assert dec(dk=96) == UNSUPPORTED
    assert dec(N=0) == OK                                              # nothing launched


def test_binding_checks_fused_dtypes():
    import torch
    q = torch.zeros(4, 1, 64)
    with pytest.raises(TypeError):    # a must have q's dtype, not fp32 g beside bf16 q
        kda._check_inputs(q.bfloat16(), q.bfloat16(), q.bfloat16(), q, torch.zeros(4, 1).bfloat16(),
                          None, fused=True)


def _cpu_prefill(T=8, H=2, d=64, dt=None):
    import torch
    dt = dt or torch.bfloat16
    q = torch.zeros(T, H, d, dtype=dt)
    return dict(q=q, k=q.clone(), v=q.clone(), g=torch.zeros(T, H, d), beta=torch.zeros(T, H))


@pytest.mark.parametrize("name,bad,exc", [
    ("y", dict(shape=(8, 2, 32)), ValueError),                   # too few value channels
    ("y", dict(shape=(7, 2, 64)), ValueError),                   # too few tokens
    ("y", dict(dtype="f32"), TypeError),                         # fp32 y beside bf16 inputs
    ("final_state", dict(shape=(1, 2, 64, 32)), ValueError),
    ("final_state", dict(dtype="bf16", shape=(1, 2, 64, 64)), TypeError),
    ("initial_state", dict(shape=(2, 2, 64, 64)), ValueError),   # one sequence, two states
    ("workspace", dict(dtype="f32", shape=(1024,)), TypeError),
    ("workspace", dict(shape=(4, 256)), TypeError),
])
def test_binding_refuses_wrong_buffers_for_chunk_fwd(name, bad, exc):
    """Buffers the caller passes are checked for shape and dtype before the
    call: an undersized y or state would be written out of bounds."""
    import torch
    x = _cpu_prefill()
    dts = {"f32": torch.float32, "bf16": torch.bfloat16}
    default = {"y": ((8, 2, 64), torch.bfloat16), "final_state": ((1, 2, 64, 64), torch.float32),
               "initial_state": ((1, 2, 64, 64), torch.float32), "workspace": ((1024,), torch.uint8)}
    shape, dtype = default[name]
    t = torch.zeros(bad.get("shape", shape), dtype=dts.get(bad.get("dtype"), dtype))
    with pytest.raises(exc):
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], **{name: t})


def test_binding_refuses_wrong_buffers_elsewhere():
    import torch
    x = _cpu_prefill()
    with pytest.raises(ValueError):      # kcp states are [1, H, dk, dv]
        kda.kcp_scan(x["q"], x["k"], x["v"], x["g"], x["beta"], 2,
                     initial_state=torch.zeros(2, 64, 64))
    with pytest.raises(ValueError):
        kda.kcp_scan(x["q"], x["k"], x["v"], x["g"], x["beta"], 2, y=torch.zeros(8, 2, 63).bfloat16())
    with pytest.raises(ValueError):      # more segments than tokens
        kda.kcp_scan(x["q"], x["k"], x["v"], x["g"], x["beta"], 9)
    with pytest.raises(ValueError):      # interval not a multiple of the chunk
        kda.chunk_fwd_checkpointed(x["q"], x["k"], x["v"], x["g"], x["beta"], 48, chunk=32)
    # decode: q [N, H, dk]
    q = torch.zeros(3, 2, 64, dtype=torch.bfloat16)
    g, b = torch.zeros(3, 2, 64), torch.zeros(3, 2)
    with pytest.raises(ValueError):
        kda.decode_step(q, q, q, g, b, torch.zeros(3, 2, 64, 32))
    with pytest.raises(TypeError):
        kda.decode_step(q, q, q, g, b, torch.zeros(3, 2, 64, 64, dtype=torch.float64))
    with pytest.raises(TypeError):
        kda.decode_step(q, q, q, g, b, torch.zeros(3, 2, 64, 64), y=torch.zeros(3, 2, 64))
    # replay: inputs [N, Td, H, d]
    r = torch.zeros(3, 4, 2, 64, dtype=torch.bfloat16)
    rg, rb = torch.zeros(3, 4, 2, 64), torch.zeros(3, 4, 2)
    st = torch.zeros(3, 2, 64, 64)
    with pytest.raises(ValueError):
        kda.decode_replay(r, r, r, rg, rb, st, y=torch.zeros(3, 3, 2, 64, dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        kda.decode_replay(r, r, r, rg, rb, st, accepted=torch.zeros(3, dtype=torch.int64))
    with pytest.raises(ValueError):
        kda.decode_replay(r, r, r, rg, rb, st, want_y=False)     # nothing to produce
