"""The benchmark's work model: the algorithmic bytes and flops that every
roofline fraction divides by, checked against independent counts.

- Bytes: the K3-layer prefill reads q, k, v, z (bf16), g (fp32 per key
  channel) and beta (fp32 per token and head) once, writes y (bf16) and the
  final fp32 state once: 1,796 B per (token, head) plus 96 states of
  128 x 128 fp32.  The decode step reads and writes the fp32 state and reads
  one token's inputs per request.  The counts here are written out tensor by
  tensor, not from the bench's per-element formula.
- Flops: the chunked form's products counted one by one for a chunk (the
  three state products, the triangular Gram products, W, U and P Delta) and
  compared with the closed form the bench uses.
"""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_model", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_k3_layer_prefill_bytes():
    b = _bench()
    T, H, dk, dv = 8192, 96, 128, 128
    tensors = {
        "q": T * H * dk * 2, "k": T * H * dk * 2, "v": T * H * dv * 2, "z": T * H * dv * 2,
        "g": T * H * dk * 4, "beta": T * H * 4, "y": T * H * dv * 2,
        "final_state": H * dk * dv * 4,
    }
    assert sum(tensors.values()) == 1_418_723_328
    assert b.prefill_bytes(T, H, dk, dv, 2, True, 1, False, True) == sum(tensors.values())
    # per (token, head), the figure the roofline divides by
    assert (sum(tensors.values()) - tensors["final_state"]) // (T * H) == 1796


def test_varlen_and_kcp_bytes():
    b = _bench()
    # varlen: initial and final states of every (sequence, head) chain
    T, H, N = 1000, 4, 3
    per = 2 * 128 * 2 + 128 * 2 + 128 * 2 + 128 * 2 + 128 * 4 + 4
    assert b.prefill_bytes(T, H, 128, 128, 2, True, N, True, True) == T * H * per + 2 * N * H * 128 * 128 * 4
    # KCP at 2^20 tokens, 4 heads, ungated, final state only
    T, H = 1 << 20, 4
    per = 2 * 128 * 2 + 128 * 2 + 128 * 2 + 128 * 4 + 4
    assert per == 1540
    assert b.prefill_bytes(T, H, 128, 128, 2, False, 1, False, True) == 6_459_490_304


def test_decode_bytes():
    b = _bench()
    N, H, dk, dv = 128, 96, 128, 128
    state = N * H * dk * dv * 4
    inputs = N * H * (dk * 2 + dk * 2 + dv * 2 + dv * 2 + dk * 4 + 4)   # q, k, v, z, g, beta
    y = N * H * dv * 2
    assert 2 * state + inputs + y == 1_632_681_984
    assert b.decode_bytes(N, H, dk, dv, 2, True) == 1_632_681_984
    # fused inputs: a and b in bf16 instead of fp32 g and beta
    inputs_fused = N * H * (dk * 2 + dk * 2 + dv * 2 + dv * 2 + dk * 2 + 2)
    assert b.decode_bytes(N, H, dk, dv, 2, True, gate_elt=2) == 2 * state + inputs_fused + y


def _chunk_flops_counted(C: int, dk: int, dv: int) -> int:
    """Multiply-adds of one chunk of the chunked form, product by product, x 2."""
    tri = C * (C + 1) // 2        # pairs j <= t
    strict = C * (C - 1) // 2     # pairs j < t
    macs = 0
    macs += C * dk * dv           # W S            (Delta)
    macs += C * dk * dv           # Qt S           (output)
    macs += dk * C * dv           # Kh^T Delta     (state update)
    macs += strict * dk           # A = gated k.k  (strictly lower)
    macs += tri * dk              # P = gated q.k  (lower, with the diagonal)
    macs += tri * dk              # W = Tb (K e^G) (Tb lower triangular)
    macs += tri * dv              # U = Tb V
    macs += tri * dv              # P Delta
    return 2 * macs


def test_prefill_flops_formula():
    b = _bench()
    for C, dk, dv in ((64, 128, 128), (16, 64, 64), (32, 128, 128)):
        counted = _chunk_flops_counted(C, dk, dv)
        model = b.prefill_flops(C, 1, dk, dv, C)
        # the closed form rounds the triangles to C^2 / 2; it stays within
        # the diagonal's share of the intra-chunk products
        assert abs(model - counted) <= 2 * C * (3 * dk + 2 * dv), (C, model, counted)
        assert abs(model - counted) / counted < 0.01 + 1.0 / C
