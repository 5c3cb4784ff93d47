// Decode step of the KDA recurrence: one token per request against the
// resident fp32 state, updated in place (page "Exercices", Niveau 1 Q4 and Q6:
// decode is bandwidth-limited and the state has a fixed size).
//
// Per (request n, head h) one workgroup makes ONE pass over S (dk x dv fp32):
//   S^ = Diag(alpha) S                  alpha = exp(g)       (forget)
//   u  = S^^T k,  w = S^^T q            two reductions over the key channels
//   delta = beta (v - u)                                     (erase)
//   S  <- S^ + k delta^T                written back in place (write)
//   o  = scale (w + (k.q) delta)        = scale S_t^T q
//   y  = o * sigmoid(z)                 (gated)
// The identity o = S_t^T q = S^^T q + (k^T q) delta lets the output be formed
// without a second read of the state.  Each thread owns float4 column groups
// of several rows, so every wave reads whole 512-byte rows (coalesced 16-byte
// accesses) and the state crosses HBM exactly once each way; the write-back
// uses nontemporal stores (measured 5.7 TB/s against 5.1 TB/s with plain stores).
#include "common.h"
#include "launch.h"

namespace kda {

// Request-head of hardware workgroup i.  Workgroups i, i + 8, i + 16, ... run
// on one XCD; handing each XCD its heads in runs of two consecutive ones
// (64 KiB states, so 128 KiB runs) instead of one made the 128 x 96 step
// 6 % faster (5.35 against 5.72 ms per 20 steps, alternating runs, three
// boxes); other run lengths, from 3 to 1536 heads, moved it by -7 % to +4 %
// from box to box.  Applied when the grid is a multiple of 16.
__device__ __forceinline__ int decode_head(int i, int nb) {
    if (nb % 16 != 0) return i;
    const int x = i % 8, j = i / 8;
    return (j / 2) * 16 + x * 2 + j % 2;
}

//
// FUSED: q and k arrive unnormalised and the gates as pre-activations a (per
// key channel) and b (per head), in the storage dtype: alpha = exp(g_min
// sigmoid(a)), beta = sigmoid(b), and the unit vectors k^ = k / |k|,
// q^ = q / |q| (|x| = sqrt(sum x^2 + eps)).  The reductions run on the raw
// k, q and are rescaled afterwards: S^T k^ = (S^T k) / |k|, the write uses
// k (delta / |k|), and k^.q^ = (k.q) / (|k| |q|); the norms come from the same
// wave-0 reduction as k.q.
template <typename T, int DK, int DV, bool FUSED>
__global__ __launch_bounds__(256) void decode_kernel(float scale, int H, const T* __restrict__ q,
                                                     const T* __restrict__ k,
                                                     const T* __restrict__ v,
                                                     const void* __restrict__ gp,
                                                     const void* __restrict__ betap,
                                                     const T* __restrict__ z,
                                                     float* __restrict__ state, T* __restrict__ y) {
    constexpr int CG = DV / 4;      // float4 column groups per row
    constexpr int RG = 256 / CG;    // row groups
    constexpr int RPT = DK / RG;    // rows per thread
    static_assert(RG * CG == 256 && RPT * RG == DK, "decode tiling");

    __shared__ float s_k[DK], s_q[DK], s_a[DK];
    __shared__ float s_u[RG][DV + 4], s_w[RG][DV + 4];
    __shared__ float s_delta[DV];
    __shared__ float s_kq, s_ik, s_iq;

    const int nh = decode_head(blockIdx.x, gridDim.x);
    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;
    const int64_t kb = (int64_t)nh * DK, vb = (int64_t)nh * DV;
    float* st = state + (int64_t)nh * DK * DV;

    // issue the state loads first: they are the whole cost of the step
    f32x4_t S[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int row = r * RG + rg;
        S[r] = *reinterpret_cast<const f32x4_t*>(st + (int64_t)row * DV + 4 * cg);
    }
    for (int c = tid; c < DK; c += 256) {
        s_k[c] = gload(k + kb + c);
        s_q[c] = gload(q + kb + c);
        if constexpr (FUSED) s_a[c] = fast_exp(decay_gate(gload(static_cast<const T*>(gp) + kb + c)));
        else s_a[c] = fast_exp(static_cast<const float*>(gp)[kb + c]);
    }
    __syncthreads();
    if (tid < kWave) {
        float p = 0.f, pk = 0.f, pq = 0.f;
        for (int c = tid; c < DK; c += kWave) {
            p += s_k[c] * s_q[c];
            if constexpr (FUSED) {
                pk += s_k[c] * s_k[c];
                pq += s_q[c] * s_q[c];
            }
        }
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1) {
            p += __shfl_xor(p, off);
            if constexpr (FUSED) {
                pk += __shfl_xor(pk, off);
                pq += __shfl_xor(pq, off);
            }
        }
        if (tid == 0) {
            if constexpr (FUSED) {
                const float ik = rsqrtf(pk + kNormEps), iq = rsqrtf(pq + kNormEps);
                s_ik = ik;
                s_iq = iq;
                s_kq = p * ik * iq;
            } else {
                s_kq = p;
            }
        }
    }
    f32x4_t u = {0.f, 0.f, 0.f, 0.f}, w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int row = r * RG + rg;
        S[r] *= s_a[row];
        u += s_k[row] * S[r];
        w += s_q[row] * S[r];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s_u[rg][4 * cg + i] = u[i];
        s_w[rg][4 * cg + i] = w[i];
    }
    __syncthreads();
    if (tid < DV) {
        const int j = tid;
        float U = 0.f, W = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            U += s_u[r][j];
            W += s_w[r][j];
        }
        float bt, ik = 1.f;
        if constexpr (FUSED) {
            bt = sigmoid(gload(static_cast<const T*>(betap) + nh));
            ik = s_ik;
            U *= ik;
            W *= s_iq;
        } else {
            bt = static_cast<const float*>(betap)[nh];
        }
        const float d = bt * (gload(v + vb + j) - U);
        s_delta[j] = d * ik;   // the write adds k (d / |k|)^T = k^ d^T
        float o = scale * (W + s_kq * d);
        if (z) o *= sigmoid(gload(z + vb + j));
        gstore(y + vb + j, o);
    }
    __syncthreads();
    const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(&s_delta[4 * cg]);
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int row = r * RG + rg;
        const f32x4_t val = S[r] + s_k[row] * d4;
        // streaming store: the updated state is not read again by this step
        __builtin_nontemporal_store(val, reinterpret_cast<f32x4_t*>(st + (int64_t)row * DV + 4 * cg));
    }
}

// Speculative-decoding replay (page "Exercices", Niveau 3 Q27: the state after
// any accepted prefix is fixed by the draft tokens' inputs, so only those are
// kept and the recurrence is replayed on chip).  One workgroup per
// (request, head) loads the state once, runs the decode step above for each of
// the request's draft tokens with the state in registers, emits every draft
// token's output (when y is given), and writes the state back as it stands
// after the accepted prefix (when accepted is given), in the middle of the
// loop when outputs of later draft tokens are still to come.  The state is
// read only before the loop, so writing it there is safe, and no second
// register copy is needed (154 VGPRs: three workgroups per SIMD, against two
// with a copy).
template <typename T, int DK, int DV>
__global__ __launch_bounds__(256) void replay_kernel(int Td, float scale, int H, const T* __restrict__ q,
                                                     const T* __restrict__ k, const T* __restrict__ v,
                                                     const float* __restrict__ g,
                                                     const float* __restrict__ beta,
                                                     const T* __restrict__ z,
                                                     const int32_t* __restrict__ accepted,
                                                     float* __restrict__ state, T* __restrict__ y) {
    constexpr int CG = DV / 4;
    constexpr int RG = 256 / CG;
    constexpr int RPT = DK / RG;
    static_assert(RG * CG == 256 && RPT * RG == DK, "replay tiling");

    __shared__ float s_k[DK], s_q[DK], s_a[DK];
    __shared__ float s_u[RG][DV + 4], s_w[RG][DV + 4];
    __shared__ float s_delta[DV];
    __shared__ float s_kq;

    // placement as in the decode step (the commit, which writes the state, 3 % faster)
    const int nh = decode_head(blockIdx.x, gridDim.x), n = nh / H, h = nh % H;
    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;
    int acc = 0;
    if (accepted) {
        acc = accepted[n];
        acc = acc < 0 ? 0 : (acc > Td ? Td : acc);
    }
    const int steps = y ? Td : acc;   // without outputs only the accepted prefix matters
    if (steps == 0) return;
    float* st = state + (int64_t)nh * DK * DV;

    f32x4_t S[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) S[r] = *reinterpret_cast<const f32x4_t*>(st + (int64_t)(r * RG + rg) * DV + 4 * cg);
    // a draft token's inputs, one element per thread (k, q, g below dk; v, z,
    // beta below dv), loaded while the token before it is computed: the
    // barriers in the loop wait for LDS operations only, so those loads stay
    // in flight across them
    static_assert(DK <= 256 && DV <= 256, "one input element per thread");
    float xk = 0.f, xq = 0.f, xg = 0.f, xv = 0.f, xz = 0.f, xb = 0.f;
    auto fetch = [&](int t, float& fk, float& fq, float& fg, float& fv, float& fz, float& fb) {
        const int64_t tok = ((int64_t)n * Td + t) * H + h;
        if (tid < DK) {
            fk = gload(k + tok * DK + tid);
            fq = gload(q + tok * DK + tid);
            fg = g[tok * DK + tid];
        }
        if (tid < DV) {
            fv = gload(v + tok * DV + tid);
            fz = z ? gload(z + tok * DV + tid) : 0.f;
            fb = beta[tok];
        }
    };
    fetch(0, xk, xq, xg, xv, xz, xb);
    for (int t = 0; t < steps; ++t) {
        const int64_t tok = ((int64_t)n * Td + t) * H + h;
        const int64_t vb = tok * DV;
        if (tid < DK) {
            s_k[tid] = xk;
            s_q[tid] = xq;
            s_a[tid] = fast_exp(xg);
        }
        float nk = 0.f, nq = 0.f, ng = 0.f, nv = 0.f, nz = 0.f, nb = 0.f;
        if (t + 1 < steps) fetch(t + 1, nk, nq, ng, nv, nz, nb);
        barrier_keep_loads();
        if (tid < kWave) {
            float pk = 0.f;
            for (int c = tid; c < DK; c += kWave) pk += s_k[c] * s_q[c];
#pragma unroll
            for (int off = kWave / 2; off > 0; off >>= 1) pk += __shfl_xor(pk, off);
            if (tid == 0) s_kq = pk;
        }
        f32x4_t u = {0.f, 0.f, 0.f, 0.f}, w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const int row = r * RG + rg;
            S[r] *= s_a[row];
            u += s_k[row] * S[r];
            w += s_q[row] * S[r];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s_u[rg][4 * cg + i] = u[i];
            s_w[rg][4 * cg + i] = w[i];
        }
        barrier_keep_loads();
        if (tid < DV) {
            const int j = tid;
            float U = 0.f, W = 0.f;
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                U += s_u[r][j];
                W += s_w[r][j];
            }
            const float d = xb * (xv - U);
            s_delta[j] = d;
            if (y) {
                float o = scale * (W + s_kq * d);
                if (z) o *= sigmoid(xz);
                gstore(y + vb + j, o);
            }
        }
        barrier_keep_loads();
        const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(&s_delta[4 * cg]);
#pragma unroll
        for (int r = 0; r < RPT; ++r) S[r] += s_k[r * RG + rg] * d4;
        if (t + 1 == acc) {   // the state after the accepted prefix
#pragma unroll
            for (int r = 0; r < RPT; ++r)
                __builtin_nontemporal_store(S[r], reinterpret_cast<f32x4_t*>(st + (int64_t)(r * RG + rg) * DV + 4 * cg));
        }
        barrier_keep_loads();  // s_k, s_delta are rewritten by the next token
        xk = nk; xq = nq; xg = ng; xv = nv; xz = nz; xb = nb;
    }
}

template <typename T, int DK, int DV>
static hipError_t launch_replay_t(const DecodeArgs& a, int Td, const int32_t* accepted) {
    if (a.N == 0) return hipSuccess;
    hipLaunchKernelGGL((replay_kernel<T, DK, DV>), dim3((unsigned)(a.N * a.H)), dim3(256), 0,
                       (hipStream_t)a.stream, Td, a.scale, a.H, (const T*)a.q, (const T*)a.k,
                       (const T*)a.v, (const float*)a.g, (const float*)a.beta, (const T*)a.z, accepted,
                       a.state, (T*)a.y);
    return hipGetLastError();
}

hipError_t launch_replay(const DecodeArgs& a, int Td, const int32_t* accepted) {
    if (a.dtype == 0) {
        if (a.dk == 128) return launch_replay_t<__bf16, 128, 128>(a, Td, accepted);
        return launch_replay_t<__bf16, 64, 64>(a, Td, accepted);
    }
    if (a.dk == 128) return launch_replay_t<float, 128, 128>(a, Td, accepted);
    return launch_replay_t<float, 64, 64>(a, Td, accepted);
}

template <typename T, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs& a) {
    if (a.N == 0) return hipSuccess;
    if (a.fused) {
        hipLaunchKernelGGL((decode_kernel<T, DK, DV, true>), dim3((unsigned)(a.N * a.H)), dim3(256), 0,
                           (hipStream_t)a.stream, a.scale, a.H, (const T*)a.q, (const T*)a.k,
                           (const T*)a.v, a.g, a.beta, (const T*)a.z, a.state, (T*)a.y);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((decode_kernel<T, DK, DV, false>), dim3((unsigned)(a.N * a.H)), dim3(256), 0,
                       (hipStream_t)a.stream, a.scale, a.H, (const T*)a.q, (const T*)a.k,
                       (const T*)a.v, a.g, a.beta, (const T*)a.z, a.state, (T*)a.y);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a) {
    if (a.dtype == 0) {
        if (a.dk == 128) return launch_decode_t<__bf16, 128, 128>(a);
        return launch_decode_t<__bf16, 64, 64>(a);
    }
    if (a.dk == 128) return launch_decode_t<float, 128, 128>(a);
    return launch_decode_t<float, 64, 64>(a);
}

}  // namespace kda
