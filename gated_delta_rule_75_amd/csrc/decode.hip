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
    __shared__ __attribute__((aligned(16))) float s_delta[DV];   // read as float4
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
    // v and z are read only here: loaded beside the state (before or after
    // its loads, one value a thread or in 16-byte pieces) they made the step
    // 6-10 % slower
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
template <typename T, int DK, int DV, int TG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void replay_kernel(int Td, float scale, int H, const T* __restrict__ q,
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

    // The inputs of TG draft tokens at a time are staged in LDS, so the tokens
    // of a group wait on no global load, and the products of consecutive
    // tokens alternate between two buffers, so two barriers a token suffice.
    // Calls with outputs stage four tokens at a time (verify 209 -> 175-182 us
    // on 128 requests x 96 heads x 4 drafts); a commit alone stages one (with
    // four it ran 6 % slower: loads issued next to the state's reads slow a
    // pass that also writes the state back, as in the decode step).
    __shared__ float s_k[TG][DK], s_q[TG][DK], s_a[TG][DK], s_v[TG][DV], s_z[TG][DV], s_b[TG];
    __shared__ float s_u[2][RG][DV + 4], s_w[2][RG][DV + 4];
    __shared__ __attribute__((aligned(16))) float s_delta[2][DV];   // read as float4
    __shared__ float s_kq[2];

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

    // one input element per thread and token: k, q, g of channel ck, v, z of
    // column cv (threads past dk / dv re-read an element and write it again)
    static_assert(DK <= 256 && DV <= 256 && (DK & (DK - 1)) == 0 && (DV & (DV - 1)) == 0, "one element per thread");
    const int ck = tid & (DK - 1), cv = tid & (DV - 1);
    const T* zp = z ? z : v;   // read and ignored when ungated
    T rk[TG], rq[TG], rv[TG], rz[TG];
    float rgv[TG], rb[TG];
    auto load_group = [&](int t0, int tn) {
#pragma unroll
        for (int j = 0; j < TG; ++j) {
            if (j < tn) {   // workgroup-uniform
                const int64_t tok = ((int64_t)n * Td + t0 + j) * H + h;
                rk[j] = k[tok * DK + ck];
                rq[j] = q[tok * DK + ck];
                rgv[j] = g[tok * DK + ck];
                rv[j] = v[tok * DV + cv];
                rz[j] = zp[tok * DV + cv];
                rb[j] = beta[tok];
            }
        }
    };
    auto write_group = [&](int tn) {
#pragma unroll
        for (int j = 0; j < TG; ++j) {
            if (j >= tn) break;
            s_k[j][ck] = to_f32(rk[j]);
            s_q[j][ck] = to_f32(rq[j]);
            s_a[j][ck] = fast_exp(rgv[j]);
            s_v[j][cv] = to_f32(rv[j]);
            s_z[j][cv] = to_f32(rz[j]);
            if (tid == 0) s_b[j] = rb[j];
        }
    };
    f32x4_t S[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) S[r] = *reinterpret_cast<const f32x4_t*>(st + (int64_t)(r * RG + rg) * DV + 4 * cg);
    // the tokens of one staged group
    auto run_group = [&](int t0, int tn) {
        for (int j = 0; j < tn; ++j) {
            const int t = t0 + j, par = t & 1;
            if (tid < kWave) {
                float pk = 0.f;
                for (int c = tid; c < DK; c += kWave) pk += s_k[j][c] * s_q[j][c];
#pragma unroll
                for (int off = kWave / 2; off > 0; off >>= 1) pk += __shfl_xor(pk, off);
                if (tid == 0) s_kq[par] = pk;
            }
            f32x4_t u = {0.f, 0.f, 0.f, 0.f}, w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                const int row = r * RG + rg;
                S[r] *= s_a[j][row];
                u += s_k[j][row] * S[r];
                w += s_q[j][row] * S[r];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s_u[par][rg][4 * cg + i] = u[i];
                s_w[par][rg][4 * cg + i] = w[i];
            }
            barrier_keep_loads();
            if (tid < DV) {
                float U = 0.f, W = 0.f;
#pragma unroll
                for (int r = 0; r < RG; ++r) {
                    U += s_u[par][r][tid];
                    W += s_w[par][r][tid];
                }
                const float d = s_b[j] * (s_v[j][tid] - U);
                s_delta[par][tid] = d;
                if (y) {
                    float o = scale * (W + s_kq[par] * d);
                    if (z) o *= sigmoid(s_z[j][tid]);
                    gstore(y + (((int64_t)n * Td + t) * H + h) * DV + tid, o);
                }
            }
            barrier_keep_loads();
            const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(&s_delta[par][4 * cg]);
#pragma unroll
            for (int r = 0; r < RPT; ++r) S[r] += s_k[j][r * RG + rg] * d4;
            if (t + 1 == acc) {   // the state after the accepted prefix
#pragma unroll
                for (int r = 0; r < RPT; ++r)
                    __builtin_nontemporal_store(S[r], reinterpret_cast<f32x4_t*>(st + (int64_t)(r * RG + rg) * DV + 4 * cg));
            }
        }
    };
    for (int t0 = 0; t0 < steps; t0 += TG) {
        const int tn = steps - t0 < TG ? steps - t0 : TG;
        if (t0 > 0) barrier_keep_loads();   // every wave is done with the previous group
        load_group(t0, tn);
        write_group(tn);
        barrier_keep_loads();
        run_group(t0, tn);
    }
}

template <typename T, int DK, int DV>
static hipError_t launch_replay_t(const DecodeArgs& a, int Td, const int32_t* accepted) {
    if (a.N == 0) return hipSuccess;
    auto kern = a.y ? replay_kernel<T, DK, DV, 4> : replay_kernel<T, DK, DV, 1>;
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.N * a.H)), dim3(256), 0, (hipStream_t)a.stream, Td, a.scale,
                       a.H, (const T*)a.q, (const T*)a.k, (const T*)a.v, (const float*)a.g,
                       (const float*)a.beta, (const T*)a.z, accepted, a.state, (T*)a.y);
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
