// KCP phase 2: fold the segment pairs in order to give every segment its
// entering state (page "Exercices", Niveau 3 Q21-Q22: a segment acts on the
// state entering it as S_end = M S_start + Sloc, and pairs compose
// associatively, (M2, S2) o (M1, S1) = (M2 M1, M2 S1 + S2)).
//
// Phase 1 (the pairs) and phase 3 (every segment's outputs from its entering
// state) are the prefill kernel; see kda_kcp_scan in api.cpp.
//
// This kernel applies the pairs to the state directly: starts[0] = S0 and
// starts[s+1] = M_s starts[s] + Sloc_s.  State columns are independent, so a
// workgroup owns CW columns of one head and walks the segments.  Each step
// is a dk x dk times dk x CW product: thread (row r, column half) reads row r
// of M_s from LDS once and the state block by broadcast, and M_{s+1} and the
// thread's row of Sloc_{s+1} are in flight meanwhile (the head's column blocks
// share M in L2).  The barriers wait for LDS operations only, so those loads
// stay in flight across them; a step waits on memory only where it writes
// M_{s+1} into LDS, after its own product.
#include "common.h"
#include "launch.h"

namespace kda {

template <int DK, int DV, int CW>
__global__ __launch_bounds__(256) void kcp_scan_kernel(int H, int nseg,
                                                       const float* __restrict__ pairs,
                                                       const float* __restrict__ s0,
                                                       float* __restrict__ starts) {
    constexpr int NT = 256;
    constexpr int TPR = NT / DK;          // threads per state row
    constexpr int CPT = CW / TPR;         // columns per thread
    constexpr int W = DK + DV;            // row width of a pair [M | Sloc]
    constexpr int LM = DK + 4;            // padded LDS pitch of M
    constexpr int MV4 = DK * DK / 4;      // float4s of M
    static_assert(TPR * DK == NT && CPT * TPR == CW && CPT % 4 == 0, "scan tiling");
    extern __shared__ __attribute__((aligned(16))) float sm[];
    float* sM = sm;                        // [2][DK][LM]
    float* sS = sm + 2 * DK * LM;          // [2][DK][CW]

    const int nblk_h = DV / CW;
    const int h = blockIdx.x / nblk_h;
    const int col0 = (blockIdx.x % nblk_h) * CW;
    const int tid = threadIdx.x;
    const int r = tid / TPR;
    const int cj = (tid % TPR) * CPT;

    auto pair_row = [&](int s, int row) { return pairs + (((int64_t)s * H + h) * DK + row) * W; };
    // M of segment s into LDS buffer b (vector loads, then LDS writes)
    auto stage_m = [&](int s, int b, f32x4_t* tmp) {
#pragma unroll
        for (int i = 0; i < MV4 / NT; ++i) {
            const int e = (i * NT + tid) * 4, row = e / DK, c = e % DK;
            tmp[i] = *reinterpret_cast<const f32x4_t*>(pair_row(s, row) + c);
        }
    };
    auto put_m = [&](int b, const f32x4_t* tmp) {
#pragma unroll
        for (int i = 0; i < MV4 / NT; ++i) {
            const int e = (i * NT + tid) * 4, row = e / DK, c = e % DK;
            *reinterpret_cast<f32x4_t*>(sM + (b * DK + row) * LM + c) = tmp[i];
        }
    };

    float cur[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j)
        cur[j] = s0 ? s0[((int64_t)h * DK + r) * DV + col0 + cj + j] : 0.f;
    f32x4_t tmp[MV4 / NT];
    f32x4_t lnext[CPT / 4];   // Sloc row r of the next step, prefetched
    auto stage_l = [&](int s) {
#pragma unroll
        for (int j = 0; j < CPT; j += 4)
            lnext[j / 4] = *reinterpret_cast<const f32x4_t*>(pair_row(s, r) + DK + col0 + cj + j);
    };
    if (nseg > 1) {
        stage_m(0, 0, tmp);
        stage_l(0);
        put_m(0, tmp);
    }
    int buf = 0;
    for (int s = 0; s < nseg; ++s) {
        float* st = starts + (((int64_t)s * H + h) * DK + r) * DV + col0 + cj;
#pragma unroll
        for (int j = 0; j < CPT; j += 4) {
            const f32x4_t v = f32x4_t{cur[j], cur[j + 1], cur[j + 2], cur[j + 3]};
            *reinterpret_cast<f32x4_t*>(st + j) = v;
            *reinterpret_cast<f32x4_t*>(sS + (buf * DK + r) * CW + cj + j) = v;
        }
        if (s + 1 == nseg) break;
        const bool more = s + 2 < nseg;
        float acc[CPT];
#pragma unroll
        for (int j = 0; j < CPT; j += 4) {
            acc[j] = lnext[j / 4][0];
            acc[j + 1] = lnext[j / 4][1];
            acc[j + 2] = lnext[j / 4][2];
            acc[j + 3] = lnext[j / 4][3];
        }
        if (more) {   // M and Sloc of the next step, in flight during this one
            stage_m(s + 1, buf ^ 1, tmp);
            stage_l(s + 1);
        }
        barrier_keep_loads();                      // M_s and S_s visible; M_{s+1} stays in flight
        const float* mrow = sM + (buf * DK + r) * LM;
        const float* sblk = sS + buf * DK * CW + cj;
#pragma unroll 4
        for (int c = 0; c < DK; c += 4) {
            const f32x4_t m4 = *reinterpret_cast<const f32x4_t*>(mrow + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
#pragma unroll
                for (int j = 0; j < CPT; j += 4) {
                    const f32x4_t s4 = *reinterpret_cast<const f32x4_t*>(sblk + (c + e) * CW + j);
                    acc[j] += m4[e] * s4[0];
                    acc[j + 1] += m4[e] * s4[1];
                    acc[j + 2] += m4[e] * s4[2];
                    acc[j + 3] += m4[e] * s4[3];
                }
            }
        }
        if (more) put_m(buf ^ 1, tmp);
#pragma unroll
        for (int j = 0; j < CPT; ++j) cur[j] = acc[j];
        buf ^= 1;
        // the next iteration's writes to buffer buf (= the one read two steps
        // later) are ordered by its own barrier; buffer buf^1 was last read here
        barrier_keep_loads();
    }
}

template <int DK, int DV, int CW>
static hipError_t launch_scan_t(int H, int nseg, const float* pairs, const float* s0,
                                float* starts, hipStream_t stream) {
    const size_t lds = (size_t)(2 * DK * (DK + 4) + 2 * DK * CW) * sizeof(float);
    auto kern = kcp_scan_kernel<DK, DV, CW>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(H * (DV / CW)), dim3(256), lds, stream, H, nseg, pairs, s0,
                       starts);
    return hipGetLastError();
}

hipError_t launch_kcp_scan(int H, int dk, int dv, int nseg, const float* pairs,
                           const float* initial_state, float* starts, float* /*final_state*/,
                           hipStream_t stream) {
    if (dk == 128) return launch_scan_t<128, 128, 8>(H, nseg, pairs, initial_state, starts, stream);
    return launch_scan_t<64, 64, 16>(H, nseg, pairs, initial_state, starts, stream);
}

}  // namespace kda
