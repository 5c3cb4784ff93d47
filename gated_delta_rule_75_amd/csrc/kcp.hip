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
// workgroup owns CW columns of one head and walks the segments; the M_s rows
// it streams are shared by the head's other column blocks through L2.
#include "common.h"
#include "launch.h"

namespace kda {

template <int DK, int DV, int CW>
__global__ __launch_bounds__(256) void kcp_scan_kernel(int H, int nseg,
                                                       const float* __restrict__ pairs,
                                                       const float* __restrict__ s0,
                                                       float* __restrict__ starts) {
    constexpr int TPR = 256 / DK;     // threads per state row
    constexpr int CPT = CW / TPR;     // columns per thread
    constexpr int W = DK + DV;        // row width of a pair [M | Sloc]
    static_assert(TPR * DK == 256 && CPT * TPR == CW && CPT >= 1, "scan tiling");
    __shared__ float sS[2][DK][CW];

    const int nblk_h = DV / CW;
    const int h = blockIdx.x / nblk_h;
    const int col0 = (blockIdx.x % nblk_h) * CW;
    const int tid = threadIdx.x;
    const int r = tid / TPR;
    const int cj = (tid % TPR) * CPT;

    float cur[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j)
        cur[j] = s0 ? s0[((int64_t)h * DK + r) * DV + col0 + cj + j] : 0.f;
    int buf = 0;
    for (int s = 0; s < nseg; ++s) {
        float* st = starts + (((int64_t)s * H + h) * DK + r) * DV + col0 + cj;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            st[j] = cur[j];
            sS[buf][r][cj + j] = cur[j];
        }
        if (s + 1 == nseg) break;
        __syncthreads();
        const float* prow = pairs + (((int64_t)s * H + h) * DK + r) * W;
        float acc[CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) acc[j] = prow[DK + col0 + cj + j];
#pragma unroll 4
        for (int c = 0; c < DK; c += 4) {
            const f32x4_t m4 = *reinterpret_cast<const f32x4_t*>(prow + c);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int j = 0; j < CPT; ++j) acc[j] += m4[e] * sS[buf][c + e][cj + j];
        }
#pragma unroll
        for (int j = 0; j < CPT; ++j) cur[j] = acc[j];
        buf ^= 1;
    }
}

hipError_t launch_kcp_scan(int H, int dk, int dv, int nseg, const float* pairs,
                           const float* initial_state, float* starts, float* /*final_state*/,
                           hipStream_t stream) {
    constexpr int CW = 8;
    if (dk == 128) {
        hipLaunchKernelGGL((kcp_scan_kernel<128, 128, CW>), dim3(H * (128 / CW)), dim3(256), 0,
                           stream, H, nseg, pairs, initial_state, starts);
    } else {
        hipLaunchKernelGGL((kcp_scan_kernel<64, 64, CW>), dim3(H * (64 / CW)), dim3(256), 0,
                           stream, H, nseg, pairs, initial_state, starts);
    }
    return hipGetLastError();
}

}  // namespace kda
