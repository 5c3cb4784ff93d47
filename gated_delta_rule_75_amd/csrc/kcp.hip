// KCP phase 2: the state entering every segment (page "Exercices", Niveau 3
// Q21-Q22: a segment acts on the state entering it as S_end = M S_start +
// Sloc, and pairs compose associatively, (M2, S2) o (M1, S1) =
// (M2 M1, M2 S1 + S2)).  Phase 1 (the pairs) and phase 3 (every segment's
// outputs from its entering state) are the prefill kernels; see kda_kcp_scan
// in api.cpp.
//
// The segments are cut into G groups of L ~ sqrt(nseg).  Three launches of
// the chain kernel (in a narrow or a wide form, below): (1) each group's pairs composed into one pair, all groups
// side by side; (2) one chain over the G group pairs from S0, giving the
// state entering each group; (3) each group's segments replayed from its
// entering state, all groups side by side, writing every segment's entering
// state.  The dependent depth is about 3 sqrt(nseg) steps instead of nseg.
#include "common.h"
#include "launch.h"

namespace kda {

// One chain of pairs applied to a slice of the columns of a DK-row state X:
//     for j = 0 .. L-1:  [out_each[s0 + j] = X;]  X <- M_{s0+j} X + A_{s0+j}
//     [out_final[g] = X]
// with (M_s, A_s) from the pair rows [M | Sloc] of `pairs` (row width W).
// Plain chains carry a state of dv columns (A = Sloc, X starts at `init`);
// augmented chains carry [M | S] (dk + dv columns: the first dk start at the
// identity and take no additive term, A = Sloc on the rest), which composes
// the chain's pairs into one pair (page "Exercices", Niveau 3 Q21-Q22).
//
// Narrow form, for launches with few chains (one round of workgroups): a
// step is a DK x DK by DK x 16 product on fp32 MFMA 16x16x4.  Sixteen
// columns a workgroup spread a chain over many CUs (the steps of a chain
// are sequential, and a 64-column slice kept one CU busy for ~8k cycles a
// step: the one chain over the group pairs takes 55 us against 104).  Four
// waves split the rows: wave w forms rows [w DK/4, (w+1) DK/4) of the new X
// in accumulator tiles (lane: rows 4 (l/16) + i, column l%16).
// The state crosses between waves through LDS, stored transposed (X^T, a
// column per row) so that a lane reads the four k values of its MFMA
// operands with one 16-byte access; two buffers alternate, one barrier a
// step.  Each wave reads its rows of M_s straight from memory as 16-byte
// runs, one step ahead, into registers: lane (l%16, l/16) of k-block kb
// holds M[row][16 kb + 4 (l/16) + i], MFMA i of the k-block taking that k.
struct ChainParams {
    int H, nseg, L;          // pairs entries, steps per chain (chain g starts at g L)
    int W;                   // row width of a pair: dk + dv
    int aug;                 // augmented [M | S] state
    int ncol;                // state columns: dv, or dk + dv when augmented
    const float* pairs;      // [nseg][H][dk][W]
    const float* init;       // plain chains: [G][H][dk][dv] or NULL (zeros)
    float* out_each;         // plain chains: [nseg][H][dk][dv] or NULL
    float* out_final;        // [G][H][dk][ncol] or NULL
};

template <int DK>
__global__ __launch_bounds__(256) void kcp_chain_narrow_kernel(ChainParams p) {
    constexpr int RW = DK / 4;          // rows per wave
    constexpr int NRT = RW / 16;        // 16-row tiles per wave
    constexpr int NKB = DK / 16;        // 16-wide k-blocks
    constexpr int XP = DK + 4;          // LDS pitch of a column of X^T (floats)
    __shared__ __attribute__((aligned(16))) float sX[2][16 * XP];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4, l16 = lane & 15;
    const int g = blockIdx.x, h = blockIdx.y;
    const int col = blockIdx.z * 16 + l16;   // this lane's state column
    const int s0 = g * p.L;
    const int L = p.nseg - s0 < p.L ? p.nseg - s0 : p.L;
    if (L <= 0) return;
    const int dv = p.W - DK;
    const int r0 = wave * RW;                // first row of the wave
    auto prow = [&](int s, int r) { return p.pairs + (((int64_t)s * p.H + h) * DK + r) * p.W; };
    const bool ident = p.aug && col < DK;    // transition columns: start I, no additive term
    const int acol = p.aug ? col : DK + col;

    // M rows of the wave and the additive terms of its accumulator rows, step s
    auto load = [&](int s, f32x4_t (*M)[NKB], f32x4_t* A) {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            const float* pr = prow(s, r0 + 16 * rt + l16);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) M[rt][kb] = *reinterpret_cast<const f32x4_t*>(pr + 16 * kb + 4 * g4);
#pragma unroll
            for (int i = 0; i < 4; ++i) A[rt][i] = ident ? 0.f : prow(s, r0 + 16 * rt + 4 * g4 + i)[acol];
        }
    };

    // the initial state: this wave's rows in registers and X^T in LDS buffer 0
    f32x4_t X[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = r0 + 16 * rt + 4 * g4 + i;
            float x = 0.f;
            if (p.aug) x = (col == r) ? 1.f : 0.f;
            else if (p.init) x = p.init[(((int64_t)g * p.H + h) * DK + r) * dv + col];
            X[rt][i] = x;
        }
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
        *reinterpret_cast<f32x4_t*>(&sX[0][l16 * XP + r0 + 16 * rt + 4 * g4]) = X[rt];
    f32x4_t M[NRT][NKB], A[NRT];
    load(s0, M, A);
    __syncthreads();
    for (int j = 0; j < L; ++j) {
        const int s = s0 + j;
        if (p.out_each) {
            float* o = p.out_each + ((int64_t)s * p.H + h) * DK * dv;
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[(int64_t)(r0 + 16 * rt + 4 * g4 + i) * dv + col] = X[rt][i];
        }
        f32x4_t Mn[NRT][NKB], An[NRT];
        if (j + 1 < L) load(s + 1, Mn, An);
        const float* xb = sX[j & 1];
        f32x4_t xo[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) xo[kb] = *reinterpret_cast<const f32x4_t*>(xb + l16 * XP + 16 * kb + 4 * g4);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            f32x4_t acc = A[rt];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(M[rt][kb][i], xo[kb][i], acc, 0, 0, 0);
            X[rt] = acc;
            *reinterpret_cast<f32x4_t*>(&sX[(j + 1) & 1][l16 * XP + r0 + 16 * rt + 4 * g4]) = acc;
        }
        __syncthreads();   // the new X^T is complete; the old buffer is free for the step after
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            A[rt] = An[rt];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) M[rt][kb] = Mn[rt][kb];
        }
    }
    if (p.out_final) {
        float* o = p.out_final + ((int64_t)g * p.H + h) * DK * p.ncol;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[(int64_t)(r0 + 16 * rt + 4 * g4 + i) * p.ncol + col] = X[rt][i];
    }
}

// Wide form, for launches with many chains side by side: a 64-column slice
// a workgroup, four waves of 16 columns, each forming all DK rows of its
// columns; X stays in accumulator tiles and enters the next product as the B
// operand, MFMA i taking row 4 (l/16) + i (fp32 16x16x4); M_{s+1} streams into
// the other half of a double buffer in LDS by global-to-LDS copies while
// step s computes, and the barrier between steps waits for LDS only.  It
// reads each M once for 64 columns, where the narrow form reads it once for
// 16: with more than one round of workgroups the narrow form is bound by
// those reads (152 us against 103 for 1024 narrow workgroups).
template <int DK>
__global__ __launch_bounds__(256) void kcp_chain_wide_kernel(ChainParams p) {
    constexpr int NRT = DK / 16;                 // 16-row tiles of the state
    constexpr int RPC = 1024 / (DK * 4);         // M rows per 1 KiB copy
    constexpr int NCP = DK / RPC;                // copies per M
    constexpr int MP = 1024 + 16;                // LDS pitch of a copy (bank spread)
    constexpr int MBUF = NCP * MP;
    static_assert(NCP % 4 == 0, "copies per wave");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4, l16 = lane & 15;
    const int g = blockIdx.x, h = blockIdx.y;
    const int col = blockIdx.z * 64 + wave * 16 + l16;   // this lane's state column
    const int s0 = g * p.L;
    const int L = p.nseg - s0 < p.L ? p.nseg - s0 : p.L;
    if (L <= 0) return;
    const int dv = p.W - DK;
    auto prow = [&](int s, int r) { return p.pairs + (((int64_t)s * p.H + h) * DK + r) * p.W; };

    // copies [4 j + wave] of M_s into buffer b: rows RPC c .. RPC c + RPC - 1
    auto stage = [&](int s, int b) {
        char* buf = smem + b * MBUF;
#pragma unroll
        for (int jj = 0; jj < NCP / 4; ++jj) {
            const int c = jj * 4 + wave;
            const int r = RPC * c + lane / (64 / RPC), k = (lane % (64 / RPC)) * 4;
            lds_dma16(prow(s, r) + k, buf + c * MP);
        }
    };
    auto mread = [&](const char* buf, int r, int k) -> f32x4_t {
        return *reinterpret_cast<const f32x4_t*>(buf + (r / RPC) * MP + (r % RPC) * DK * 4 + k * 4);
    };
    // additive column of step s for this lane's rows
    const bool ident = p.aug && col < DK;
    const int acol = p.aug ? col : DK + col;
    auto load_a = [&](int s, f32x4_t* a) {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) a[rt][i] = ident ? 0.f : prow(s, 16 * rt + 4 * g4 + i)[acol];
    };

    f32x4_t X[NRT], A[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * rt + 4 * g4 + i;
            float x = 0.f;
            if (p.aug) x = (col == r) ? 1.f : 0.f;
            else if (p.init) x = p.init[(((int64_t)g * p.H + h) * DK + r) * dv + col];
            X[rt][i] = x;
        }
    stage(s0, 0);
    load_a(s0, A);
    for (int j = 0; j < L; ++j) {
        const int s = s0 + j;
        const char* buf = smem + (j & 1) * MBUF;
        if (p.out_each) {
            float* o = p.out_each + ((int64_t)s * p.H + h) * DK * dv;
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[(16 * rt + 4 * g4 + i) * dv + col] = X[rt][i];
        }
        f32x4_t acc[NRT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) acc[rt] = A[rt];
        wait_vmcnt<0>();           // M_s (and A_s) have landed
        barrier_keep_loads();      // ... for every wave; buffer (j+1)&1 is free
        if (j + 1 < L) {
            stage(s + 1, (j + 1) & 1);
            load_a(s + 1, A);
        }
#pragma unroll
        for (int kt = 0; kt < NRT; ++kt)
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                const f32x4_t m4 = mread(buf, 16 * rt + l16, 16 * kt + 4 * g4);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(m4[i], X[kt][i], acc[rt], 0, 0, 0);
            }
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) X[rt] = acc[rt];
    }
    if (p.out_final) {
        float* o = p.out_final + ((int64_t)g * p.H + h) * DK * p.ncol;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[(16 * rt + 4 * g4 + i) * p.ncol + col] = X[rt][i];
    }
}

template <int DK>
static hipError_t launch_chain_t(const ChainParams& p, int nchain, hipStream_t stream) {
    // narrow form while its workgroups fit in one round at two per CU
    int cus = 0;
    hipError_t e = device_cu_count(&cus);
    if (e != hipSuccess) return e;
    const int64_t narrow_wgs = (int64_t)nchain * p.H * (p.ncol / 16);
    if (narrow_wgs <= 2 * (int64_t)cus) {
        hipLaunchKernelGGL(kcp_chain_narrow_kernel<DK>, dim3(nchain, p.H, p.ncol / 16), dim3(256), 0, stream, p);
        return hipGetLastError();
    }
    constexpr int MBUF = (DK / (1024 / (DK * 4))) * (1024 + 16);
    auto kern = kcp_chain_wide_kernel<DK>;
    e = ensure_lds_limit((const void*)kern, 2 * MBUF);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(nchain, p.H, p.ncol / 64), dim3(256), 2 * MBUF, stream, p);
    return hipGetLastError();
}

static hipError_t launch_chain(int dk, const ChainParams& p, int nchain, hipStream_t stream) {
    return dk == 128 ? launch_chain_t<128>(p, nchain, stream) : launch_chain_t<64>(p, nchain, stream);
}

int kcp_group_len(int nseg) {
    int L = 1;
    while (L * L < nseg) ++L;
    return L;
}

hipError_t launch_kcp_scan(int H, int dk, int dv, int nseg, const float* pairs, const float* initial_state,
                           float* starts, float* group_pairs, float* group_starts, hipStream_t stream) {
    const int L = kcp_group_len(nseg), G = (nseg + L - 1) / L;
    ChainParams p{};
    p.H = H;
    p.W = dk + dv;
    // 1. every group's pairs composed into one pair, groups side by side
    p.nseg = nseg;
    p.L = L;
    p.aug = 1;
    p.ncol = dk + dv;
    p.pairs = pairs;
    p.out_final = group_pairs;
    hipError_t e = launch_chain(dk, p, G, stream);
    if (e != hipSuccess) return e;
    // 2. the state entering every group: one chain over the group pairs
    p = ChainParams{};
    p.H = H;
    p.W = dk + dv;
    p.nseg = G;
    p.L = G;
    p.ncol = dv;
    p.pairs = group_pairs;
    p.init = initial_state;
    p.out_each = group_starts;
    e = launch_chain(dk, p, 1, stream);
    if (e != hipSuccess) return e;
    // 3. the state entering every segment, groups side by side from their starts
    p = ChainParams{};
    p.H = H;
    p.W = dk + dv;
    p.nseg = nseg;
    p.L = L;
    p.ncol = dv;
    p.pairs = pairs;
    p.init = group_starts;
    p.out_each = starts;
    return launch_chain(dk, p, G, stream);
}

}  // namespace kda
