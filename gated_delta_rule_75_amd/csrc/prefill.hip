// Chunkwise prefill of the KDA recurrence on gfx950 MFMA.
//
// Recurrence (page "Exercices", Niveau 2 Q7: forget Diag(alpha), erase
// I - beta k k^T, write beta k v^T):
//     S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T,
//     o_t = scale S_t^T q_t,  y_t = o_t sigmoid(z_t).
// The pages refer the blocked ("UT transform") form to another paper and do
// not print it; the form below is derived from the recurrence.  Unrolling a
// chunk of C tokens that starts from state S, with G_t the in-chunk running
// sum of g:
//     S_t = Diag(e^{G_t}) S + sum_{j<=t} Diag(e^{G_t - G_j}) k_j delta_j^T
//     delta_t + beta_t sum_{j<t} A_tj delta_j = beta_t (v_t - S^T (k_t e^{G_t}))
// with A_tj = sum_c k_tc k_jc e^{G_tc - G_jc}.  Hence, per chunk,
//     Delta = L^{-1} R,   L = I + diag(beta) A,  R = diag(beta)(V - (K e^G) S)
//     O     = (Q e^G) S + P Delta,   P_tj = sum_c q_tc k_jc e^{G_tc - G_jc}, j <= t
//     S    <- Diag(e^{G_C}) S + (K e^{G_C - G})^T Delta.
// All products are MFMA tiles (bf16 operands and fp32 accumulation for bf16
// inputs, fp32 throughout for fp32 inputs); the state is carried in fp32
// registers across chunks and never leaves the chip until the final write.
//
// Exponent range.  e^{-G} over a 64-token chunk can reach e^{320}.  The
// factors are therefore taken relative to 16-token sub-tile references, the
// tile size the bounded decay g >= -5 is sized for (page "Exercices",
// Niveau 2 Q8: 16 tokens at g_min give e^{80}, inside bf16's range):
//   diagonal Gram block (a,a):  (x_t e^{G_t - R_a}) . (k_j e^{R_a - G_j})   <= 1 and <= e^80
//   off-diagonal block (a,b):   (x_t e^{G_t - E_b}) . (k_j e^{E_b - G_j})   both <= 1
// where R_a is G at the start of sub-tile a and E_b at the end of sub-tile b.
// The off-diagonal factors are applied while loading MMA fragments:
// e^{G_t - E_b} = e^{G_t - R_a} e^{R_a - E_b} and e^{E_b - G_j} = e^{R_b - G_j} e^{E_b - R_b}.
//
// Work decomposition: one workgroup (4 waves) per (sequence, head, value
// slice of VS columns).  State columns evolve independently, so slices only
// repeat the key-side products (A, P, L^{-1}).  Workgroups of one head land on
// the same XCD (blockIdx round-robins over the 8 XCDs) so the slices share the
// q/k/g reads through that XCD's L2.
#include "common.h"
#include "launch.h"

namespace kda {

struct PrefillParams {
    int H, num_seqs, nchains, nslices, final_seq_lo, dvt;  // dvt: value width of the state
    float scale;
    int64_t T_total, seg_len;
    const int32_t* cu_seqlens;
    const void *q, *k, *v;
    const float *g, *beta;
    const void* z;
    const float* s0;
    float* sfin;
    void* y;
};

// Launch modes.  They share one kernel body; distinct instantiations keep the
// per-kernel profiler statistics of the different call sites apart.
enum PfMode : int {
    kModeSeq = 0,     // one sequence, or equal segments (no offsets array)
    kModeVarlen = 1,  // packed sequences given by cu_seqlens
    kModePairs = 2,   // KCP segment pairs: augmented state [I | 0], values [0 | v], no outputs
    kModeFinish = 3,  // KCP outputs of every segment from its entering state
};

template <typename E_, int DK_, int VS_, int CH_, int MODE_>
struct PfCfg {
    using E = E_;
    using T = typename E::T;
    static constexpr int DK = DK_, VS = VS_, CH = CH_, MODE = MODE_;
    static constexpr bool AUG = MODE_ == kModePairs;
    static constexpr int NT = CH / 16, NCT = DK / 16, NVT = VS / 16;
    static constexpr int PADE = 16 / (int)sizeof(T);
    static constexpr int LDK = DK + PADE;  // pitch of [.][DK] operand arrays
    static constexpr int LCH = CH + PADE;  // pitch of [.][CH] operand arrays
    static constexpr int LN = CH + 4;      // pitch of the fp32 N array
    static constexpr int NW = 8, NTHR = 64 * NW;
    // Waves 0-3 own the state and the R tiles; waves 4-7 own the output tiles
    // and the diagonal inverses.
    // decay phase: each thread holds TPT tokens x CPT channels; a wave holds
    // GPTW token groups x CGW channel groups of one 16-token tile
    static constexpr int CPT = (CH == 16 && DK == 64) ? 2 : 4;
    static constexpr int CGW = DK * NT / (8 * CPT);
    static constexpr int GPTW = 64 / CGW;
    static constexpr int TPT = 16 / GPTW;
    static constexpr int NOT = NT * NVT;        // (t, v) tiles of R, Delta and O
    static constexpr int OPW = (NOT + 3) / 4;   // R / O tiles per wave of a 4-wave group
    static constexpr int DPW = (NOT + NW - 1) / NW;  // Delta tiles per wave
    static constexpr int NST = NCT * NVT;       // (c, v) state tiles
    static constexpr int SPW = NST / 4;         // state tiles per wave of waves 0-3
    static constexpr int NPAIR = NT * (NT + 1) / 2;
    static constexpr int NTASK = AUG ? NPAIR : 2 * NPAIR;
    static_assert(NT == 1 || NT == 4, "chunk of 16 or 64 tokens");
    static_assert(GPTW * CGW == 64 && TPT * GPTW == 16 && TPT >= 1, "decay-phase mapping");
    static_assert(NST % 4 == 0 && 4 % NVT == 0, "state tiles per wave share one value tile");

    static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
    static constexpr size_t SZ_OP = (size_t)CH * LDK * sizeof(T);
    static constexpr size_t O_KR = 0;
    static constexpr size_t O_QR = O_KR + SZ_OP;
    static constexpr size_t O_KC = O_QR + SZ_OP;
    static constexpr size_t O_KT = O_KC + SZ_OP;
    static constexpr size_t O_ST = O_KT + al((size_t)DK * LCH * sizeof(T));
    static constexpr size_t O_N = O_ST + al((size_t)VS * LDK * sizeof(T));
    static constexpr size_t SZ_N0 = (size_t)CH * LN * 4, SZ_N1 = (size_t)VS * LCH * sizeof(T);
    static constexpr size_t O_NT = O_N + al(SZ_N0 > SZ_N1 ? SZ_N0 : SZ_N1);
    static constexpr size_t O_T = O_NT + (size_t)NT * 16 * 16 * 4;
    static constexpr size_t O_P = O_T + al((size_t)CH * LCH * sizeof(T));
    static constexpr size_t O_RT = O_P + al((size_t)CH * LCH * sizeof(T));
    static constexpr size_t O_TP = O_RT + al((size_t)VS * LCH * sizeof(T));
    static constexpr size_t O_ES = O_TP + (size_t)NT * DK * 4;
    static constexpr size_t O_D = O_ES + (size_t)NT * DK * 4;
    static constexpr size_t O_EGC = O_D + (size_t)NT * NT * DK * 4;
    static constexpr size_t O_BETA = O_EGC + (size_t)DK * 4;
    static constexpr size_t O_MISC = O_BETA + (size_t)CH * 4;
    static constexpr size_t BYTES = O_MISC + 16;
    // aliases of regions that are dead while they are used
    static constexpr size_t O_TT = O_KC;   // L^{-1} transposed, during the inverse only
    static constexpr size_t O_YT = O_KR;   // per-wave 16x16 scratch of the inverse
    static constexpr size_t O_DT = O_N;    // Delta^T, after the inverse
    static constexpr size_t O_SORT = O_KR; // sequence lengths, before the first chunk
    static constexpr bool FITS = BYTES <= 160 * 1024 &&
        (size_t)CH * LCH * sizeof(T) <= SZ_OP &&
        (NT == 1 || (size_t)3 * 16 * (16 + PADE) * sizeof(T) <= SZ_OP);
};

// Pairs of consecutive channels of q / k as loaded from global memory.
template <typename T> struct Pair2;
template <> struct Pair2<__bf16> { using type = bf16x2_t; };
template <> struct Pair2<float> { using type = f32x2_t; };

template <typename T, int n> struct VecT;
template <> struct VecT<__bf16, 2> { using type = bf16x2_t; };
template <> struct VecT<__bf16, 4> { using type = bf16x4_t; };
template <> struct VecT<float, 2> { using type = f32x2_t; };
template <> struct VecT<float, 4> { using type = f32x4_t; };
template <int n> using f32xn = typename VecT<float, n>::type;

// four consecutive elements as fp32 (8-byte aligned for bf16, 16 for fp32)
__device__ __forceinline__ f32x4_t gload4(const __bf16* p) {
    const bf16x4_t v = *reinterpret_cast<const bf16x4_t*>(p);
    return f32x4_t{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4_t gload4(const float* p) { return *reinterpret_cast<const f32x4_t*>(p); }
__device__ __forceinline__ void gstore4(__bf16* p, f32x4_t v) {
    *reinterpret_cast<bf16x4_t*>(p) = bf16x4_t{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
}
__device__ __forceinline__ void gstore4(float* p, f32x4_t v) { *reinterpret_cast<f32x4_t*>(p) = v; }

__device__ __forceinline__ void st_vec4(bf16x4_t& d, const float* v) {
    d = bf16x4_t{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
}
__device__ __forceinline__ void st_vec4(f32x4_t& d, const float* v) { d = f32x4_t{v[0], v[1], v[2], v[3]}; }

__device__ __forceinline__ void st_pair(__bf16* p, float a, float b) {
    *reinterpret_cast<bf16x2_t*>(p) = bf16x2_t{(__bf16)a, (__bf16)b};
}
__device__ __forceinline__ void st_pair(float* p, float a, float b) {
    *reinterpret_cast<f32x2_t*>(p) = f32x2_t{a, b};
}

// n consecutive elements (n*sizeof(T) a multiple of 4, 4-byte aligned).
template <int n>
__device__ __forceinline__ void st_row(__bf16* p, const float* v) {
    if constexpr (n == 4) {
        *reinterpret_cast<bf16x4_t*>(p) = bf16x4_t{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    } else if constexpr (n == 2) {
        *reinterpret_cast<bf16x2_t*>(p) = bf16x2_t{(__bf16)v[0], (__bf16)v[1]};
    } else if constexpr (n % 8 == 0) {
#pragma unroll
        for (int i = 0; i < n; i += 8) {
            bf16x8_t w;
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = (__bf16)v[i + e];
            *reinterpret_cast<bf16x8_t*>(p + i) = w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < n; ++i) p[i] = (__bf16)v[i];
    }
}
template <int n>
__device__ __forceinline__ void st_row(float* p, const float* v) {
    if constexpr (n % 4 == 0) {
#pragma unroll
        for (int i = 0; i < n; i += 4)
            *reinterpret_cast<f32x4_t*>(p + i) = f32x4_t{v[i], v[i + 1], v[i + 2], v[i + 3]};
    } else {
#pragma unroll
        for (int i = 0; i < n; ++i) p[i] = v[i];
    }
}

// 16x16x16 product acc += A B^T over a 16-deep reduction, operands in LDS:
// A rows r (k contiguous; fp32 or the element type), B stored as rows =
// output columns (k contiguous, element type).  bf16: one 16x16x32 MFMA whose
// upper k half is zero; fp32: four 16x16x4 MFMAs.
template <typename E, typename TA>
__device__ __forceinline__ f32x4_t mma16(f32x4_t acc, const TA* A, int lda,
                                         const typename E::T* B, int ldb, int lane);

template <>
__device__ __forceinline__ f32x4_t mma16<BF16, float>(f32x4_t acc, const float* A, int lda,
                                                      const __bf16* B, int ldb, int lane) {
    const int r = lane & 15, gq = lane >> 4;
    bf16x8_t fa, fb;
    if (gq < 2) {
        const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(A + r * lda + 8 * gq);
        const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(A + r * lda + 8 * gq + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            fa[e] = (__bf16)a0[e];
            fa[e + 4] = (__bf16)a1[e];
        }
        fb = *reinterpret_cast<const bf16x8_t*>(B + r * ldb + 8 * gq);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) fa[e] = fb[e] = (__bf16)0.f;
    }
    return BF16::mma(fa, fb, acc);
}

template <>
__device__ __forceinline__ f32x4_t mma16<BF16, __bf16>(f32x4_t acc, const __bf16* A, int lda,
                                                       const __bf16* B, int ldb, int lane) {
    const int r = lane & 15, gq = lane >> 4;
    bf16x8_t fa, fb;
    if (gq < 2) {
        fa = *reinterpret_cast<const bf16x8_t*>(A + r * lda + 8 * gq);
        fb = *reinterpret_cast<const bf16x8_t*>(B + r * ldb + 8 * gq);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) fa[e] = fb[e] = (__bf16)0.f;
    }
    return BF16::mma(fa, fb, acc);
}

template <>
__device__ __forceinline__ f32x4_t mma16<F32, float>(f32x4_t acc, const float* A, int lda,
                                                     const float* B, int ldb, int lane) {
    const int r = lane & 15, gq = lane >> 4;
#pragma unroll
    for (int k0 = 0; k0 < 16; k0 += 4) acc = F32::mma(A[r * lda + k0 + gq], B[r * ldb + k0 + gq], acc);
    return acc;
}

// (ta, vt) of the m-th R / O tile of wave gw (0..3) of a 4-wave group.  With
// 4 sub-tiles per chunk each wave owns one row tile, so the scaled row
// operand of a k step is built once and shared by its NVT tiles.
template <class C>
__device__ __forceinline__ void ro_tile(int gw, int m, int& ta, int& vt) {
    if constexpr (C::NT == 4) {
        ta = gw;
        vt = m;
    } else {
        const int ti = gw + 4 * m;
        ta = 0;
        vt = ti;
    }
}

template <class C>
__global__ __launch_bounds__(C::NTHR) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_kernel(PrefillParams p) {
    using E = typename C::E;
    using T = typename C::T;
    using T2 = typename Pair2<T>::type;
    constexpr int DK = C::DK, VS = C::VS, CH = C::CH, NT = C::NT, NVT = C::NVT;
    constexpr int LDK = C::LDK, LCH = C::LCH, LN = C::LN;
    constexpr int KS = E::KSTEP, NTHR = C::NTHR;
    constexpr bool AUG = C::AUG;
    static_assert(C::FITS, "LDS budget of a gfx950 workgroup (160 KiB)");

    __shared__ __attribute__((aligned(16))) char smem[C::BYTES];
    T* sKr = reinterpret_cast<T*>(smem + C::O_KR);
    T* sQr = reinterpret_cast<T*>(smem + C::O_QR);
    T* sKc = reinterpret_cast<T*>(smem + C::O_KC);
    T* sKt = reinterpret_cast<T*>(smem + C::O_KT);
    T* sSt = reinterpret_cast<T*>(smem + C::O_ST);
    float* sN = reinterpret_cast<float*>(smem + C::O_N);
    float* sNt = reinterpret_cast<float*>(smem + C::O_NT);
    T* sDt = reinterpret_cast<T*>(smem + C::O_DT);
    T* sT = reinterpret_cast<T*>(smem + C::O_T);
    T* sTt = reinterpret_cast<T*>(smem + C::O_TT);
    T* sYt = reinterpret_cast<T*>(smem + C::O_YT);
    T* sP = reinterpret_cast<T*>(smem + C::O_P);
    T* sRt = reinterpret_cast<T*>(smem + C::O_RT);
    float* sTP = reinterpret_cast<float*>(smem + C::O_TP);
    float* sES = reinterpret_cast<float*>(smem + C::O_ES);
    float* sD = reinterpret_cast<float*>(smem + C::O_D);
    float* sEGC = reinterpret_cast<float*>(smem + C::O_EGC);
    float* sBeta = reinterpret_cast<float*>(smem + C::O_BETA);
    int* sMisc = reinterpret_cast<int*>(smem + C::O_MISC);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int gw = wave & 3;            // wave index within its group of four
    const bool lowg = wave < 4;         // waves 0-3: state, R; waves 4-7: outputs, inverse

    // ---- which (sequence, head, slice) this workgroup owns ------------------
    const int b = blockIdx.x;
    const int xcd = b & 7, jb = b >> 3;
    const int slot = (jb / p.nslices) * 8 + xcd;
    const int slice = jb % p.nslices;
    if (slot >= p.nchains) return;
    const int H = p.H;
    const int seqrank = slot / H, h = slot % H;
    int n = seqrank;
    if (p.cu_seqlens && p.num_seqs > 1 && p.num_seqs <= 256) {
        // longest sequences first: find the sequence of rank `seqrank`
        int* sLen = reinterpret_cast<int*>(smem + C::O_SORT);
        for (int i = tid; i < p.num_seqs; i += NTHR) sLen[i] = p.cu_seqlens[i + 1] - p.cu_seqlens[i];
        __syncthreads();
        for (int i = tid; i < p.num_seqs; i += NTHR) {
            const int li = sLen[i];
            int rank = 0;
            for (int j = 0; j < p.num_seqs; ++j) {
                const int lj = sLen[j];
                rank += (lj > li) || (lj == li && j < i);
            }
            if (rank == seqrank) sMisc[0] = i;
        }
        __syncthreads();
        n = sMisc[0];
        __syncthreads();
    }
    int64_t t0, t1;
    if (p.cu_seqlens) {
        t0 = p.cu_seqlens[n];
        t1 = p.cu_seqlens[n + 1];
    } else {
        t0 = (int64_t)n * p.seg_len;
        t1 = t0 + p.seg_len < p.T_total ? t0 + p.seg_len : p.T_total;
    }
    const int64_t len = t1 > t0 ? t1 - t0 : 0;
    const int cb = slice * VS;                 // first state column of the slice
    const bool ident = AUG && cb < DK;         // KCP transition columns: V = 0, S0 = I
    const int vcol0 = ident ? 0 : (AUG ? cb - DK : cb);  // column of v feeding this slice
    const int DV = AUG ? p.dvt - DK : p.dvt;   // row width of v / z / y

    const T* gq = static_cast<const T*>(p.q);
    const T* gk = static_cast<const T*>(p.k);
    const T* gv = static_cast<const T*>(p.v);
    const T* gz = static_cast<const T*>(p.z);
    T* gy = static_cast<T*>(p.y);
    const bool gated = !AUG && gz != nullptr;

    // ---- state tiles (waves 0-3): (ct, vt) = si / NVT, si % NVT, si = gw + 4m --
    f32x4_t S[C::SPW];
    {
        const int64_t sbase = ((int64_t)n * H + h) * DK * (int64_t)p.dvt;
#pragma unroll
        for (int m = 0; m < C::SPW; ++m) {
            const int si = gw + 4 * m, ct = si / NVT, vt = si % NVT;
            const int col = cb + 16 * vt + r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = 16 * ct + 4 * g4 + i;
                float s = 0.f;
                if (AUG) s = (col == c) ? 1.f : 0.f;
                else if (p.s0 && lowg) s = p.s0[sbase + (int64_t)c * p.dvt + col];
                S[m][i] = s;
            }
            if (lowg) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sSt[(16 * vt + r16) * LDK + 16 * ct + 4 * g4 + i] = from_f32<T>(S[m][i]);
            }
        }
    }
    // zero the upper-triangular blocks of P and L^{-1} (never written later)
    for (int idx = tid; idx < CH * CH; idx += NTHR) {
        const int t = idx / CH, j = idx % CH;
        if ((j >> 4) > (t >> 4)) {
            sT[t * LCH + j] = from_f32<T>(0.f);
            sP[t * LCH + j] = from_f32<T>(0.f);
        }
    }

    // ---- decay-phase thread mapping ------------------------------------------
    // Wave w covers 16-token tile dtile = w / (8 / NT) and a block of CPW
    // channels; lane = (token group tgrp, channel group cg) holds TPT
    // consecutive tokens x CPT consecutive channels, so q, k and g arrive in
    // CPT-wide vector loads and a tile's token groups sit in one wave.
    constexpr int CPT = C::CPT, TPT = C::TPT, CGW = C::CGW, GPTW = C::GPTW;
    const int dtile = wave / (8 / NT);
    const int tgrp = lane / CGW, cg = lane % CGW;
    const int c0 = (wave % (8 / NT)) * (DK * NT / 8) + CPT * cg;   // first channel
    const int tl0 = 16 * dtile + TPT * tgrp;                        // first token (in chunk)

    using TV = typename VecT<T, CPT>::type;
    TV rq[TPT], rk[TPT];
    f32xn<CPT> rgv[TPT];
    float rbeta = 0.f;
    // v (waves 0-3, R tiles) or z (waves 4-7, output tiles): 4 consecutive
    // value columns of one token per tile, the transposed MMA-output layout
    const int HDK = H * DK, HDV = H * DV;   // token strides (elements)
    // Kept as raw storage vectors: converting at load time would make the wave
    // wait for the prefetch right away.  vz_n is in flight for the next chunk,
    // vz the current chunk's copy.
    using TV4 = typename VecT<T, 4>::type;
    TV4 vz[C::OPW], vz_n[C::OPW];
    // outputs of the previous chunk, stored in the middle of the next one so
    // that no wait for prefetched data also waits for these stores
    TV4 yd[C::OPW];
    T* yd_base = nullptr;
    int yd_nvalid = 0;
    auto store_y = [&]() {
#pragma unroll
        for (int m = 0; m < C::OPW; ++m) {
            int ta, vt;
            ro_tile<C>(gw, m, ta, vt);
            const int t = 16 * ta + r16;
            if (vt < NVT && t < yd_nvalid)
                *reinterpret_cast<TV4*>(yd_base + t * HDV + 16 * vt) = yd[m];
        }
    };
    const int64_t tclamp = len > 0 ? len - 1 : 0;
    // Global addresses: a 64-bit row base per chunk plus 32-bit in-chunk offsets.
    // Loads are unconditional from clamped rows; invalid tokens are masked at use.
    auto load_qkg = [&](int64_t cs) {
        const int64_t row = (t0 + cs) * H + h;
        const int last = (int)(tclamp - cs);   // >= 0 while cs < len
        const T* kb = gk + row * DK + c0;
        const T* qb = gq + row * DK + c0;
        const float* gb = p.g + row * DK + c0;
#pragma unroll
        for (int l = 0; l < TPT; ++l) {
            const int tr = tl0 + l < last ? tl0 + l : last;
            rk[l] = *reinterpret_cast<const TV*>(kb + tr * HDK);
            if (!AUG) rq[l] = *reinterpret_cast<const TV*>(qb + tr * HDK);
            rgv[l] = *reinterpret_cast<const f32xn<CPT>*>(gb + tr * HDK);
        }
        if (tid < CH) {
            const int tr = tid < last ? tid : last;
            rbeta = p.beta[row + (int64_t)tr * H];
        }
    };
    auto load_vz = [&](int64_t cs) {
        if (lowg || gated) {
            const int64_t row = (t0 + cs) * H + h;
            const int last = (int)(tclamp - cs);
            const T* src = (lowg ? gv : gz) + row * DV + vcol0 + 4 * g4;
#pragma unroll
            for (int m = 0; m < C::OPW; ++m) {
                int ta, vt;
                ro_tile<C>(gw, m, ta, vt);
                const int vtc = vt < NVT ? vt : 0;
                const int t = 16 * ta + r16;
                const int tr = t < last ? t : last;
                vz_n[m] = *reinterpret_cast<const TV4*>(src + tr * HDV + 16 * vtc);
            }
        }
    };

    const int64_t nchunks = (len + CH - 1) / CH;
    if (nchunks > 0) {
        load_qkg(0);
        load_vz(0);
    }
    __syncthreads();  // initial S^T and zeroed blocks visible; sort scratch consumed

    for (int64_t ch = 0; ch < nchunks; ++ch) {
        const int64_t cs = ch * CH;
        const int nvalid = len - cs < CH ? (int)(len - cs) : CH;
        // everything prefetched for this chunk is waited for here, once
#pragma unroll
        for (int m = 0; m < C::OPW; ++m) vz[m] = vz_n[m];
        // ================= phase 1: decay prefix and scaled operands ==========
        // Running products of alpha = e^g inside the thread's tokens, then a
        // multiplicative scan over the tile's token groups (lanes CGW apart);
        // tile products go through LDS for the chunk-level references.
        float cpv[CPT][TPT], sfv[CPT][TPT], ex[CPT], gp[CPT];
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
            float al[TPT], pr = 1.f;
#pragma unroll
            for (int l = 0; l < TPT; ++l) {
                al[l] = tl0 + l < nvalid ? fast_exp(rgv[l][e]) : 1.f;
                pr *= al[l];
                cpv[e][l] = pr;           // e^{G_t - G_before_group}
            }
            sfv[e][TPT - 1] = 1.f;
#pragma unroll
            for (int l = TPT - 2; l >= 0; --l) sfv[e][l] = sfv[e][l + 1] * al[l + 1];
            gp[e] = pr;                   // group product
            float inc = pr;               // inclusive product scan over token groups
#pragma unroll
            for (int st = 1; st < GPTW; st *= 2) {
                const float o = __shfl_up(inc, st * CGW);
                if (tgrp >= st) inc *= o;
            }
            ex[e] = inc * __builtin_amdgcn_rcpf(pr);   // exclusive: e^{G_before_group - R_a} (>= e^-80)
            if (tgrp == GPTW - 1) sTP[dtile * DK + c0 + e] = inc;   // tile product
        }
        if (tid < CH) sBeta[tid] = tid < nvalid ? rbeta : 0.f;
        __syncthreads();
        {
            float eGCmR[CPT];   // e^{G_C - R_a}
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
                float tp[NT];
#pragma unroll
                for (int a = 0; a < NT; ++a) tp[a] = sTP[a * DK + c0 + e];
                float suf = 1.f;
#pragma unroll
                for (int a = NT - 1; a >= 0; --a) {
                    suf *= tp[a];
                    if (a == dtile) eGCmR[e] = suf;
                }
                if (tgrp == 0) {
                    // per-channel tables: e^{R_a}, e^{R_a - R_b} (b < a), e^{G_C}
                    float pre = 1.f;
#pragma unroll
                    for (int a = 0; a < NT; ++a) {
                        if (a == dtile) {
                            sES[a * DK + c0 + e] = pre;
                            float dab = 1.f;
#pragma unroll
                            for (int bb = a - 1; bb >= 0; --bb) {
                                dab *= tp[bb];
                                sD[(a * NT + bb) * DK + c0 + e] = dab;
                            }
                        }
                        pre *= tp[a];
                    }
                    if (dtile == 0) sEGC[c0 + e] = pre;
                }
            }
            float kt[CPT][TPT], inv[CPT], g3[CPT];
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
                inv[e] = __builtin_amdgcn_rcpf(ex[e] * gp[e]);   // e^{R_a - G_last}
                g3[e] = eGCmR[e] * inv[e];                       // e^{G_C - G_last}
            }
            const bool full = nvalid == CH;
#pragma unroll
            for (int l = 0; l < TPT; ++l) {
                const int t = tl0 + l;
                const bool valid = full || t < nvalid;
                float f1[CPT], f2[CPT], kv[CPT], qv[CPT];
#pragma unroll
                for (int e = 0; e < CPT; ++e) {
                    kv[e] = valid ? to_f32(rk[l][e]) : 0.f;
                    qv[e] = (valid && !AUG) ? to_f32(rq[l][e]) : 0.f;
                    f1[e] = ex[e] * cpv[e][l];        // e^{G_t - R_a}  (<= 1)
                    f2[e] = inv[e] * sfv[e][l];       // e^{R_a - G_t}  (<= e^80)
                    kt[e][l] = kv[e] * (g3[e] * sfv[e][l]);   // k e^{G_C - G_t}
                }
                float o[CPT];
#pragma unroll
                for (int e = 0; e < CPT; ++e) o[e] = kv[e] * f1[e];
                st_row<CPT>(sKr + t * LDK + c0, o);
                if (!AUG) {
#pragma unroll
                    for (int e = 0; e < CPT; ++e) o[e] = qv[e] * f1[e];
                    st_row<CPT>(sQr + t * LDK + c0, o);
                }
#pragma unroll
                for (int e = 0; e < CPT; ++e) o[e] = kv[e] * f2[e];
                st_row<CPT>(sKc + t * LDK + c0, o);
            }
#pragma unroll
            for (int e = 0; e < CPT; ++e) st_row<TPT>(sKt + (c0 + e) * LCH + tl0, kt[e]);
        }
        // prefetch the next chunk's q, k, g, beta while this one computes
        if (ch + 1 < nchunks) {
            load_qkg(cs + CH);
            load_vz(cs + CH);
        }
        __syncthreads();

        // ================= phase 2: gated Gram blocks A and P ===================
        // Block (a, b): rows use e^{G_t - R_a} (<= 1); columns use e^{R_a - G_j},
        // i.e. the diagonal-reference column operand times e^{R_a - R_b} for b < a.
        for (int task = wave; task < C::NTASK; task += C::NW) {
            const int mat = task / C::NPAIR;  // 0: A (keys), 1: P (queries)
            const int pi = task % C::NPAIR;
            int a = 0;
            while ((a + 1) * (a + 2) / 2 <= pi) ++a;
            const int bb = pi - a * (a + 1) / 2;
            const T* X = mat ? sQr : sKr;
            constexpr int NK = DK / KS;
            typename E::Frag fa[NK], fb[NK];
#pragma unroll
            for (int q = 0; q < NK; ++q) {
                fa[q] = lds_frag<E>(X, LDK, 16 * a, q * KS, lane);
                fb[q] = (bb < a)
                    ? lds_frag_scaled<E>(sKc, LDK, 16 * bb, q * KS, lane, sD + (a * NT + bb) * DK)
                    : lds_frag<E>(sKc, LDK, 16 * bb, q * KS, lane);
            }
            __builtin_amdgcn_sched_barrier(0);   // all reads of the block before its MFMAs
            // two independent accumulation chains, summed at the end
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < NK; q += 2) {
                acc = E::mma(fa[q], fb[q], acc);
                if (q + 1 < NK) acc1 = E::mma(fa[q + 1], fb[q + 1], acc1);
            }
            acc += acc1;
            const int j = 16 * bb + r16;
            if (mat == 0) {
                if (bb == a) {
                    // diagonal block of N = diag(beta) A, stored transposed for the inverse
                    f32x4_t nv;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = 16 * a + 4 * g4 + i;
                        nv[i] = (j < t) ? sBeta[t] * acc[i] : 0.f;
                    }
                    *reinterpret_cast<f32x4_t*>(sNt + (a * 16 + r16) * 16 + 4 * g4) = nv;
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = 16 * a + 4 * g4 + i;
                        sN[t * LN + j] = sBeta[t] * acc[i];
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * a + 4 * g4 + i;
                    sP[t * LCH + j] = from_f32<T>((bb < a || j <= t) ? acc[i] : 0.f);
                }
            }
        }
        __syncthreads();

        // ================= phase 3: R = beta (V - (K e^G) S)  |  diagonal inverses
        if (lowg) {
            f32x4_t ak[C::OPW];
#pragma unroll
            for (int m = 0; m < C::OPW; ++m) ak[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            int ta0, vt0;
            ro_tile<C>(gw, 0, ta0, vt0);
            // transposed products: lane (r16, g4) of tile (ta, vt) holds token
            // 16 ta + r16 and value columns 16 vt + 4 g4 + i
#pragma unroll
            for (int kk = 0; kk < DK; kk += KS) {
                const typename E::Frag fb = lds_frag_scaled<E>(sKr, LDK, 16 * ta0, kk, lane, sES + ta0 * DK);
                typename E::Frag fa[C::OPW];
#pragma unroll
                for (int m = 0; m < C::OPW; ++m) {
                    int ta, vt;
                    ro_tile<C>(gw, m, ta, vt);
                    fa[m] = lds_frag<E>(sSt, LDK, 16 * (vt < NVT ? vt : 0), kk, lane);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int m = 0; m < C::OPW; ++m) {
                    int ta, vt;
                    ro_tile<C>(gw, m, ta, vt);
                    if (vt < NVT) ak[m] = E::mma(fa[m], fb, ak[m]);
                }
            }
#pragma unroll
            for (int m = 0; m < C::OPW; ++m) {
                int ta, vt;
                ro_tile<C>(gw, m, ta, vt);
                if (vt < NVT) {
                    const int t = 16 * ta + r16;
                    const float bt = sBeta[t];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float vv = ident ? 0.f : to_f32(vz[m][i]);
                        sRt[(16 * vt + 4 * g4 + i) * LCH + t] = from_f32<T>(bt * (vv - ak[m][i]));
                    }
                }
            }
        }
        if (wave == 4 && lane < 16 * NT) {
            // L_aa^{-1} of the 16x16 unit lower-triangular diagonal blocks, one
            // column per lane, right-looking forward substitution
            const int a = lane >> 4, jj = lane & 15;
            const float* Nt = sNt + a * 256;  // Nt[m * 16 + i] = N[i][m]
            float x[16], acc[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                x[m] = (m < jj) ? 0.f : (m == jj ? 1.f : -acc[m]);
                if (m + 1 < 16) {
                    float col[16];
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const f32x4_t w = *reinterpret_cast<const f32x4_t*>(Nt + m * 16 + 4 * q4);
                        col[4 * q4] = w[0];
                        col[4 * q4 + 1] = w[1];
                        col[4 * q4 + 2] = w[2];
                        col[4 * q4 + 3] = w[3];
                    }
#pragma unroll
                    for (int i = m + 1; i < 16; ++i) acc[i] += col[i] * x[m];
                }
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sT[(16 * a + i) * LCH + 16 * a + jj] = from_f32<T>(x[i]);
            if (NT > 1) {
                float xr[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) xr[i] = x[i];
                st_row<16>(sTt + (16 * a + jj) * LCH + 16 * a, xr);
            }
        }
        if (!lowg && !AUG && yd_base) store_y();   // outputs of the previous chunk
        __syncthreads();

        // ================= phase 4: off-diagonal blocks of L^{-1} ==============
#pragma unroll
        for (int d = 1; d < NT; ++d) {
            if (wave < NT - d) {
                // block (a, bb) = -L_aa^{-1} sum_{bb <= c < a} N_ac X_c,bb
                const int bb = wave, a = wave + d;
                f32x4_t y = {0.f, 0.f, 0.f, 0.f};
                for (int c = bb; c < a; ++c)
                    y = mma16<E>(y, sN + (16 * a) * LN + 16 * c, LN, sTt + (16 * bb) * LCH + 16 * c, LCH, lane);
                T* yt = sYt + wave * 16 * (16 + C::PADE);
#pragma unroll
                for (int i = 0; i < 4; ++i) yt[r16 * (16 + C::PADE) + 4 * g4 + i] = from_f32<T>(y[i]);
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                f32x4_t xab = {0.f, 0.f, 0.f, 0.f};
                xab = mma16<E>(xab, sT + (16 * a) * LCH + 16 * a, LCH, yt, 16 + C::PADE, lane);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const T xv = from_f32<T>(-xab[i]);
                    sT[(16 * a + 4 * g4 + i) * LCH + 16 * bb + r16] = xv;
                    sTt[(16 * bb + r16) * LCH + 16 * a + 4 * g4 + i] = xv;
                }
            }
            __syncthreads();
        }

        // ================= phase 5: Delta = L^{-1} R ==========================
#pragma unroll
        for (int m = 0; m < C::DPW; ++m) {
            const int ti = wave + C::NW * m;
            if (ti < C::NOT) {
                const int ta = ti / NVT, vt = ti % NVT;
                constexpr int NK = (CH + KS - 1) / KS;
                const int kend = 16 * (ta + 1);
                typename E::Frag fa[NK], fb[NK];
#pragma unroll
                for (int q = 0; q < NK; ++q) {
                    fa[q] = lds_frag_lim<E, CH>(sT, LCH, 16 * ta, q * KS, lane);
                    fb[q] = lds_frag_lim<E, CH>(sRt, LCH, 16 * vt, q * KS, lane);
                }
                __builtin_amdgcn_sched_barrier(0);
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int q = 0; q < NK; ++q)
                    if (q * KS < kend) acc = E::mma(fa[q], fb[q], acc);
                T dv4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) dv4[i] = from_f32<T>(acc[i]);
#pragma unroll
                for (int i = 0; i < 4; ++i) sDt[(16 * vt + r16) * LCH + 16 * ta + 4 * g4 + i] = dv4[i];
            }
        }
        __syncthreads();

        // ================= phase 6: state update  |  outputs ===================
        if (lowg) {
            {
                f32x4_t eg[C::SPW];
#pragma unroll
                for (int m = 0; m < C::SPW; ++m) {
                    const int ct = (gw + 4 * m) / NVT;
                    eg[m] = *reinterpret_cast<const f32x4_t*>(sEGC + 16 * ct + 4 * g4);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int m = 0; m < C::SPW; ++m) S[m] *= eg[m];
            }
#pragma unroll
            for (int kk = 0; kk < CH; kk += KS) {
                // all fragments of the k step first, then the MFMAs; every state
                // tile of the wave has value tile gw % NVT (NVT divides 4)
                typename E::Frag fa[C::SPW];
                const typename E::Frag fb = lds_frag_lim<E, CH>(sDt, LCH, 16 * (gw % NVT), kk, lane);
#pragma unroll
                for (int m = 0; m < C::SPW; ++m) {
                    const int ct = (gw + 4 * m) / NVT;
                    fa[m] = lds_frag_lim<E, CH>(sKt, LCH, 16 * ct, kk, lane);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int m = 0; m < C::SPW; ++m) S[m] = E::mma(fa[m], fb, S[m]);
            }
        } else if (!AUG) {
            // O = (Q e^G) S_old + P Delta, y = scale O sigmoid(z); transposed
            // products as for R: lane holds token 16 ta + r16, columns 16 vt + 4 g4 + i
            f32x4_t ao[C::OPW];
#pragma unroll
            for (int m = 0; m < C::OPW; ++m) ao[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            int ta0, vt0;
            ro_tile<C>(gw, 0, ta0, vt0);
#pragma unroll
            for (int kk = 0; kk < DK; kk += KS) {
                const typename E::Frag fb = lds_frag_scaled<E>(sQr, LDK, 16 * ta0, kk, lane, sES + ta0 * DK);
                typename E::Frag fa[C::OPW];
#pragma unroll
                for (int m = 0; m < C::OPW; ++m) {
                    int ta, vt;
                    ro_tile<C>(gw, m, ta, vt);
                    fa[m] = lds_frag<E>(sSt, LDK, 16 * (vt < NVT ? vt : 0), kk, lane);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int m = 0; m < C::OPW; ++m) {
                    int ta, vt;
                    ro_tile<C>(gw, m, ta, vt);
                    if (vt < NVT) ao[m] = E::mma(fa[m], fb, ao[m]);
                }
            }
            const int kend = 16 * (ta0 + 1);
#pragma unroll
            for (int kk = 0; kk < CH; kk += KS) {
                if (kk < kend) {
                    const typename E::Frag fb = lds_frag_lim<E, CH>(sP, LCH, 16 * ta0, kk, lane);
                    typename E::Frag fa[C::OPW];
#pragma unroll
                    for (int m = 0; m < C::OPW; ++m) {
                        int ta, vt;
                        ro_tile<C>(gw, m, ta, vt);
                        fa[m] = lds_frag_lim<E, CH>(sDt, LCH, 16 * (vt < NVT ? vt : 0), kk, lane);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int m = 0; m < C::OPW; ++m) {
                        int ta, vt;
                        ro_tile<C>(gw, m, ta, vt);
                        if (vt < NVT) ao[m] = E::mma(fa[m], fb, ao[m]);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < C::OPW; ++m) {
                float o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    o[i] = p.scale * ao[m][i];
                    if (gated) o[i] *= sigmoid(to_f32(vz[m][i]));
                }
                st_vec4(yd[m], o);
            }
            yd_base = gy + ((t0 + cs) * H + h) * DV + vcol0 + 4 * g4;
            yd_nvalid = nvalid;
        }
        __syncthreads();  // every read of the old S^T is done
        if (lowg) {
#pragma unroll
            for (int m = 0; m < C::SPW; ++m) {
                const int si = gw + 4 * m, ct = si / NVT, vt = si % NVT;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sSt[(16 * vt + r16) * LDK + 16 * ct + 4 * g4 + i] = from_f32<T>(S[m][i]);
            }
        }
        __syncthreads();
    }

    if (!lowg && !AUG && yd_base) store_y();   // outputs of the last chunk

    // ---- final state ---------------------------------------------------------
    if (lowg && p.sfin && n >= p.final_seq_lo) {
        const int64_t sbase = ((int64_t)(n - p.final_seq_lo) * H + h) * DK * (int64_t)p.dvt;
#pragma unroll
        for (int m = 0; m < C::SPW; ++m) {
            const int si = gw + 4 * m, ct = si / NVT, vt = si % NVT;
            const int col = cb + 16 * vt + r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = 16 * ct + 4 * g4 + i;
                p.sfin[sbase + (int64_t)c * p.dvt + col] = S[m][i];
            }
        }
    }
}

// ---------------------------------------------------------------------------
template <class C>
static hipError_t launch_cfg(const PrefillArgs& a) {
    PrefillParams p;
    p.H = a.H;
    p.num_seqs = a.num_seqs;
    p.nchains = a.num_seqs * a.H;
    p.dvt = C::AUG ? a.dk + a.dv : a.dv;
    p.nslices = p.dvt / C::VS;
    p.final_seq_lo = a.final_seq_lo;
    p.scale = a.scale;
    p.T_total = a.T_total;
    p.seg_len = a.seg_len;
    p.cu_seqlens = a.cu_seqlens;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.g = a.g;
    p.beta = a.beta;
    p.z = a.z;
    p.s0 = a.initial_state;
    p.sfin = a.final_state;
    p.y = a.y;
    if (p.nchains == 0) return hipSuccess;
    const long nblk = (long)((p.nchains + 7) / 8) * 8 * p.nslices;
    hipLaunchKernelGGL((prefill_kernel<C>), dim3((unsigned)nblk), dim3(C::NTHR), 0,
                       (hipStream_t)a.stream, p);
    return hipGetLastError();
}

template <class E, int DK, int CH, int MODE>
static hipError_t launch_vs(const PrefillArgs& a, int vs) {
    if constexpr (PfCfg<E, DK, 64, CH, MODE>::FITS) {
        if (vs != 32) return launch_cfg<PfCfg<E, DK, 64, CH, MODE>>(a);
    }
    return launch_cfg<PfCfg<E, DK, 32, CH, MODE>>(a);
}

template <class E, int DK, int CH>
static hipError_t launch_mode(const PrefillArgs& a, int vs) {
    switch (a.mode) {
        case kModeSeq: return launch_vs<E, DK, CH, kModeSeq>(a, vs);
        case kModeVarlen: return launch_vs<E, DK, CH, kModeVarlen>(a, vs);
        case kModePairs: return launch_vs<E, DK, CH, kModePairs>(a, vs);
        default: return launch_vs<E, DK, CH, kModeFinish>(a, vs);
    }
}

bool prefill_supported(int dtype, int dk, int dv, int chunk) {
    if (!((dk == 64 && dv == 64) || (dk == 128 && dv == 128))) return false;
    if (chunk != 16 && chunk != 64) return false;
    if (dtype == 1 && dk == 128 && chunk == 64) return false;  // fp32 tiles exceed LDS
    return dtype == 0 || dtype == 1;
}

hipError_t launch_prefill(const PrefillArgs& a) {
    int vs = a.vs;
    if (vs != 32 && vs != 64) {
        // wide slices (fewer repeats of the key-side work) unless that leaves
        // most compute units without a workgroup
        const long chains = (long)a.num_seqs * a.H;
        const long wide = chains * ((a.mode == 2 ? a.dk + a.dv : a.dv) / 64);
        vs = wide >= 128 ? 64 : 32;
    }
    if (a.dtype == 0) {
        if (a.dk == 128)
            return a.chunk == 64 ? launch_mode<BF16, 128, 64>(a, vs) : launch_mode<BF16, 128, 16>(a, vs);
        return a.chunk == 64 ? launch_mode<BF16, 64, 64>(a, vs) : launch_mode<BF16, 64, 16>(a, vs);
    }
    if (a.dk == 128) return launch_mode<F32, 128, 16>(a, vs);
    return a.chunk == 64 ? launch_mode<F32, 64, 64>(a, vs) : launch_mode<F32, 64, 16>(a, vs);
}

}  // namespace kda
