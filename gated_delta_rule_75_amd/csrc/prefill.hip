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
    static constexpr int NG = NTHR / (DK / 2);  // token groups of the decay phase
    static constexpr int L = CH / NG;           // tokens per thread in that phase
    static constexpr int GPT = 16 / L;          // token groups per 16-token tile
    static constexpr int NOT = NT * NVT;        // (t, v) tiles of R, Delta and O
    static constexpr int OPW = (NOT + 3) / 4;   // R / O tiles per wave of a 4-wave group
    static constexpr int DPW = (NOT + NW - 1) / NW;  // Delta tiles per wave
    static constexpr int NST = NCT * NVT;       // (c, v) state tiles
    static constexpr int SPW = NST / 4;         // state tiles per wave of waves 0-3
    static constexpr int NPAIR = NT * (NT + 1) / 2;
    static constexpr int NTASK = AUG ? NPAIR : 2 * NPAIR;
    static_assert(NT == 1 || NT == 4, "chunk of 16 or 64 tokens");
    static_assert(L >= 1 && 16 % L == 0, "decay-phase token groups must tile 16");
    static_assert(NST % 4 == 0, "state tiles per wave");

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
    static constexpr size_t O_GS = O_RT + al((size_t)VS * LCH * sizeof(T));
    static constexpr size_t O_ES = O_GS + (size_t)NG * DK * 4;
    static constexpr size_t O_D = O_ES + (size_t)NT * DK * 4;
    static constexpr size_t O_EGC = O_D + (size_t)NT * NT * DK * 4;
    static constexpr size_t O_BETA = O_EGC + (size_t)DK * 4;
    static constexpr size_t O_MISC = O_BETA + (size_t)CH * 4;
    static constexpr size_t BYTES = O_MISC + 16;
    // aliases of regions that are dead while they are used
    static constexpr size_t O_TT = O_KC;   // L^{-1} transposed, during the inverse only
    static constexpr size_t O_YT = O_GS;   // per-wave 16x16 scratch of the inverse
    static constexpr size_t O_DT = O_N;    // Delta^T, after the inverse
    static constexpr size_t O_SORT = O_KR; // sequence lengths, before the first chunk
    static constexpr bool FITS = BYTES <= 160 * 1024 &&
        (size_t)CH * LCH * sizeof(T) <= SZ_OP &&
        (NT == 1 || (size_t)3 * 16 * (16 + PADE) * sizeof(T) <= (size_t)NG * DK * 4);
};

// Pairs of consecutive channels of q / k as loaded from global memory.
template <typename T> struct Pair2;
template <> struct Pair2<__bf16> { using type = bf16x2_t; };
template <> struct Pair2<float> { using type = f32x2_t; };

__device__ __forceinline__ void st_pair(__bf16* p, float a, float b) {
    *reinterpret_cast<bf16x2_t*>(p) = bf16x2_t{(__bf16)a, (__bf16)b};
}
__device__ __forceinline__ void st_pair(float* p, float a, float b) {
    *reinterpret_cast<f32x2_t*>(p) = f32x2_t{a, b};
}

// n consecutive elements (n*sizeof(T) a multiple of 4, 4-byte aligned).
template <int n>
__device__ __forceinline__ void st_row(__bf16* p, const float* v) {
    if constexpr (n % 8 == 0) {
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
#pragma unroll
    for (int i = 0; i < n; ++i) p[i] = v[i];
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
__global__ __launch_bounds__(C::NTHR) void prefill_kernel(PrefillParams p) {
    using E = typename C::E;
    using T = typename C::T;
    using T2 = typename Pair2<T>::type;
    constexpr int DK = C::DK, VS = C::VS, CH = C::CH, NT = C::NT, NVT = C::NVT;
    constexpr int LDK = C::LDK, LCH = C::LCH, LN = C::LN, L = C::L, GPT = C::GPT, NG = C::NG;
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
    float* sGs = reinterpret_cast<float*>(smem + C::O_GS);
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

    // ---- decay-phase thread mapping: channel pair cp, token group tg --------
    const int cp = tid % (DK / 2), tg = tid / (DK / 2);
    const int c0 = 2 * cp;
    const int tile = tg / GPT, gi = tg % GPT;

    T2 rq[L], rk[L];
    f32x2_t rgv[L];
    float rbeta = 0.f;
    // v (waves 0-3, R tiles) or z (waves 4-7, output tiles) in MMA-output layout
    float vz[C::OPW][4];
    const int64_t tclamp = len > 0 ? len - 1 : 0;
    const int HDK = H * DK, HDV = H * DV;   // token strides (elements)
    // Global addresses: a 64-bit row base per chunk plus 32-bit in-chunk offsets.
    // Loads are unconditional from clamped rows; invalid tokens are masked at use.
    auto load_qkg = [&](int64_t cs) {
        const int64_t row = (t0 + cs) * H + h;
        const int last = (int)(tclamp - cs);   // >= 0 while cs < len
        const T* kb = gk + row * DK + c0;
        const T* qb = gq + row * DK + c0;
        const float* gb = p.g + row * DK + c0;
#pragma unroll
        for (int l = 0; l < L; ++l) {
            const int tr = tg * L + l < last ? tg * L + l : last;
            rk[l] = *reinterpret_cast<const T2*>(kb + tr * HDK);
            if (!AUG) rq[l] = *reinterpret_cast<const T2*>(qb + tr * HDK);
            rgv[l] = *reinterpret_cast<const f32x2_t*>(gb + tr * HDK);
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
            const T* src = (lowg ? gv : gz) + row * DV + vcol0 + r16;
#pragma unroll
            for (int m = 0; m < C::OPW; ++m) {
                int ta, vt;
                ro_tile<C>(gw, m, ta, vt);
                const int vtc = vt < NVT ? vt : 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * ta + 4 * g4 + i;
                    const int tr = t < last ? t : last;
                    vz[m][i] = gload(src + tr * HDV + 16 * vtc);
                }
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
        // ================= phase 1: decay prefix and scaled operands ==========
        // Thread (tg, cp) holds tokens tg*L .. tg*L+L-1 of channels c0, c0+1.
        float cpv[2][L], sfv[2][L];
        float gsum2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            float al[L], pr = 1.f, gs = 0.f;
#pragma unroll
            for (int l = 0; l < L; ++l) {
                const bool valid = tg * L + l < nvalid;
                const float gv_ = valid ? rgv[l][e] : 0.f;
                al[l] = fast_exp(gv_);
                pr *= al[l];
                cpv[e][l] = pr;          // e^{G_t - G_first + g_first}
                gs += gv_;
            }
            sfv[e][L - 1] = 1.f;
#pragma unroll
            for (int l = L - 2; l >= 0; --l) sfv[e][l] = sfv[e][l + 1] * al[l + 1];
            gsum2[e] = gs;
        }
        st_pair(sGs + tg * DK + c0, gsum2[0], gsum2[1]);
        if (tid < CH) sBeta[tid] = tid < nvalid ? rbeta : 0.f;
        __syncthreads();
        {
            float E1[2], E2[2], E3[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int c = c0 + e;
                float gsum[NG];
#pragma unroll
                for (int q2 = 0; q2 < NG; ++q2) gsum[q2] = sGs[q2 * DK + c];
                float Sref[NT + 1];
                Sref[0] = 0.f;
#pragma unroll
                for (int a = 0; a < NT; ++a) {
                    float s = 0.f;
#pragma unroll
                    for (int q2 = 0; q2 < GPT; ++q2) s += gsum[a * GPT + q2];
                    Sref[a + 1] = Sref[a] + s;
                }
                float off = 0.f;
#pragma unroll
                for (int q2 = 0; q2 < NG; ++q2)
                    if (q2 >= tile * GPT && q2 < tg) off += gsum[q2];
                const float Sa = Sref[tile], GC = Sref[NT];
                E1[e] = fast_exp(off);                        // times cpv: e^{G_t - R_a}  (<= 1)
                E2[e] = fast_exp(-off - gsum2[e]);            // times sfv: e^{R_a - G_t}  (<= e^80)
                E3[e] = fast_exp(GC - Sa - off - gsum2[e]);   // times sfv: e^{G_C - G_t}  (<= 1)
                if (tg == 0) {
                    // per-channel tables: e^{R_a}, e^{R_a - R_b} (b < a), e^{G_C}
#pragma unroll
                    for (int a = 0; a < NT; ++a) {
                        sES[a * DK + c] = fast_exp(Sref[a]);
#pragma unroll
                        for (int bb = 0; bb < a; ++bb)
                            sD[(a * NT + bb) * DK + c] = fast_exp(Sref[a] - Sref[bb]);
                    }
                    sEGC[c] = fast_exp(GC);
                }
            }
            float kt0[L], kt1[L];
#pragma unroll
            for (int l = 0; l < L; ++l) {
                const int t = tg * L + l;
                const bool valid = t < nvalid;
                const float k0 = valid ? to_f32(rk[l][0]) : 0.f, k1 = valid ? to_f32(rk[l][1]) : 0.f;
                const float f10 = E1[0] * cpv[0][l], f11 = E1[1] * cpv[1][l];
                st_pair(sKr + t * LDK + c0, k0 * f10, k1 * f11);
                if (!AUG) {
                    const float q0 = valid ? to_f32(rq[l][0]) : 0.f, q1 = valid ? to_f32(rq[l][1]) : 0.f;
                    st_pair(sQr + t * LDK + c0, q0 * f10, q1 * f11);
                }
                st_pair(sKc + t * LDK + c0, k0 * (E2[0] * sfv[0][l]), k1 * (E2[1] * sfv[1][l]));
                kt0[l] = k0 * (E3[0] * sfv[0][l]);
                kt1[l] = k1 * (E3[1] * sfv[1][l]);
            }
            st_row<L>(sKt + c0 * LCH + tg * L, kt0);
            st_row<L>(sKt + (c0 + 1) * LCH + tg * L, kt1);
        }
        // prefetch the next chunk's q, k, g, beta while this one computes
        if (ch + 1 < nchunks) load_qkg(cs + CH);
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
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
            for (int kk = 0; kk < DK; kk += KS) {
                const typename E::Frag fa = lds_frag<E>(X, LDK, 16 * a, kk, lane);
                const typename E::Frag fb = (bb < a)
                    ? lds_frag_scaled<E>(sKc, LDK, 16 * bb, kk, lane, sD + (a * NT + bb) * DK)
                    : lds_frag<E>(sKc, LDK, 16 * bb, kk, lane);
                acc = E::mma(fa, fb, acc);
            }
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
#pragma unroll 2
            for (int kk = 0; kk < DK; kk += KS) {
                const typename E::Frag fa = lds_frag_scaled<E>(sKr, LDK, 16 * ta0, kk, lane, sES + ta0 * DK);
#pragma unroll
                for (int m = 0; m < C::OPW; ++m) {
                    int ta, vt;
                    ro_tile<C>(gw, m, ta, vt);
                    if (vt < NVT) ak[m] = E::mma(fa, lds_frag<E>(sSt, LDK, 16 * vt, kk, lane), ak[m]);
                }
            }
#pragma unroll
            for (int m = 0; m < C::OPW; ++m) {
                int ta, vt;
                ro_tile<C>(gw, m, ta, vt);
                if (vt < NVT) {
                    T rv[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = 16 * ta + 4 * g4 + i;
                        const float vv = ident ? 0.f : vz[m][i];
                        rv[i] = from_f32<T>(sBeta[t] * (vv - ak[m][i]));
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) sRt[(16 * vt + r16) * LCH + 16 * ta + 4 * g4 + i] = rv[i];
                }
            }
            if (ch + 1 < nchunks) load_vz(cs + CH);   // v of the next chunk
        } else if (wave == 4 && lane < 16 * NT) {
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
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
                const int kend = 16 * (ta + 1);
#pragma unroll
                for (int kk = 0; kk < CH; kk += KS)
                    if (kk < kend)
                        acc = E::mma(lds_frag_lim<E>(sT, LCH, 16 * ta, kk, lane, CH),
                                     lds_frag_lim<E>(sRt, LCH, 16 * vt, kk, lane, CH), acc);
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
#pragma unroll
            for (int m = 0; m < C::SPW; ++m) {
                const int si = gw + 4 * m, ct = si / NVT;
#pragma unroll
                for (int i = 0; i < 4; ++i) S[m][i] *= sEGC[16 * ct + 4 * g4 + i];
            }
#pragma unroll
            for (int kk = 0; kk < CH; kk += KS) {
#pragma unroll
                for (int m = 0; m < C::SPW; ++m) {
                    const int si = gw + 4 * m, ct = si / NVT, vt = si % NVT;
                    S[m] = E::mma(lds_frag_lim<E>(sKt, LCH, 16 * ct, kk, lane, CH),
                                  lds_frag_lim<E>(sDt, LCH, 16 * vt, kk, lane, CH), S[m]);
                }
            }
        } else if (!AUG) {
            // O = (Q e^G) S_old + P Delta, y = scale O sigmoid(z)
            f32x4_t ao[C::OPW];
#pragma unroll
            for (int m = 0; m < C::OPW; ++m) ao[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            int ta0, vt0;
            ro_tile<C>(gw, 0, ta0, vt0);
#pragma unroll 2
            for (int kk = 0; kk < DK; kk += KS) {
                const typename E::Frag fa = lds_frag_scaled<E>(sQr, LDK, 16 * ta0, kk, lane, sES + ta0 * DK);
#pragma unroll
                for (int m = 0; m < C::OPW; ++m) {
                    int ta, vt;
                    ro_tile<C>(gw, m, ta, vt);
                    if (vt < NVT) ao[m] = E::mma(fa, lds_frag<E>(sSt, LDK, 16 * vt, kk, lane), ao[m]);
                }
            }
            T* ychunk = gy + ((t0 + cs) * H + h) * DV + vcol0 + r16;
            const int kend = 16 * (ta0 + 1);
#pragma unroll
            for (int kk = 0; kk < CH; kk += KS) {
                if (kk < kend) {
                    const typename E::Frag fa = lds_frag_lim<E>(sP, LCH, 16 * ta0, kk, lane, CH);
#pragma unroll
                    for (int m = 0; m < C::OPW; ++m) {
                        int ta, vt;
                        ro_tile<C>(gw, m, ta, vt);
                        if (vt < NVT) ao[m] = E::mma(fa, lds_frag_lim<E>(sDt, LCH, 16 * vt, kk, lane, CH), ao[m]);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < C::OPW; ++m) {
                int ta, vt;
                ro_tile<C>(gw, m, ta, vt);
                if (vt < NVT) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = 16 * ta + 4 * g4 + i;
                        if (t < nvalid) {
                            float o = p.scale * ao[m][i];
                            if (gated) o *= sigmoid(vz[m][i]);
                            gstore(ychunk + t * HDV + 16 * vt, o);
                        }
                    }
                }
            }
            if (gated && ch + 1 < nchunks) load_vz(cs + CH);   // z of the next chunk
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
