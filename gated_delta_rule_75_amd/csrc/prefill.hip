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

template <typename E_, int DK_, int VS_, int CH_, bool AUG_>
struct PfCfg {
    using E = E_;
    using T = typename E::T;
    static constexpr int DK = DK_, VS = VS_, CH = CH_;
    static constexpr bool AUG = AUG_;
    static constexpr int NT = CH / 16, NCT = DK / 16, NVT = VS / 16;
    static constexpr int PADE = 16 / (int)sizeof(T);
    static constexpr int LDK = DK + PADE;  // pitch of [.][DK] operand arrays
    static constexpr int LCH = CH + PADE;  // pitch of [.][CH] operand arrays
    static constexpr int LN = CH + 4;      // pitch of the fp32 N array
    static constexpr int NW = 4, NTHR = 256;
    static constexpr int NG = NTHR / (DK / 2);  // token groups of the decay phase
    static constexpr int L = CH / NG;           // tokens per thread in that phase
    static constexpr int GPT = 16 / L;          // token groups per 16-token tile
    static constexpr int NOT = NT * NVT;        // output (t, v) tiles
    static constexpr int OPW = (NOT + NW - 1) / NW;
    static constexpr int NST = NCT * NVT;       // state (c, v) tiles
    static constexpr int SPW = NST / NW;
    static constexpr int NPAIR = NT * (NT + 1) / 2;
    static constexpr int NTASK = AUG ? NPAIR : 2 * NPAIR;
    static_assert(L >= 1 && 16 % L == 0, "decay-phase token groups must tile 16");
    static_assert(NST % NW == 0, "state tiles per wave");

    static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
    static constexpr size_t SZ_OP = (size_t)CH * LDK * sizeof(T);
    static constexpr size_t O_KR = 0;
    static constexpr size_t O_QR = O_KR + SZ_OP;
    static constexpr size_t O_KC = O_QR + SZ_OP;
    static constexpr size_t O_KT = O_KC + SZ_OP;
    static constexpr size_t O_ST = O_KT + al((size_t)DK * LCH * sizeof(T));
    static constexpr size_t O_N = O_ST + al((size_t)VS * LDK * sizeof(T));
    static constexpr size_t SZ_N0 = (size_t)CH * LN * 4, SZ_N1 = (size_t)VS * LCH * sizeof(T);
    static constexpr size_t O_T = O_N + al(SZ_N0 > SZ_N1 ? SZ_N0 : SZ_N1);
    static constexpr size_t O_P = O_T + al((size_t)CH * LCH * sizeof(T));
    static constexpr size_t O_RT = O_P + al((size_t)CH * LCH * sizeof(T));
    static constexpr size_t O_GS = O_RT + al((size_t)VS * LCH * sizeof(T));
    static constexpr size_t O_ES = O_GS + (size_t)NG * DK * 4;
    static constexpr size_t O_TAU = O_ES + (size_t)NT * DK * 4;
    static constexpr size_t O_F = O_TAU + (size_t)NT * DK * 4;
    static constexpr size_t O_EGC = O_F + (size_t)NT * NT * DK * 4;
    static constexpr size_t O_BETA = O_EGC + (size_t)DK * 4;
    static constexpr size_t O_MISC = O_BETA + (size_t)CH * 4;
    static constexpr size_t BYTES = O_MISC + 16;
    // aliases of regions that are dead while they are used
    static constexpr size_t O_TT = O_KR;   // L^{-1} transposed, during the inverse only
    static constexpr size_t O_YT = O_QR;   // per-wave 16x16 scratch of the inverse
    static constexpr size_t O_DT = O_N;    // Delta^T, after the inverse
    static constexpr size_t O_SORT = O_KR; // sequence lengths / ranks, before the first chunk
    static_assert((size_t)CH * LCH * sizeof(T) <= SZ_OP, "L^-1 transpose fits the Kr region");
    static_assert(NT == 1 || (size_t)NW * 16 * (16 + PADE) * sizeof(T) <= SZ_OP, "inverse scratch fits");
    static_assert(BYTES <= 160 * 1024, "LDS budget of a gfx950 workgroup");
};

// Pairs of consecutive channels of q / k as loaded from global memory.
template <typename T> struct Pair2;
template <> struct Pair2<__bf16> { using type = bf16x2_t; };
template <> struct Pair2<float> { using type = f32x2_t; };

template <typename T>
__device__ __forceinline__ f32x2_t pair_f32(const typename Pair2<T>::type& p) {
    return f32x2_t{to_f32(p[0]), to_f32(p[1])};
}

// 16x16x16 product acc += A[16 x 16] B[16 x 16]^T-stored, operands in LDS:
// A rows r (k contiguous, fp32 or element type), B stored as rows = output
// columns with k contiguous (element type).
template <typename E, typename TA>
__device__ __forceinline__ f32x4_t mma16(f32x4_t acc, const TA* A, int lda,
                                         const typename E::T* B, int ldb, int lane) {
    const int r = lane & 15, gq = lane >> 4;
#pragma unroll
    for (int k0 = 0; k0 < 16; k0 += E::KSTEP) {
        typename E::Frag fa, fb;
#pragma unroll
        for (int e = 0; e < E::KPL; ++e) {
            const int kk = k0 + E::KPL * gq + e;
            const bool in = kk < 16;
            frag_set<E>(fa, e, in ? to_f32(A[r * lda + (in ? kk : 0)]) : 0.f);
            frag_set<E>(fb, e, in ? to_f32(B[r * ldb + (in ? kk : 0)]) : 0.f);
        }
        acc = E::mma(fa, fb, acc);
    }
    return acc;
}

template <class C>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillParams p) {
    using E = typename C::E;
    using T = typename C::T;
    using T2 = typename Pair2<T>::type;
    constexpr int DK = C::DK, VS = C::VS, CH = C::CH, NT = C::NT, NVT = C::NVT;
    constexpr int LDK = C::LDK, LCH = C::LCH, LN = C::LN, L = C::L, GPT = C::GPT, NG = C::NG;
    constexpr int KS = E::KSTEP;
    constexpr bool AUG = C::AUG;

    __shared__ __attribute__((aligned(16))) char smem[C::BYTES];
    T* sKr = reinterpret_cast<T*>(smem + C::O_KR);
    T* sQr = reinterpret_cast<T*>(smem + C::O_QR);
    T* sKc = reinterpret_cast<T*>(smem + C::O_KC);
    T* sKt = reinterpret_cast<T*>(smem + C::O_KT);
    T* sSt = reinterpret_cast<T*>(smem + C::O_ST);
    float* sN = reinterpret_cast<float*>(smem + C::O_N);
    T* sDt = reinterpret_cast<T*>(smem + C::O_DT);
    T* sT = reinterpret_cast<T*>(smem + C::O_T);
    T* sTt = reinterpret_cast<T*>(smem + C::O_TT);
    T* sYt = reinterpret_cast<T*>(smem + C::O_YT);
    T* sP = reinterpret_cast<T*>(smem + C::O_P);
    T* sRt = reinterpret_cast<T*>(smem + C::O_RT);
    float* sGs = reinterpret_cast<float*>(smem + C::O_GS);
    float* sES = reinterpret_cast<float*>(smem + C::O_ES);
    float* sTau = reinterpret_cast<float*>(smem + C::O_TAU);
    float* sF = reinterpret_cast<float*>(smem + C::O_F);
    float* sEGC = reinterpret_cast<float*>(smem + C::O_EGC);
    float* sBeta = reinterpret_cast<float*>(smem + C::O_BETA);
    int* sMisc = reinterpret_cast<int*>(smem + C::O_MISC);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g4 = lane >> 4;

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
        for (int i = tid; i < p.num_seqs; i += C::NTHR) sLen[i] = p.cu_seqlens[i + 1] - p.cu_seqlens[i];
        __syncthreads();
        for (int i = tid; i < p.num_seqs; i += C::NTHR) {
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
    const int vcol0 = AUG ? (cb - DK) : cb;    // column of v feeding this slice
    const int DV = AUG ? p.dvt - DK : p.dvt;   // row width of v / z / y

    const T* gq = static_cast<const T*>(p.q);
    const T* gk = static_cast<const T*>(p.k);
    const T* gv = static_cast<const T*>(p.v);
    const T* gz = static_cast<const T*>(p.z);
    T* gy = static_cast<T*>(p.y);

    // ---- state tiles owned by this wave: (ct, vt) = si / NVT, si % NVT -----
    f32x4_t S[C::SPW];
    {
        const int64_t sbase = ((int64_t)n * H + h) * DK * (int64_t)p.dvt;
#pragma unroll
        for (int m = 0; m < C::SPW; ++m) {
            const int si = wave + C::NW * m, ct = si / NVT, vt = si % NVT;
            const int col = cb + 16 * vt + r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = 16 * ct + 4 * g4 + i;
                float s = 0.f;
                if (AUG) s = (col == c) ? 1.f : 0.f;
                else if (p.s0) s = p.s0[sbase + (int64_t)c * p.dvt + col];
                S[m][i] = s;
            }
        }
    }
    // zero the upper-triangular blocks of P and L^{-1} (never written later)
    for (int idx = tid; idx < CH * CH; idx += C::NTHR) {
        const int t = idx / CH, j = idx % CH;
        if ((j >> 4) > (t >> 4)) {
            sT[t * LCH + j] = from_f32<T>(0.f);
            sP[t * LCH + j] = from_f32<T>(0.f);
        }
    }
    __syncthreads();  // also orders the sort scratch before its region is reused

    // ---- decay-phase thread mapping: channel pair cp, token group tg --------
    const int cp = tid % (DK / 2), tg = tid / (DK / 2);
    const int c0 = 2 * cp;
    const int tile = tg / GPT, gi = tg % GPT;

    T2 rq[L], rk[L];
    f32x2_t rgv[L];
    float rbeta = 0.f;
    auto load_chunk = [&](int64_t cs) {
#pragma unroll
        for (int l = 0; l < L; ++l) {
            const int64_t tt = cs + tg * L + l;
            const bool valid = tt < len;
            const int64_t base = ((t0 + (valid ? tt : 0)) * H + h) * DK + c0;
            if (valid) {
                rk[l] = *reinterpret_cast<const T2*>(gk + base);
                if (!AUG) rq[l] = *reinterpret_cast<const T2*>(gq + base);
                rgv[l] = *reinterpret_cast<const f32x2_t*>(p.g + base);
            } else {
                rk[l] = T2{from_f32<T>(0.f), from_f32<T>(0.f)};
                rq[l] = rk[l];
                rgv[l] = f32x2_t{0.f, 0.f};
            }
        }
        if (tid < CH) {
            const int64_t tt = cs + tid;
            rbeta = tt < len ? p.beta[(t0 + tt) * H + h] : 0.f;
        }
    };

    const int64_t nchunks = (len + CH - 1) / CH;
    if (nchunks > 0) load_chunk(0);

    // initial S^T (element type) for the first chunk's state products
#pragma unroll
    for (int m = 0; m < C::SPW; ++m) {
        const int si = wave + C::NW * m, ct = si / NVT, vt = si % NVT;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sSt[(16 * vt + r16) * LDK + 16 * ct + 4 * g4 + i] = from_f32<T>(S[m][i]);
    }

    f32x4_t O[C::OPW];
    float vreg[C::OPW][4], zreg[C::OPW][4];

    for (int64_t ch = 0; ch < nchunks; ++ch) {
        const int64_t cs = ch * CH;
        // v and z of the output tiles this wave owns, in MMA-output layout
#pragma unroll
        for (int m = 0; m < C::OPW; ++m) {
            const int ti = wave + C::NW * m;
            const int ta = ti / NVT, vt = ti % NVT;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t tt = cs + 16 * ta + 4 * g4 + i;
                const bool valid = ti < C::NOT && tt < len;
                const int64_t off = ((t0 + (valid ? tt : 0)) * H + h) * (int64_t)DV + vcol0 + 16 * vt + r16;
                vreg[m][i] = (valid && !ident) ? gload(gv + off) : 0.f;
                zreg[m][i] = (valid && !AUG && gz) ? gload(gz + off) : 0.f;
            }
        }

        // ================= phase 1: decay prefix and scaled operands ==========
        float al0[L], al1[L], cp0[L], cp1[L], sf0[L], sf1[L];
        float gs0 = 0.f, gs1 = 0.f;
        {
            float pr0 = 1.f, pr1 = 1.f;
#pragma unroll
            for (int l = 0; l < L; ++l) {
                al0[l] = fast_exp(rgv[l][0]);
                al1[l] = fast_exp(rgv[l][1]);
                pr0 *= al0[l];
                pr1 *= al1[l];
                cp0[l] = pr0;
                cp1[l] = pr1;
                gs0 += rgv[l][0];
                gs1 += rgv[l][1];
            }
            sf0[L - 1] = 1.f;
            sf1[L - 1] = 1.f;
#pragma unroll
            for (int l = L - 2; l >= 0; --l) {
                sf0[l] = sf0[l + 1] * al0[l + 1];
                sf1[l] = sf1[l + 1] * al1[l + 1];
            }
        }
        sGs[tg * DK + c0] = gs0;
        sGs[tg * DK + c0 + 1] = gs1;
        if (tid < CH) sBeta[tid] = rbeta;
        __syncthreads();
        {
            float gsum[2][NG];
#pragma unroll
            for (int q2 = 0; q2 < NG; ++q2) {
                gsum[0][q2] = sGs[q2 * DK + c0];
                gsum[1][q2] = sGs[q2 * DK + c0 + 1];
            }
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int c = c0 + e;
                float tileTot[NT], Sref[NT + 1];
#pragma unroll
                for (int a = 0; a < NT; ++a) {
                    float s = 0.f;
#pragma unroll
                    for (int q2 = 0; q2 < GPT; ++q2) s += gsum[e][a * GPT + q2];
                    tileTot[a] = s;
                }
                Sref[0] = 0.f;
#pragma unroll
                for (int a = 0; a < NT; ++a) Sref[a + 1] = Sref[a] + tileTot[a];
                float off = 0.f;
#pragma unroll
                for (int q2 = 0; q2 < NG; ++q2)
                    if (q2 >= tile * GPT && q2 < tg) off += gsum[e][q2];
                const float Sa = Sref[tile], GC = Sref[NT];
                const float gs = e ? gs1 : gs0;
                const float E1 = fast_exp(off);                   // e^{G_first - R_a} / alpha_first
                const float E2 = fast_exp(-off - gs);             // e^{R_a - G_last}
                const float E3 = fast_exp(GC - Sa - off - gs);    // e^{G_C - G_last}
                const float* cpv = e ? cp1 : cp0;
                const float* sfv = e ? sf1 : sf0;
                T ktv[L];
#pragma unroll
                for (int l = 0; l < L; ++l) {
                    const int t = tg * L + l;
                    const float kv = to_f32(rk[l][e]);
                    const float f1 = E1 * cpv[l];   // e^{G_t - R_a}  (<= 1)
                    const float f2 = E2 * sfv[l];   // e^{R_a - G_t}  (<= e^80)
                    const float f3 = E3 * sfv[l];   // e^{G_C - G_t}  (<= 1)
                    sKr[t * LDK + c] = from_f32<T>(kv * f1);
                    if (!AUG) sQr[t * LDK + c] = from_f32<T>(to_f32(rq[l][e]) * f1);
                    sKc[t * LDK + c] = from_f32<T>(kv * f2);
                    ktv[l] = from_f32<T>(kv * f3);
                }
#pragma unroll
                for (int l = 0; l < L; ++l) sKt[c * LCH + tg * L + l] = ktv[l];
                if (gi == 0) {
                    sES[tile * DK + c] = fast_exp(Sa);
                    sTau[tile * DK + c] = fast_exp(tileTot[tile]);
#pragma unroll
                    for (int bb = 0; bb + 1 < tile; ++bb)
                        sF[(tile * NT + bb) * DK + c] = fast_exp(Sa - Sref[bb + 1]);
                    if (tile == 0) sEGC[c] = fast_exp(GC);
                }
            }
        }
        // prefetch the next chunk's q, k, g, beta while this one computes
        if (ch + 1 < nchunks) load_chunk(cs + CH);
        __syncthreads();

        // ================= phase 2: gated Gram blocks A (and P) ==============
        for (int task = wave; task < C::NTASK; task += C::NW) {
            const int mat = task / C::NPAIR;  // 0: A (keys), 1: P (queries)
            const int pi = task % C::NPAIR;
            int a = 0;
            while ((a + 1) * (a + 2) / 2 <= pi) ++a;
            const int bb = pi - a * (a + 1) / 2;
            const T* X = mat ? sQr : sKr;
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < DK; kk += KS) {
                typename E::Frag fa = (bb + 1 < a)
                    ? lds_frag_scaled<E>(X, LDK, 16 * a, kk, lane, sF + (a * NT + bb) * DK)
                    : lds_frag<E>(X, LDK, 16 * a, kk, lane);
                typename E::Frag fb = (bb < a)
                    ? lds_frag_scaled<E>(sKc, LDK, 16 * bb, kk, lane, sTau + bb * DK)
                    : lds_frag<E>(sKc, LDK, 16 * bb, kk, lane);
                acc = E::mma(fa, fb, acc);
            }
            const int j = 16 * bb + r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * a + 4 * g4 + i;
                if (mat == 0) {
                    const bool keep = bb < a || j < t;
                    sN[t * LN + j] = keep ? sBeta[t] * acc[i] : 0.f;
                } else {
                    const bool keep = bb < a || j <= t;
                    sP[t * LCH + j] = from_f32<T>(keep ? acc[i] : 0.f);
                }
            }
        }
        __syncthreads();

        // ================= phase 3: R = beta (V - (K e^G) S), O = (Q e^G) S ===
#pragma unroll
        for (int m = 0; m < C::OPW; ++m) {
            const int ti = wave + C::NW * m;
            if (ti < C::NOT) {
                const int ta = ti / NVT, vt = ti % NVT;
                f32x4_t ak = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < DK; kk += KS) {
                    const typename E::Frag fb = lds_frag<E>(sSt, LDK, 16 * vt, kk, lane);
                    ak = E::mma(lds_frag_scaled<E>(sKr, LDK, 16 * ta, kk, lane, sES + ta * DK), fb, ak);
                    if (!AUG)
                        aq = E::mma(lds_frag_scaled<E>(sQr, LDK, 16 * ta, kk, lane, sES + ta * DK), fb, aq);
                }
                O[m] = aq;
                T rv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * ta + 4 * g4 + i;
                    rv[i] = from_f32<T>(sBeta[t] * (vreg[m][i] - ak[i]));
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) sRt[(16 * vt + r16) * LCH + 16 * ta + 4 * g4 + i] = rv[i];
            }
        }
        __syncthreads();

        // ================= phase 4: L^{-1}, L = I + N (N = diag(beta) A) ======
        if (wave == 0 && lane < 16 * NT) {
            // diagonal 16x16 blocks by forward substitution, one column per lane
            const int a = lane >> 4, jj = lane & 15;
            const float* Nb = sN + (16 * a) * LN + 16 * a;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < i; ++m) acc += Nb[i * LN + m] * x[m];
                x[i] = (i > jj) ? -acc : (i == jj ? 1.f : 0.f);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const T xv = from_f32<T>(x[i]);
                sT[(16 * a + i) * LCH + 16 * a + jj] = xv;
                if (NT > 1) sTt[(16 * a + jj) * LCH + 16 * a + i] = xv;
            }
        }
        __syncthreads();
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
        for (int m = 0; m < C::OPW; ++m) {
            const int ti = wave + C::NW * m;
            if (ti < C::NOT) {
                const int ta = ti / NVT, vt = ti % NVT;
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
                const int kend = 16 * (ta + 1);
#pragma unroll
                for (int kk = 0; kk < CH; kk += KS)
                    if (kk < kend)
                        acc = E::mma(lds_frag<E>(sT, LCH, 16 * ta, kk, lane),
                                     lds_frag<E>(sRt, LCH, 16 * vt, kk, lane), acc);
                T dv4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) dv4[i] = from_f32<T>(acc[i]);
#pragma unroll
                for (int i = 0; i < 4; ++i) sDt[(16 * vt + r16) * LCH + 16 * ta + 4 * g4 + i] = dv4[i];
            }
        }
        __syncthreads();

        // ================= phase 6: outputs and state update ==================
        if (!AUG) {
#pragma unroll
            for (int m = 0; m < C::OPW; ++m) {
                const int ti = wave + C::NW * m;
                if (ti < C::NOT) {
                    const int ta = ti / NVT, vt = ti % NVT;
                    f32x4_t acc = O[m];
                    const int kend = 16 * (ta + 1);
#pragma unroll
                    for (int kk = 0; kk < CH; kk += KS)
                        if (kk < kend)
                            acc = E::mma(lds_frag<E>(sP, LCH, 16 * ta, kk, lane),
                                         lds_frag<E>(sDt, LCH, 16 * vt, kk, lane), acc);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t tt = cs + 16 * ta + 4 * g4 + i;
                        if (tt < len) {
                            float o = p.scale * acc[i];
                            if (gz) o *= sigmoid(zreg[m][i]);
                            gstore(gy + ((t0 + tt) * H + h) * (int64_t)DV + vcol0 + 16 * vt + r16, o);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int m = 0; m < C::SPW; ++m) {
            const int si = wave + C::NW * m, ct = si / NVT, vt = si % NVT;
            f32x4_t acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = sEGC[16 * ct + 4 * g4 + i] * S[m][i];
#pragma unroll
            for (int kk = 0; kk < CH; kk += KS)
                acc = E::mma(lds_frag<E>(sKt, LCH, 16 * ct, kk, lane),
                             lds_frag<E>(sDt, LCH, 16 * vt, kk, lane), acc);
            S[m] = acc;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sSt[(16 * vt + r16) * LDK + 16 * ct + 4 * g4 + i] = from_f32<T>(acc[i]);
        }
        __syncthreads();
    }

    // ---- final state ---------------------------------------------------------
    if (p.sfin && n >= p.final_seq_lo) {
        const int64_t sbase = ((int64_t)(n - p.final_seq_lo) * H + h) * DK * (int64_t)p.dvt;
#pragma unroll
        for (int m = 0; m < C::SPW; ++m) {
            const int si = wave + C::NW * m, ct = si / NVT, vt = si % NVT;
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
    p.dvt = a.aug ? a.dk + a.dv : a.dv;
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

// LDS bytes of a configuration, to keep only the slice widths that fit.
template <class E, int DK, int VS, int CH>
constexpr size_t pf_lds_bytes() {
    using T = typename E::T;
    constexpr size_t pe = 16 / sizeof(T), ldk = DK + pe, lch = CH + pe, nt = CH / 16;
    constexpr size_t ng = 256 / (DK / 2);
    constexpr size_t n0 = (size_t)CH * (CH + 4) * 4, n1 = (size_t)VS * lch * sizeof(T);
    return (3 * CH * ldk + DK * lch + VS * ldk + 2 * CH * lch + VS * lch) * sizeof(T) +
           (n0 > n1 ? n0 : n1) + (ng * DK + 2 * nt * DK + nt * nt * DK + DK + CH) * 4 + 16;
}

template <class E, int DK, int CH, bool AUG>
static hipError_t launch_vs(const PrefillArgs& a, int vs) {
    if constexpr (pf_lds_bytes<E, DK, 64, CH>() <= 160 * 1024) {
        if (vs != 32) return launch_cfg<PfCfg<E, DK, 64, CH, AUG>>(a);
    }
    return launch_cfg<PfCfg<E, DK, 32, CH, AUG>>(a);
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
        // enough workgroups to cover the CUs, preferring wide slices
        const long chains = (long)a.num_seqs * a.H;
        vs = (chains * (a.dv / 64) >= 256 || a.dv == 32) ? 64 : 32;
    }
    if (a.dtype == 0) {
        if (a.dk == 128) {
            if (a.chunk == 64)
                return a.aug ? launch_vs<BF16, 128, 64, true>(a, vs) : launch_vs<BF16, 128, 64, false>(a, vs);
            return a.aug ? launch_vs<BF16, 128, 16, true>(a, vs) : launch_vs<BF16, 128, 16, false>(a, vs);
        }
        if (a.chunk == 64)
            return a.aug ? launch_vs<BF16, 64, 64, true>(a, vs) : launch_vs<BF16, 64, 64, false>(a, vs);
        return a.aug ? launch_vs<BF16, 64, 16, true>(a, vs) : launch_vs<BF16, 64, 16, false>(a, vs);
    }
    if (a.dk == 128)
        return a.aug ? launch_vs<F32, 128, 16, true>(a, vs) : launch_vs<F32, 128, 16, false>(a, vs);
    if (a.chunk == 64)
        return a.aug ? launch_vs<F32, 64, 64, true>(a, vs) : launch_vs<F32, 64, 64, false>(a, vs);
    return a.aug ? launch_vs<F32, 64, 16, true>(a, vs) : launch_vs<F32, 64, 16, false>(a, vs);
}

}  // namespace kda
