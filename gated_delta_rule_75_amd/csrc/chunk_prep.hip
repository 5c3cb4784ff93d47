// Chunk preparation: every product of a chunk that does not involve the state
// entering it, for all (chunk, head) pairs at once (the two-pass form and the
// workspace layout are described in twopass.h).
//
// One workgroup (8 waves; 4 for dk = 64 with 16-token chunks) per (chunk, head):
//  1. decay: a wave owns 64 channels of a slice of consecutive tokens, so each
//     load instruction reads whole 128-byte rows (a layout with fewer channels
//     per wave touched four times the cache lines per byte); a thread holds
//     TPT consecutive tokens x 4 consecutive channels of g, k and q (beta and
//     g are loaded first, so that the sums below wait for them alone).  The
//     in-chunk running sum G of g is a per-thread sum, a shuffle scan over
//     the wave's token groups, and a sum of the earlier slices' totals
//     exchanged through LDS.
//  2. gated Gram products A (k.k, strictly lower) and P (q.k, lower) on MFMA.
//     The factor e^{G_t - G_j} is split at 16-token sub-tile references so no
//     operand exceeds e^{16 |g_min|}: page "Exercices", Niveau 2 Q8 sizes
//     g_min = -5 for exactly this (16 tokens give e^80, inside the bf16
//     range).  Row operand x_t e^{G_t - R_a(t)} <= 1, column operand
//     k_j e^{R_b(j) - G_j} <= e^80, and for an off-diagonal block (a, b) the
//     column factor e^{R_a - R_b} <= 1, applied while loading the fragment.
//  3. L = I + diag(beta) A is unit lower triangular; its inverse is blocked:
//     16 x 16 diagonal blocks by forward substitution, then off-diagonal
//     blocks level by level, X_ab = -X_aa sum_{b<=c<a} L_ac X_cb (fp32 MFMA).
//     Each block is also written, times beta_j, in the storage type into the
//     table of Tb = L^{-1} diag(beta) that phase 4 reads.
//  4. W = Tb (K e^G) on MFMA, a wave taking one channel tile; Tb itself leaves
//     as fragments for the scan kernel, which forms U = Tb V from v (v is not
//     read here at all).
// Qt, Kh and gam leave straight from the decay phase; the tiles of W and P
// leave as they are produced.
//
// Waves share data only through LDS, so the barriers between phases wait for
// LDS operations alone; the global stores of each phase (and loads still in
// flight) drain in the background instead of at every barrier.
//
// The FUSED variant takes raw inputs instead: q and k of any length, the
// decay pre-activation a (in the storage dtype) in place of g, and the beta
// pre-activation b in place of beta.  Phase 1 then forms g = g_min sigmoid(a)
// while loading, beta = sigmoid(b), and scales each token's q and k to unit
// length (unit keys: page "Exercices", Niveau 2 Q9; the low-rank W_alpha and
// W_beta that produce a and b: page "Retrouver les 2,8 T de paramètres",
// Bloc 4).  The squared norms are summed over the 16 lanes of a token group
// by DPP moves; each thread then adds the channel sets' partials of its own
// tokens from LDS that phase 2 later reuses.
#include "launch.h"
#include "twopass.h"

namespace kda {

struct PrepParams {
    int H, num_seqs, cps;   // cps: chunks per segment when cu_seqlens is NULL
    int gc0;                // global chunk of workspace block 0 (the first chunk of the slab)
    int rect_w, rect_c0, rect_s0;   // rectangular slab (rect_w > 0): chunks [c0, c0 + w) of segments s0..
    float scale;
    int64_t T_total, seg_len;
    const int32_t* cu_seqlens;
    const int32_t* chunk_off;  // [num_seqs + 1] chunk offsets of packed sequences, or NULL
    const void *q, *k;      // v is not read here: U = Tb V is formed by the scan kernel
    const void *g, *beta;   // fp32 g and beta, or (FUSED) the pre-activations a, b in the storage dtype
    TwoPassBufs ws;
};

template <typename E_, int DK_, int CH_, bool FUSED_, bool NOQP_ = false>
struct PrepCfg {
    static constexpr bool FUSED = FUSED_;
    // NOQP: only what the KCP pairs read (W, T, Kh^T, gam): q is not loaded
    // and neither Qt nor P is formed
    static constexpr bool NOQP = NOQP_;
    static_assert(!(FUSED && NOQP), "no fused pairs pass");
    using E = E_;
    using K = KBlk<E_>;
    using T = typename E::T;
    static constexpr int DK = DK_, DV = DK_, CH = CH_;
    static constexpr int NT = CH / 16, NCT = DK / 16, NPAIR = NT * (NT + 1) / 2;
    static constexpr int CP = (CH + K::KB - 1) / K::KB * K::KB;
    static constexpr int NKT = CP / K::KB;                  // k-blocks over tokens
    static constexpr int NPM = pm_frags(NT, NKT, K::KB);    // stored fragments of Pm
    static constexpr int NW = (DK == 64 && CH == 16) ? 4 : 8, NTHR = 64 * NW;
    // decay-phase mapping: wave w owns 64 channels (channel set w % NWC) of
    // TPW consecutive tokens (token slice w / NWC); lane = (token group tg,
    // channel group cg) holds TPT consecutive tokens x 4 channels, so one load
    // instruction reads TGW whole 64-channel rows
    static constexpr int CGW = 16, TGW = 64 / CGW;
    static constexpr int NWC = DK / 64, NTS = NW / NWC, TPW = CH / NTS, TPT = TPW / TGW;
    static constexpr int SPT = 16 / TPW;   // token slices per 16-token sub-tile
    static_assert(NWC * 64 == DK && NTS * NWC == NW && TPT >= 1 && TPT * TGW == TPW && TPW * SPT == 16,
                  "decay mapping");
    static constexpr int PADE = 16 / (int)sizeof(T);
    static constexpr int LK = DK + PADE;  // pitch of [token][channel] tables
    static constexpr int LC = CP + PADE;  // pitch of [row][token] tables
    static constexpr int BLK = 16 * 17;   // fp32 16x16 block, pitch 17
    static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
    static constexpr size_t SZ_TAB = (size_t)CH * LK * sizeof(T);
    static constexpr size_t SZ_X1 = 3 * SZ_TAB;                       // Kr, Qr, Kc
    static constexpr size_t SZ_KVT = al((size_t)DK * LC * sizeof(T));  // Kt^T
    static constexpr size_t SZ_LB = al((size_t)CH * LC * sizeof(T));
    static constexpr size_t SZ_X2 = 2 * SZ_KVT + SZ_LB;                // after the Gram: Kt^T, Tb, Kh^T
    static constexpr size_t O_KR = 0, O_QR = SZ_TAB, O_KC = 2 * SZ_TAB;
    static constexpr size_t O_KTT = 0, O_LB = SZ_KVT, O_KHT = SZ_KVT + SZ_LB;
    static constexpr size_t SZ_X = al(SZ_X1 > SZ_X2 ? SZ_X1 : SZ_X2);
    static constexpr size_t O_L = SZ_X;                         // blocks of beta A
    static constexpr size_t O_Z = O_L + (size_t)NPAIR * BLK * 4;  // blocks of L^{-1}
    static constexpr int ND = NT * (NT - 1) / 2;
    static constexpr size_t O_D = O_Z + (size_t)NPAIR * BLK * 4;   // e^{R_a - R_b}, a > b
    static constexpr size_t O_BETA = O_D + (size_t)(ND > 0 ? ND : 1) * DK * 4;
    static constexpr size_t O_TOT = O_BETA + (size_t)CH * 4;   // per-slice sums of g, [NTS][DK]
    static constexpr size_t BYTES = O_TOT + (size_t)NTS * DK * 4;
    static_assert(BYTES <= 160 * 1024, "LDS");
    // FUSED: partial squared norms of k and q per channel set, [2][NWC][CH]
    // fp32, on the L blocks
    static_assert(!FUSED || 2 * NWC * CH * 4 <= NPAIR * BLK * 4, "norm scratch");
    // waves per SIMD the LDS allows (2 workgroups of 8 waves per CU at 80 KB
    // or less): the register budget is held to match
    static constexpr int WPE = BYTES <= 80 * 1024 ? (2 * NTHR / 64 + 3) / 4 : 1;
};

__device__ __forceinline__ int pair_index(int a, int b) { return a * (a + 1) / 2 + b; }

// four consecutive elements <-> fp32
__device__ __forceinline__ f32x4_t ld4f(const __bf16* p) {
    const bf16x4_t v = *reinterpret_cast<const bf16x4_t*>(p);
    return f32x4_t{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4_t ld4f(const float* p) { return *reinterpret_cast<const f32x4_t*>(p); }
__device__ __forceinline__ void st4(__bf16* p, float a, float b, float c, float d) {
    *reinterpret_cast<bf16x4_t*>(p) = bf16x4_t{(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
}
__device__ __forceinline__ void st4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4_t*>(p) = f32x4_t{a, b, c, d};
}
__device__ __forceinline__ f32x4_t cvt4(bf16x4_t v) { return f32x4_t{(float)v[0], (float)v[1], (float)v[2], (float)v[3]}; }
__device__ __forceinline__ f32x4_t cvt4(f32x4_t v) { return v; }
// four elements kept in the storage type between phases (half the registers at bf16)
template <typename T> struct Vec4;
template <> struct Vec4<__bf16> { using type = bf16x4_t; };
template <> struct Vec4<float> { using type = f32x4_t; };
template <typename T>
__device__ __forceinline__ typename Vec4<T>::type pack4(float a, float b, float c, float d) {
    return typename Vec4<T>::type{from_f32<T>(a), from_f32<T>(b), from_f32<T>(c), from_f32<T>(d)};
}

template <class C>
__global__ __launch_bounds__(C::NTHR) __attribute__((amdgpu_waves_per_eu(C::WPE)))
void chunk_prep_kernel(PrepParams p) {
    using E = typename C::E;
    using K = typename C::K;
    using T = typename C::T;
    constexpr int DK = C::DK, DV = C::DV, CH = C::CH, NT = C::NT, NCT = C::NCT, CP = C::CP;
    constexpr int LK = C::LK, LC = C::LC, BLK = C::BLK, NTHR = C::NTHR, NW = C::NW;
    constexpr int CGW = C::CGW, TGW = C::TGW, TPT = C::TPT;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    T* sKr = reinterpret_cast<T*>(smem + C::O_KR);
    T* sQr = reinterpret_cast<T*>(smem + C::O_QR);
    T* sKc = reinterpret_cast<T*>(smem + C::O_KC);
    T* sKtT = reinterpret_cast<T*>(smem + C::O_KTT);
    T* sLB = reinterpret_cast<T*>(smem + C::O_LB);
    T* sKhT = reinterpret_cast<T*>(smem + C::O_KHT);
    float* sL = reinterpret_cast<float*>(smem + C::O_L);
    float* sZ = reinterpret_cast<float*>(smem + C::O_Z);
    float* sD = reinterpret_cast<float*>(smem + C::O_D);
    float* sBeta = reinterpret_cast<float*>(smem + C::O_BETA);

    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);  // wave-uniform
    const int H = p.H;
    constexpr int NTS = C::NTS, TPW = C::TPW, SPT = C::SPT;
    const int cset = wave % C::NWC, tsl = wave / C::NWC;   // wave-uniform
    const T* gq = static_cast<const T*>(p.q);
    const T* gk = static_cast<const T*>(p.k);
    using T4 = typename Vec4<T>::type;

    const int tid = threadIdx.x, lane = tid & 63;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int64_t wsb = blockIdx.x;  // (chunk, head) block of the workspace
    const int h = (int)(wsb % H);
    // global chunk index: the slab's chunks in order, or those of a rectangle
    // of segments x chunks, segment by segment
    const int rb = (int)(wsb / H);
    const int gc = p.rect_w > 0 ? (p.rect_s0 + rb / p.rect_w) * p.cps + p.rect_c0 + rb % p.rect_w : p.gc0 + rb;

    // ---- locate the chunk ----------------------------------------------------
    int64_t ts;
    int nvalid;
    if (p.chunk_off) {
        if (gc >= p.chunk_off[p.num_seqs]) return;
        int lo = 0, hi = p.num_seqs;  // chunk_off[lo] <= gc < chunk_off[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (p.chunk_off[mid] <= gc) lo = mid;
            else hi = mid;
        }
        ts = p.cu_seqlens[lo] + (int64_t)(gc - p.chunk_off[lo]) * CH;
        const int64_t rem = p.cu_seqlens[lo + 1] - ts;
        nvalid = (int)(rem < CH ? rem : CH);
    } else {
        const int sq = gc / p.cps;
        if (sq >= p.num_seqs) return;
        const int64_t s0 = (int64_t)sq * p.seg_len;
        const int64_t s1 = s0 + p.seg_len < p.T_total ? s0 + p.seg_len : p.T_total;
        ts = s0 + (int64_t)(gc % p.cps) * CH;
        if (ts >= s1) return;  // past the end of a short last segment
        nvalid = (int)(s1 - ts < CH ? s1 - ts : CH);
    }
    // never read past T_total, whatever the offsets say
    if (ts >= p.T_total) return;
    if (ts + nvalid > p.T_total) nvalid = (int)(p.T_total - ts);

    // phase-1 mapping (see below): this thread's channels and first token
    const int tg = lane / CGW, cg = lane % CGW;
    const int c0 = cset * 64 + 4 * cg;
    const int tl0 = tsl * TPW + tg * TPT;
    // the block's inputs as stored, converted where they are used: g (fp32)
    // or the pre-activation a, k, q, and one beta (or b) per thread below C
    using GRaw = typename std::conditional<C::FUSED, T4, f32x4_t>::type;
    GRaw rg[TPT];
    T4 rk[TPT], rq[TPT];
    // beta, then g: vector loads complete in issue order, so the running
    // sums below wait for these alone while k and q are still on their way
    using BRaw = typename std::conditional<C::FUSED, T, float>::type;
    BRaw braw = BRaw(0.f);
    if (tid < CH && tid < nvalid) {
        const int64_t at = (ts + tid) * H + h;
        braw = static_cast<const BRaw*>(p.beta)[at];
    }
    int64_t rows[TPT];
#pragma unroll
    for (int i = 0; i < TPT; ++i) rows[i] = (ts + (tl0 + i < nvalid ? tl0 + i : 0)) * H + h;
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
        if constexpr (C::FUSED) rg[i] = *reinterpret_cast<const T4*>(static_cast<const T*>(p.g) + rows[i] * DK + c0);
        else rg[i] = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(p.g) + rows[i] * DK + c0);
    }
#pragma unroll
    for (int i = 0; i < TPT; ++i) rk[i] = *reinterpret_cast<const T4*>(gk + rows[i] * DK + c0);
    if constexpr (!C::NOQP) {
#pragma unroll
        for (int i = 0; i < TPT; ++i) rq[i] = *reinterpret_cast<const T4*>(gq + rows[i] * DK + c0);
    } else {
#pragma unroll
        for (int i = 0; i < TPT; ++i) rq[i] = T4{};
    }
    if (tid < CH) {
        if constexpr (C::FUSED) sBeta[tid] = tid < nvalid ? sigmoid(to_f32(braw)) : 0.f;
        else sBeta[tid] = braw;
    }

    T* Wn = static_cast<T*>(p.ws.wn) + wsb * (CH * DK);
    T* Qt = static_cast<T*>(p.ws.qt) + wsb * (CH * DK);
    T* KhT = static_cast<T*>(p.ws.kht) + wsb * (DK * CP);
    T* Pm = static_cast<T*>(p.ws.pm) + wsb * (C::NPM * 64 * (K::KB / 4));
    T* Tb = static_cast<T*>(p.ws.tt) + wsb * (C::NPM * 64 * (K::KB / 4));
    float* gam = p.ws.gam + wsb * DK;

    // ---- 1. loads and decay ----------------------------------------------------
    // k and q stay in the storage type (rk, rq) until they are used
    f32x4_t G[TPT];
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
        // log-decay in base 2: every exponential below is one v_exp_f32
        if constexpr (C::FUSED) {
            const f32x4_t aa = cvt4(rg[i]);
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) G[i][ch] = decay_gate(aa[ch]) * kLog2e;
        } else {
            G[i] = rg[i] * kLog2e;
        }
    }
    if (nvalid < CH) {  // tokens past the end of a ragged chunk take no part
#pragma unroll
        for (int i = 0; i < TPT; ++i)
            if (tl0 + i >= nvalid) {
                G[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                rk[i] = T4{};
                rq[i] = T4{};
            }
    }
    // running sum over the thread's tokens, then over the wave's token groups,
    // then over the token slices before this wave's (slice sums through LDS)
#pragma unroll
    for (int i = 1; i < TPT; ++i) G[i] += G[i - 1];
    float* sTot = reinterpret_cast<float*>(smem + C::O_TOT);   // [NTS][DK]
    f32x4_t ex;   // sum over the wave's earlier token groups
    {
        f32x4_t inc = G[TPT - 1];
#pragma unroll
        for (int d = 1; d < TGW; d <<= 1) {
            f32x4_t y;
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) y[ch] = __shfl_up(inc[ch], d * CGW, 64);
            if (tg >= d) inc += y;
        }
        ex = inc - G[TPT - 1];
        if (tg == TGW - 1) *reinterpret_cast<f32x4_t*>(sTot + tsl * DK + c0) = inc;
    }
    float* sNorm = sL;  // FUSED: [2][NWC][CH] partial squared norms (k, then q)
    if constexpr (C::FUSED) {
        // this thread's 4 channels, then the CGW lanes of a token group, then
        // one partial per (channel set, token) in LDS; placed after the slice
        // sums, which wait for g alone, so that their shuffles are not queued
        // behind the loads of k and q
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            float sk = 0.f, sq = 0.f;
            const f32x4_t kk = cvt4(rk[i]), qq = cvt4(rq[i]);
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) {
                sk += kk[ch] * kk[ch];
                sq += qq[ch] * qq[ch];
            }
            static_assert(CGW == 16, "a token group is one 16-lane row");
            sk = row16_sum(sk);
            sq = row16_sum(sq);
            if (cg == 0) {
                sNorm[cset * CH + tl0 + i] = sk;
                sNorm[(C::NWC + cset) * CH + tl0 + i] = sq;
            }
        }
    }

    barrier_keep_loads();
    // FUSED: each thread sums the channel-set partials of its own tokens (the
    // barrier above has made them visible), with no further exchange; read
    // before the slice sums so that the two LDS round trips overlap
    float ik[TPT], iq[TPT];
    if constexpr (C::FUSED) {
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int w = 0; w < C::NWC; ++w) {
                sk += sNorm[w * CH + tl0 + i];
                sq += sNorm[(C::NWC + w) * CH + tl0 + i];
            }
            ik[i] = rsqrtf(sk + kNormEps);
            iq[i] = rsqrtf(sq + kNormEps);
        }
    }
    // sub-tile references R_b = G at token 16 b - 1 (R_0 = 0), the sum over
    // the slices before this one, and G_C
    f32x4_t Rb[NT], Ro, RoL, GC;
    {
        f32x4_t run = {0.f, 0.f, 0.f, 0.f}, pre = run;
#pragma unroll
        for (int sl = 0; sl < NTS; ++sl) {
            if (sl % SPT == 0) Rb[sl / SPT] = run;
            if (sl == tsl) pre = run;
            run += *reinterpret_cast<const f32x4_t*>(sTot + sl * DK + c0);
        }
        GC = run;
        Ro = Rb[0];
#pragma unroll
        for (int a = 1; a < NT; ++a)
            if (tsl / SPT == a) Ro = Rb[a];
        RoL = Ro - pre - ex;   // the reference relative to the thread's own running sums
    }
    if (tsl == 0 && tg == 0) {
#pragma unroll
        for (int a = 1; a < NT; ++a)
#pragma unroll
            for (int b = 0; b < a; ++b) {
                float* d = sD + (a * (a - 1) / 2 + b) * DK + c0;
#pragma unroll
                for (int ch = 0; ch < 4; ++ch) d[ch] = exp2_fast(Rb[a][ch] - Rb[b][ch]);
            }
        st4(gam + c0, exp2_fast(GC[0]), exp2_fast(GC[1]), exp2_fast(GC[2]), exp2_fast(GC[3]));
    }
    // two exponentials per element, e^{G - R} <= 1 and e^{R - G} <= e^80 (R the
    // sub-tile reference); e^G and e^{G_C - G} follow by per-channel factors
    // e^R <= 1 and e^{G_C - R} <= 1
    const float scale = p.scale;
    f32x4_t eR, eCR, sR;
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
        eR[ch] = exp2_fast(Ro[ch]);
        eCR[ch] = exp2_fast(GC[ch] - Ro[ch]);
        sR[ch] = scale * eR[ch];
    }
    T4 kh[TPT];  // K e^{G_C - G}, the rows of Kh^T, in the storage type until phase 3
    T4 kw[TPT];  // K e^G, the W operand, in the storage type until phase 3
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
        const int t = tl0 + i;
        f32x4_t kx = cvt4(rk[i]), qx = cvt4(rq[i]);
        if constexpr (C::FUSED) {
            kx *= ik[i];
            qx *= iq[i];
        }
        f32x4_t kr, qr, kc, qt, kg, kx2;
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
            const float d = G[i][ch] - RoL[ch];
            const float er = exp2_fast(d);    // e^{G - R}
            const float ec = exp2_fast(-d);   // e^{R - G}
            kr[ch] = kx[ch] * er;
            qr[ch] = qx[ch] * er;
            kc[ch] = kx[ch] * ec;
            qt[ch] = qr[ch] * sR[ch];         // scale q e^G
            kx2[ch] = kc[ch] * eCR[ch];       // k e^{G_C - G}
            kg[ch] = kr[ch] * eR[ch];         // k e^G
        }
        kw[i] = pack4<T>(kg[0], kg[1], kg[2], kg[3]);
        kh[i] = pack4<T>(kx2[0], kx2[1], kx2[2], kx2[3]);
        st4(sKr + t * LK + c0, kr[0], kr[1], kr[2], kr[3]);
        st4(sKc + t * LK + c0, kc[0], kc[1], kc[2], kc[3]);
        if constexpr (!C::NOQP) {
            st4(sQr + t * LK + c0, qr[0], qr[1], qr[2], qr[3]);
            st4(Qt + frag_elem<K>((c0 / K::KB) * NT + t / 16, t, c0), qt[0], qt[1], qt[2], qt[3]);
        }
    }
    barrier_keep_loads();

    // ---- 2. gated Gram products -------------------------------------------------
    for (int task = wave; task < C::NPAIR; task += NW) {
        int a = 0;
        while ((a + 1) * (a + 2) / 2 <= task) ++a;
        const int b = task - a * (a + 1) / 2;
        const float* dsc = sD + (a > b ? (a * (a - 1) / 2 + b) : 0) * DK;
        f32x4_t accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
        // all fragments of the task first, then the products
        constexpr int NKS = DK / E::KSTEP;
        constexpr int UNR = NKS < 4 ? NKS : 4;
        for (int k0 = 0; k0 < NKS; k0 += UNR) {
            typename E::Frag fc[UNR], fr[UNR], fq[UNR];
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int kk = (k0 + u) * E::KSTEP;
                fc[u] = a > b ? lds_frag_scaled<E>(sKc, LK, 16 * b, kk, lane, dsc)
                              : lds_frag<E>(sKc, LK, 16 * b, kk, lane);
                fr[u] = lds_frag<E>(sKr, LK, 16 * a, kk, lane);
                if constexpr (!C::NOQP) fq[u] = lds_frag<E>(sQr, LK, 16 * a, kk, lane);
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                accA = E::mma(fr[u], fc[u], accA);  // A[t][j]
                if constexpr (!C::NOQP) accP = E::mma(fc[u], fq[u], accP);  // P^T[j][t]
            }
        }
        // beta_t A[t][j] (strictly lower): lane holds rows 16a+4g4+i, column 16b+l16
        float* Lb = sL + pair_index(a, b) * BLK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g4 + i;
            Lb[r * 17 + l16] = (a > b || l16 < r) ? sBeta[16 * a + r] * accA[i] : 0.f;
        }
        if constexpr (!C::NOQP) {
            // scale P[t][j] (j <= t): lane holds token 16a+l16, columns 16b+4g4+i
            float pv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) pv[i] = (a > b || 4 * g4 + i <= l16) ? scale * accP[i] : 0.f;
            const int j0 = 16 * b + 4 * g4;
            st4(Pm + frag_elem<K>(pm_frag_index(a, j0 / K::KB, C::NKT, K::KB), l16, j0), pv[0], pv[1], pv[2], pv[3]);
            // a two-tile k-block holds tile a + 1 beside an even diagonal tile a
            // (past C when a + 1 = NT): zeros there
            if (K::TPB == 2 && a == b && a % 2 == 0) {
                const int jz = j0 + 16;
                st4(Pm + frag_elem<K>(pm_frag_index(a, jz / K::KB, C::NKT, K::KB), l16, jz), 0.f, 0.f, 0.f, 0.f);
            }
        }
    }
    barrier_keep_loads();

    // ---- 3. operand of W and the Kh^T table; inverse of L --------------------
    // In the [channel][token] tables the 16-byte unit x of row c sits at unit
    // x ^ ((c >> 3) & SWM): the rows four channels apart that one write
    // instruction covers then fall on different banks (bank conflicts of these
    // writes were most of pass 1's), while a fragment read still takes whole
    // units of eight consecutive rows
    constexpr int TU = 16 / (int)sizeof(T);   // tokens per 16-byte unit
    constexpr int NU = CP / TU;
    static_assert((NU & (NU - 1)) == 0, "units per row");
    constexpr int SWM = (NU < 8 ? NU : 8) - 1;
    auto tcol = [](int c, int t) { return ((t / TU) ^ ((c >> 3) & SWM)) * TU + t % TU; };
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
        const int c = c0 + ch;
        T* kt = sKtT + c * LC;
        T* kb = sKhT + c * LC;
        if constexpr (TPT % 4 == 0) {
#pragma unroll
            for (int i = 0; i < TPT; i += 4) {
                const int x = tcol(c, tl0 + i);   // four tokens inside one unit
                *reinterpret_cast<T4*>(kt + x) = T4{kw[i][ch], kw[i + 1][ch], kw[i + 2][ch], kw[i + 3][ch]};
                *reinterpret_cast<T4*>(kb + x) = T4{kh[i][ch], kh[i + 1][ch], kh[i + 2][ch], kh[i + 3][ch]};
            }
        } else {
#pragma unroll
            for (int i = 0; i < TPT; ++i) {
                kt[tcol(c, tl0 + i)] = kw[i][ch];
                kb[tcol(c, tl0 + i)] = kh[i][ch];
            }
        }
    }
    if constexpr (CP > CH) {
        for (int idx = tid; idx < DK * (CP - CH); idx += NTHR) {
            const int c = idx / (CP - CH), t = CH + idx % (CP - CH);
            sKtT[c * LC + tcol(c, t)] = from_f32<T>(0.f);
            sKhT[c * LC + tcol(c, t)] = from_f32<T>(0.f);
        }
    }
    if (wave < NT) {  // diagonal block `wave`, one column per lane (lanes >= 16 repeat)
        const float* Lb = sL + pair_index(wave, wave) * BLK;
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float s = (t == l16) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < t; ++m) s -= Lb[t * 17 + m] * x[m];
            x[t] = s;
        }
        // the block of L^{-1} and of L^{-1} diag(beta), the operand of phase 4;
        // with two-tile k-blocks phase 4 also reads tile (a, a + 1) for even a:
        // zeros there
        const int a = wave;
        if (lane < 16) {
            float* Zb = sZ + pair_index(a, a) * BLK;
            const float bj = sBeta[16 * a + l16];
            T* lb = sLB + (16 * a) * LC + 16 * a + l16;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                Zb[t * 17 + l16] = x[t];
                lb[t * LC] = from_f32<T>(x[t] * bj);
            }
        } else if (K::TPB == 2 && a % 2 == 0) {
            T* lb = sLB + (16 * a) * LC + 16 * (a + 1) + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) lb[(4 * (g4 - 1) + i) * LC] = from_f32<T>(0.f);
            if (g4 == 3) {
#pragma unroll
                for (int i = 12; i < 16; ++i) lb[i * LC] = from_f32<T>(0.f);
            }
        }
    }
    barrier_keep_loads();
    // off-diagonal blocks, level l = a - b: wave b forms M = sum_{b<=c<a} L_ac X_cb
    // and X_ab = -X_aa M with fp32 MFMAs (16x16x4, four per 16-wide reduction);
    // M stays in the accumulator and feeds the second product directly, MFMA i
    // taking row 4 g + i of it (the reduction order of the accumulator layout)
    for (int l = 1; l < NT; ++l) {
        const int b = wave, a = b + l;
        if (b < NT - l) {
            f32x4_t m = {0.f, 0.f, 0.f, 0.f};
            for (int c = b; c < a; ++c) {
                const float* La = sL + pair_index(a, c) * BLK;
                const float* Zc = sZ + pair_index(c, b) * BLK;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    m = __builtin_amdgcn_mfma_f32_16x16x4f32(La[l16 * 17 + 4 * ks + g4], Zc[(4 * ks + g4) * 17 + l16],
                                                             m, 0, 0, 0);
            }
            const float* Za = sZ + pair_index(a, a) * BLK;
            f32x4_t x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                x = __builtin_amdgcn_mfma_f32_16x16x4f32(Za[l16 * 17 + 4 * g4 + i], m[i], x, 0, 0, 0);
            float* Zab = sZ + pair_index(a, b) * BLK;
            const float bj = sBeta[16 * b + l16];
            T* lb = sLB + (16 * a + 4 * g4) * LC + 16 * b + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Zab[(4 * g4 + i) * 17 + l16] = -x[i];
                lb[i * LC] = from_f32<T>(-x[i] * bj);
            }
        }
        barrier_keep_loads();
    }

    // ---- 4. Tb = L^{-1} diag(beta) out as fragments; W^T = (K e^G)^T Tb^T ------
    // Tb's fragments on or below the diagonal (those of Pm), natural k order:
    // lane (row r, group g) holds Tb[16 ta + r][u KB + g KB/4 ..], one 16-byte
    // read of the table and one 16-byte store each
    {
        int f = 0;
#pragma unroll
        for (int ta = 0; ta < NT; ++ta)
#pragma unroll
            for (int u = 0; u < C::NKT; ++u)
                if (u * K::KB <= 16 * ta + 15) {
                    if (f % NW == wave) {
                        const uint4 x = *reinterpret_cast<const uint4*>(sLB + (16 * ta + l16) * LC + u * K::KB +
                                                                        g4 * (K::KB / 4));
                        *reinterpret_cast<uint4*>(Tb + (f * 64 + lane) * (K::KB / 4)) = x;
                    }
                    ++f;
                }
    }
    // Kh^T fragments (channel tile ct, k-block u over tokens): lane (row r,
    // group g) holds element e at token u KB + k, pos(k) = g KB/4 + e; runs of
    // four consecutive tokens are consecutive elements, so the lane reads its
    // runs from the table and stores its 16 bytes at once
    {
        constexpr int KPL = K::KB / 4;
        for (int f = wave; f < NCT * C::NKT; f += NW) {
            const int ct = f / C::NKT, u = f % C::NKT;
            const int rc = 16 * ct + l16;
            const T* row = sKhT + rc * LC;
            typename K::Frag x;
#pragma unroll
            for (int r = 0; r < KPL / 4; ++r) {
                // the run holding element 4 r of this lane: token k with pos(k) = g4 KPL + 4 r
                int k = 0;
#pragma unroll
                for (int kk = 0; kk < K::KB; kk += 4)
                    if (K::pos(kk) == g4 * KPL + 4 * r) k = kk;
                const T4 v = *reinterpret_cast<const T4*>(row + tcol(rc, u * K::KB + k));
#pragma unroll
                for (int e = 0; e < 4; ++e) K::set(x, 4 * r + e, v[e]);
            }
            *reinterpret_cast<typename K::Frag*>(KhT + (f * 64 + lane) * KPL) = x;
        }
    }
    // A wave owns channel tile ct of W: its operand along the tokens is loaded
    // once, and each fragment of Tb is the B operand of W^T.
    {
        constexpr int NKK = (16 * NT + E::KSTEP - 1) / E::KSTEP;  // k-steps of the last token tile
        for (int ct = wave; ct < NCT; ct += NW) {
            typename E::Frag fk[NKK];
#pragma unroll
            for (int s = 0; s < NKK; ++s) {
                // lds_frag's element order on the swizzled table: E::KPL consecutive
                // tokens from a 16-byte boundary lie inside one unit
                const int rc = 16 * ct + l16, t = s * E::KSTEP + E::KPL * g4;
                fk[s] = *reinterpret_cast<const typename E::Frag*>(sKtT + rc * LC + tcol(rc, t));
            }
#pragma unroll
            for (int ta = 0; ta < NT; ++ta) {
                f32x4_t aw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s * E::KSTEP < 16 * (ta + 1); ++s)
                    aw = E::mma(fk[s], lds_frag<E>(sLB, LC, 16 * ta, s * E::KSTEP, lane), aw);
                // lane holds W[16ta+l16][16ct+4g4+i]; stored negated
                const int c = 16 * ct + 4 * g4;
                st4(Wn + frag_elem<K>((c / K::KB) * NT + ta, l16, c), -aw[0], -aw[1], -aw[2], -aw[3]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
template <class C>
static hipError_t launch_prep_cfg(const TwoPassArgs& a, const int32_t* chunk_off, int64_t nblocks) {
    if (nblocks <= 0) return hipSuccess;
    PrepParams p;
    p.H = a.H;
    p.num_seqs = a.num_seqs;
    p.cps = (int)((a.seg_len + a.chunk - 1) / a.chunk);
    p.gc0 = (int)a.slab_lo;
    p.rect_w = a.rect_w;
    p.rect_c0 = a.rect_c0;
    p.rect_s0 = a.rect_s0;
    p.scale = a.scale;
    p.T_total = a.T_total;
    p.seg_len = a.seg_len;
    p.cu_seqlens = a.cu_seqlens;
    p.chunk_off = chunk_off;
    p.q = a.q;
    p.k = a.k;
    p.g = a.g;
    p.beta = a.beta;
    p.ws = a.bufs;
    auto kern = chunk_prep_kernel<C>;
    if (C::BYTES > 64 * 1024) {
        const hipError_t e = ensure_lds_limit((const void*)kern, (int)C::BYTES);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)nblocks), dim3(C::NTHR), C::BYTES, (hipStream_t)a.stream, p);
    return hipGetLastError();
}

template <class E, int DK, bool FUSED, bool NOQP>
static hipError_t launch_prep_chunk(const TwoPassArgs& a, const int32_t* co, int64_t nb) {
    if (a.chunk == 64) return launch_prep_cfg<PrepCfg<E, DK, 64, FUSED, NOQP>>(a, co, nb);
    if (a.chunk == 32) return launch_prep_cfg<PrepCfg<E, DK, 32, FUSED, NOQP>>(a, co, nb);
    return launch_prep_cfg<PrepCfg<E, DK, 16, FUSED, NOQP>>(a, co, nb);
}

template <class E, int DK>
static hipError_t launch_prep_dk(const TwoPassArgs& a, const int32_t* co, int64_t nb) {
    if (a.fused) return launch_prep_chunk<E, DK, true, false>(a, co, nb);
    if (a.pairs_only) return launch_prep_chunk<E, DK, false, true>(a, co, nb);
    return launch_prep_chunk<E, DK, false, false>(a, co, nb);
}

hipError_t launch_chunk_prep(const TwoPassArgs& a, const int32_t* chunk_off, int64_t nchunks) {
    // the slab's chunks [slab_lo, slab_lo + nchunks) into workspace blocks 0 ..
    const int64_t nb = nchunks * a.H;
    if (a.dtype == 0)
        return a.dk == 128 ? launch_prep_dk<BF16, 128>(a, chunk_off, nb) : launch_prep_dk<BF16, 64>(a, chunk_off, nb);
    return a.dk == 128 ? launch_prep_dk<F32, 128>(a, chunk_off, nb) : launch_prep_dk<F32, 64>(a, chunk_off, nb);
}

}  // namespace kda
