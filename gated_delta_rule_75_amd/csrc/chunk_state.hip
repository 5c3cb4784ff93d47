// State scan: carries the state of every (sequence, head) through its chunks
// with the per-chunk products the preparation kernel stored (twopass.h):
//     Delta = U + Wn S,   O = Qt S + Pm Delta,   S <- gam * S + Kh^T Delta,
//     y = O * sigmoid(z).
//
// State columns evolve independently.  A workgroup of NW waves owns
// 16 NVT NW consecutive columns of one (sequence, head); each wave owns
// 16 NVT of them and keeps its part of S and Delta in MFMA accumulator tiles,
// fed back as operands straight from the lanes that hold them (the k-block
// order of twopass.h).  The chunk operands every wave needs (Wn, Qt, Kh^T,
// Pm, gam) are copied once per workgroup into LDS by direct global-to-LDS
// loads, double-buffered so chunk c+1 streams in while chunk c is computed.
// In LDS each operand fragment (16 rows x one k-block) is stored in lane
// order, 16 bytes per lane, so that every wave reads a fragment with one
// conflict-free 16-byte access per lane.  Without loader waves (below), U^T
// and z, private to a wave, go straight to registers one chunk ahead.
// Products (lane layout: rows 4*(l/16)+i, column l%16 of a 16x16 tile):
//     Delta [t][v]  += Wn[t][c] . S[c][v]            A = Wn rows,   B = S
//     O^T  [v][t]   += S^T[v][c] . Qt^T[c][t]        A = S,         B = Qt rows
//                    + Delta^T[v][j] . Pm^T[j][t]    A = Delta,     B = Pm rows
//     S    [c][v]   += Kh^T[c][t] . Delta[t][v]      A = Kh^T rows, B = Delta
// so a lane of O^T holds four consecutive value columns of one token, and
// the gate input z and the output y move in 8-byte (bf16) runs.
//
// The workgroups of one chain take ids with equal residue mod 8, which places
// them on one XCD, so they share the chunk operands through its L2.
//
// Loader waves.  When two buffers of the chunk operands plus the workgroup's
// U^T tiles fit in LDS (one value tile per wave), four extra waves do all the
// staging: they issue the global-to-LDS copies of chunk c+1 while chunk c is
// computed and meet the compute waves at its barriers (two per chunk: one
// once U^T and Wn, the operands of Delta, are in; one before the state
// update, once the rest is).  A wave that issues a 1 KiB copy stalls until
// the memory pipeline takes it, so the compute waves, which now issue only
// their z loads and y stores, no longer lose those cycles.  Those move as whole
// 128-byte rows: right after the first barrier of chunk c each compute wave
// loads its share of chunk c+1's z rows into registers, and writes them into
// a z tile in LDS at the top of chunk c+1; outputs go into a y tile and leave
// as whole rows after the next chunk's first barrier.  (Per-lane accesses in
// the accumulator layout touched 16 lines for 32 bytes each.)  With one value
// tile per wave, each phase also reads all of its fragments from LDS before
// its first product.
#include <type_traits>

#include "launch.h"
#include "twopass.h"

namespace kda {

struct StateParams {
    int H, num_seqs, nchains, nvg, dvt, final_seq_lo, cps;
    int chunk_cap;  // chunks the workspace holds
    int64_t T_total, seg_len;
    const int32_t* cu_seqlens;
    const int32_t* chunk_off;
    const int32_t* order;
    const void* z;
    void* y;
    const float* s0;
    float* sfin;
    TwoPassBufs ws;
    float* ckpt;
    const int32_t* ckpt_off;
    int ckpt_every;
    int64_t ckpt_cap;
};

template <typename E_, int DK_, int DV_, int CH_, int NVT_, int MODE_>
struct StCfg {
    using E = E_;
    using K = KBlk<E_>;
    using T = typename K::T;
    static constexpr int DK = DK_, DV = DV_, CH = CH_, NVT = NVT_, MODE = MODE_;
    static constexpr bool AUG = MODE_ == kModePairs;
    static constexpr int NW = 4;
    static constexpr int CW = 16 * NVT * NW;            // state columns per workgroup
    static constexpr int NTT = CH / 16, NCT = DK / 16;
    static constexpr int KB = K::KB, TPB = K::TPB;
    static constexpr int NKC = DK / KB;                 // k-blocks over channels
    static constexpr int CP = (CH + KB - 1) / KB * KB;
    static constexpr int NKT = CP / KB;                 // k-blocks over tokens
    static_assert(NKC * TPB == NCT, "channel k-blocks");
    static constexpr int NPM = pm_frags(NTT, NKT, KB);  // stored fragments of Pm
    // fragment index ranges in an LDS buffer (1 KiB each)
    static constexpr int F_W = 0, N_W = NKC * NTT;
    static constexpr int F_Q = F_W + N_W, N_Q = AUG ? 0 : NKC * NTT;
    static constexpr int F_K = F_Q + N_Q, N_K = NCT * NKT;
    static constexpr int F_P = F_K + N_K, N_P = AUG ? 0 : NPM;
    static constexpr int F_G = F_P + N_P;               // gam: dk fp32, repeated to fill 1 KiB
    static constexpr int NF = F_G + 1;
    static constexpr int FPW = (NF + NW - 1) / NW;      // fragment loads per wave
    // U^T of the workgroup's columns: NW NVT value tiles x NTT token tiles in
    // accumulator layout (64 lanes x 4 elements each), after the fragments
    static constexpr int UTT = 64 * 4 * (int)sizeof(T);  // bytes of one U^T tile
    static constexpr int UTB = NW * NVT * NTT * UTT;
    static_assert(UTB % 1024 == 0, "U^T in whole 1 KiB copies");
    // z and y tiles of the workgroup's columns, [CH][CW] row-major in LDS with
    // the 16-byte units of row t stored at unit x ^ (t % ZXR), which spreads
    // the 16 rows a wave's fragment access touches over the banks
    static constexpr int ZRB = CW * (int)sizeof(T);        // bytes of one token row
    static constexpr int ZXR = ZRB / 16;                   // 16-byte units per row
    static constexpr int ZT = AUG ? 0 : CH * ZRB;          // bytes of a z or y tile
    // loader waves (with two value tiles per wave the compute waves' registers
    // are at the 256 limit already; they keep staging their own operands);
    // the z and y rows go in whole 1 KiB copies per compute wave
    static constexpr bool LW = NVT == 1 && ZT % (1024 * NW) == 0 && 2 * (NF * 1024 + UTB) + 4 * ZT <= 160 * 1024;
    static constexpr int BUF = NF * 1024 + (LW ? UTB : 0);
    static constexpr int NBUF = LW || 2 * BUF <= 150 * 1024 ? 2 : 1;
    static constexpr int O_Z = NBUF * BUF;                 // with LW: two z tiles, then two y tiles
    static constexpr int O_Y = O_Z + 2 * ZT;
    static constexpr int BYTES = NBUF * BUF + (LW ? 4 * ZT : 0);
    // loader waves: four (a wave issues a 1 KiB copy about every 170 cycles
    // on its own; with the copies dealt round-robin, two, three and four
    // loaders reach 324, 317 and 314 us on the 96-head layer)
    static constexpr int NLW = LW ? 4 : 0;
    static constexpr int NCOPY = NF + UTB / 1024;            // 1 KiB copies per chunk
    static constexpr int NTHR = 64 * (NW + NLW);
};

template <typename T> struct VecT4;
template <> struct VecT4<__bf16> { using type = bf16x4_t; };
template <> struct VecT4<float> { using type = f32x4_t; };
__device__ __forceinline__ f32x4_t to_f32x4(bf16x4_t v) {
    return f32x4_t{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4_t to_f32x4(f32x4_t v) { return v; }
template <typename T> __device__ __forceinline__ typename VecT4<T>::type from_f32x4(f32x4_t x);
template <> __device__ __forceinline__ bf16x4_t from_f32x4<__bf16>(f32x4_t x) {
    return bf16x4_t{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
}
template <> __device__ __forceinline__ f32x4_t from_f32x4<float>(f32x4_t x) { return x; }

template <class C>
__global__ __launch_bounds__(C::NTHR) void chunk_state_kernel(StateParams p) {
    using K = typename C::K;
    using T = typename C::T;
    using Frag = typename K::Frag;
    using T4 = typename VecT4<T>::type;
    constexpr int DK = C::DK, DV = C::DV, CH = C::CH, NVT = C::NVT, NTT = C::NTT, NCT = C::NCT;
    constexpr int KB = C::KB, TPB = C::TPB, NKC = C::NKC, NKT = C::NKT, CP = C::CP, NW = C::NW;
    constexpr int KPL = KB / 4;  // k values per lane
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int g4 = lane >> 4, l16 = lane & 15;

    const int blk = blockIdx.x, r = blk >> 3;
    const int slot = (r / p.nvg) * 8 + (blk & 7), vg = r % p.nvg;
    if (slot >= p.nchains) return;
    const int H = p.H, h = slot % H;
    const int n = p.order ? p.order[slot / H] : slot / H;
    int64_t t0, len;
    int cbase;
    if (p.cu_seqlens) {
        t0 = p.cu_seqlens[n];
        len = p.cu_seqlens[n + 1] - t0;
        cbase = p.chunk_off[n];
    } else {
        t0 = (int64_t)n * p.seg_len;
        const int64_t t1 = t0 + p.seg_len < p.T_total ? t0 + p.seg_len : p.T_total;
        len = t1 - t0;
        cbase = n * p.cps;
    }
    // stay inside T_total and the workspace whatever the offsets say
    if (t0 >= p.T_total) len = 0;
    else if (t0 + len > p.T_total) len = p.T_total - t0;
    int nch = len > 0 ? (int)((len + CH - 1) / CH) : 0;
    if (cbase + nch > p.chunk_cap) nch = cbase < p.chunk_cap ? p.chunk_cap - cbase : 0;
    const int dvt = p.dvt;
    // first value tile (16 columns of v / U) of the workgroup; negative for
    // the transition columns of mode 2, whose waves take no values
    const int vt_wg = (vg * C::CW - (C::AUG ? DK : 0)) / 16;

    if constexpr (C::LW) {
        if (wave >= NW) {
            // ---- loader waves: chunk c+1 into buffer (c+1) % 2 during chunk c ----
            constexpr int FB = 64 * KPL * (int)sizeof(T);   // bytes of one fragment (1 KiB)
            static_assert(FB == 1024, "fragment size");
            const char* wn = static_cast<const char*>(p.ws.wn) + 16 * lane;
            const char* qt = static_cast<const char*>(p.ws.qt) + 16 * lane;
            const char* kh = static_cast<const char*>(p.ws.kht) + 16 * lane;
            const char* pm = static_cast<const char*>(p.ws.pm) + 16 * lane;
            const char* gm = reinterpret_cast<const char*>(p.ws.gam) + 16 * (lane % (DK / 4));
            const char* ut = static_cast<const char*>(p.ws.ut) + 16 * lane;
            // copy k of a chunk: fragment k (k < NF) or U^T copy k - NF.  Two
            // groups, each with a barrier of its own: group 1 (U^T and Wn, the
            // operands of Delta) and group 2 (gam, Kh^T, Qt, Pm), whose last
            // copies land while Delta is formed.  The U^T copies, private to
            // the workgroup and so never in L2 already, go out first; the
            // copies of a group are dealt to the loaders in turn.
            const int li = wave - NW;
            constexpr int NU = C::NCOPY - C::NF;
            constexpr int NG1 = NU + C::N_W, NG2 = C::NCOPY - NG1;
            auto stage_group = [&](int c, int b, auto G) {
                const int64_t wsb = (int64_t)(cbase + c) * H + h;
                char* buf = smem + b * C::BUF;
                const char* aw = wn + wsb * (int64_t)(CH * DK * sizeof(T));
                const char* aq = qt + wsb * (int64_t)(CH * DK * sizeof(T));
                const char* ak = kh + wsb * (int64_t)(DK * CP * sizeof(T));
                const char* ap = pm + wsb * (int64_t)(C::NPM * FB);
                const char* ag = gm + wsb * (int64_t)(DK * sizeof(float));
                const char* au = ut + wsb * (int64_t)(DV * CH * sizeof(T));
                constexpr int TPC = 1024 / C::UTT;   // U^T tiles per copy
                constexpr int NJ = decltype(G)::value == 1 ? NG1 : NG2;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    if (j % C::NLW != li) continue;
                    int k;
                    if constexpr (decltype(G)::value == 1) k = j < NU ? C::NF + j : C::F_W + j - NU;
                    else k = j == 0 ? C::F_G : j <= C::N_K ? C::F_K + j - 1 : j <= C::N_K + C::N_Q ? C::F_Q + j - 1 - C::N_K
                                                                                            : C::F_P + j - 1 - C::N_K - C::N_Q;
                    const char* src;
                    if (k < C::F_Q) src = aw + (k - C::F_W) * FB;
                    else if (k < C::F_K) src = aq + (k - C::F_Q) * FB;
                    else if (k < C::F_P) src = ak + (k - C::F_K) * FB;
                    else if (k < C::F_G) src = ap + (k - C::F_P) * FB;
                    else if (k == C::F_G) src = ag;
                    else {
                        // U^T tiles [vt_wg, vt_wg + NW NVT) x all token tiles, contiguous;
                        // transition tiles (vt < 0) copy a valid tile nobody reads
                        const int lt = (k - C::NF) * TPC;   // first (wave tile, token tile)
                        int g = vt_wg + lt / NTT;
                        g = g < 0 ? 0 : g;
                        src = au + (int64_t)(g * NTT + lt % NTT) * C::UTT;
                    }
                    lds_dma16(src, buf + k * 1024);
                }
            };
            using G1 = std::integral_constant<int, 1>;
            using G2 = std::integral_constant<int, 2>;
            // copies of a group that every loader issues at least
            constexpr int M1 = NG1 / C::NLW, M2 = NG2 / C::NLW;
            static_assert(M1 <= 63 && M2 <= 63, "vmcnt range");
            if (nch > 0) {
                stage_group(0, 0, G1{});
                stage_group(0, 0, G2{});
            }
            for (int c = 0; c < nch; ++c) {
                wait_vmcnt<M2>();           // group 1 of chunk c has landed (group 2 may be in flight)
                barrier_keep_loads();       // ... and the compute waves are done with chunk c-1
                if (c + 1 < nch) {
                    stage_group(c + 1, (c + 1) % 2, G1{});
                    wait_vmcnt<M1>();       // group 2 of chunk c (group 1 of c+1 may be in flight)
                } else {
                    wait_vmcnt<0>();
                }
                barrier_keep_loads();       // group 2 of chunk c is in LDS
                if (c + 1 < nch) stage_group(c + 1, (c + 1) % 2, G2{});
            }
            if constexpr (!C::AUG) {
                if (nch > 0) barrier_keep_loads();   // matches the compute waves' last y hand-off
            }
            return;
        }
    }

    const int colw = vg * C::CW + wave * 16 * NVT;  // first state column of the wave
    const bool ident = C::AUG && colw < DK;         // transition columns: start I, values 0
    const int vcol0 = C::AUG ? colw - DK : colw;    // its first column of v / z / y

    // ---- state ---------------------------------------------------------------
    f32x4_t S[NCT][NVT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) {
            const int col = colw + 16 * vt + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) S[ct][vt][i] = (C::AUG && col == 16 * ct + 4 * g4 + i) ? 1.f : 0.f;
        }
    if (!C::AUG && p.s0) {
        const float* s0 = p.s0 + ((int64_t)n * H + h) * DK * (int64_t)dvt;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[ct][vt][i] = s0[(int64_t)(16 * ct + 4 * g4 + i) * dvt + colw + 16 * vt + l16];
    }

    const T* gz = static_cast<const T*>(p.z);
    T* gy = static_cast<T*>(p.y);

    // ---- operand staging -----------------------------------------------------
    // Fragment f of a chunk into LDS: lane i fetches the 16 bytes it (and the
    // same lane of every other wave) will read.  Wave w stages fragments
    // w, w + NW, ...; where a fragment sits in the workspace does not depend
    // on the chunk, so each is resolved once here to (array, block stride,
    // lane offset).
    const char* fbase[C::FPW];
    int64_t fstride[C::FPW];
    int foff[C::FPW];
#pragma unroll
    for (int j = 0; j < C::FPW; ++j) {
        int f = wave + NW * j;
        f = f < C::NF ? f : C::NF - 1;   // the last wave repeats its last fragment
        constexpr int FB = 64 * KPL * (int)sizeof(T);   // bytes of one fragment
        if (f < C::F_Q) {
            fbase[j] = static_cast<const char*>(p.ws.wn);
            fstride[j] = (int64_t)CH * DK * sizeof(T);
            foff[j] = (f - C::F_W) * FB;
        } else if (f < C::F_K) {
            fbase[j] = static_cast<const char*>(p.ws.qt);
            fstride[j] = (int64_t)CH * DK * sizeof(T);
            foff[j] = (f - C::F_Q) * FB;
        } else if (f < C::F_P) {
            fbase[j] = static_cast<const char*>(p.ws.kht);
            fstride[j] = (int64_t)DK * CP * sizeof(T);
            foff[j] = (f - C::F_K) * FB;
        } else if (f < C::F_G) {
            fbase[j] = static_cast<const char*>(p.ws.pm);
            fstride[j] = (int64_t)C::NPM * FB;
            foff[j] = (f - C::F_P) * FB;
        } else {
            fbase[j] = reinterpret_cast<const char*>(p.ws.gam);
            fstride[j] = (int64_t)DK * sizeof(float);
            foff[j] = -16 * lane + 16 * (lane % (DK / 4));   // dk floats, repeated
        }
        foff[j] += 16 * lane;
    }
    // fragments [J0, J1) of this wave's share of chunk c into LDS buffer b
    auto stage = [&](int c, int b, auto J0, auto J1) {
        const int64_t wsb = (int64_t)(cbase + c) * H + h;
        char* buf = smem + b * C::BUF;
#pragma unroll
        for (int j = decltype(J0)::value; j < decltype(J1)::value; ++j) {
            const int f = wave + NW * j < C::NF ? wave + NW * j : C::NF - 1;
            lds_dma16(fbase[j] + wsb * fstride[j] + foff[j], buf + f * 1024);
        }
    };
    using J_0 = std::integral_constant<int, 0>;
    using J_H = std::integral_constant<int, C::FPW / 2>;
    using J_E = std::integral_constant<int, C::FPW>;
    auto frag = [&](const char* buf, int f) -> Frag {
        return *reinterpret_cast<const Frag*>(buf + f * 1024 + 16 * lane);
    };
    // With loader waves, z and y move as whole rows: copy j (1 KiB) of a tile
    // belongs to compute wave j % NW; lane l of the copy holds token row t,
    // logical 16-byte unit x
    constexpr int ZJW = C::ZT / 1024 / NW;   // row copies per wave
    auto zpos = [&](int j, int& t, int& x) {
        const int pbyte = j * 1024 + 16 * lane;
        t = pbyte / C::ZRB;
        x = ((pbyte % C::ZRB) / 16) ^ (t % C::ZXR);
    };
    // byte offset, in a z or y tile, of this lane's 4 columns of token 16 ta + l16
    auto zy_off = [&](int ta, int vt) -> int {
        const int t = 16 * ta + l16;
        const int cb = (wave * 16 * NVT + 16 * vt + 4 * g4) * (int)sizeof(T);
        return t * C::ZRB + (((cb / 16) ^ (t % C::ZXR)) * 16) + cb % 16;
    };
    const int vcw = vcol0 - wave * 16 * NVT;   // first value column of the workgroup
    static_assert(!C::LW || ZJW <= 2, "z rows per wave");
    uint4 zrow0 = {0, 0, 0, 0}, zrow1 = {0, 0, 0, 0};   // rows in flight (copies wave, wave + NW)
    auto zrow_src = [&](int c, int jj) -> const uint4* {
        const int nv = len - (int64_t)c * CH < CH ? (int)(len - (int64_t)c * CH) : CH;
        int t, x;
        zpos(jj * NW + wave, t, x);
        t = t < nv ? t : nv - 1;
        return reinterpret_cast<const uint4*>(
            reinterpret_cast<const char*>(gz + ((t0 + (int64_t)c * CH + t) * H + h) * DV + vcw) + 16 * x);
    };
    auto load_zrows = [&](int c) {
        if constexpr (ZJW >= 1) zrow0 = *zrow_src(c, 0);
        if constexpr (ZJW >= 2) zrow1 = *zrow_src(c, 1);
    };
    auto store_yrows = [&](int c) {
        const char* yt = smem + C::O_Y + (c % 2) * C::ZT;
        const int nv = len - (int64_t)c * CH < CH ? (int)(len - (int64_t)c * CH) : CH;
#pragma unroll
        for (int jj = 0; jj < ZJW; ++jj) {
            const int j = jj * NW + wave;
            int t, x;
            zpos(j, t, x);
            const uint4 v = *reinterpret_cast<const uint4*>(yt + j * 1024 + 16 * lane);
            if (t < nv)
                *reinterpret_cast<uint4*>(reinterpret_cast<char*>(
                    gy + ((t0 + (int64_t)c * CH + t) * H + h) * DV + vcw) + 16 * x) = v;
        }
    };
    // U^T and z of the wave's columns, one chunk ahead in registers
    T4 ut[NTT][NVT], zz[NTT][NVT];
    auto load_uz = [&](int c) {
        const int64_t wsb = (int64_t)(cbase + c) * H + h;
        const T* UT = static_cast<const T*>(p.ws.ut) + wsb * (DV * CH);
        if constexpr (!C::LW) {
#pragma unroll
            for (int ta = 0; ta < NTT; ++ta)
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt) {
                    const int vtg = ident ? 0 : vcol0 / 16 + vt;   // value tile of the U^T block
                    ut[ta][vt] = *reinterpret_cast<const T4*>(UT + ((vtg * NTT + ta) * 64 + lane) * 4);
                }
        }
        if constexpr (C::LW && !C::AUG) {
            if (gz && c == 0) load_zrows(c);   // later chunks' rows go out right after the first barrier
        } else if (!C::AUG && gz) {
            const int nv = len - (int64_t)c * CH < CH ? (int)(len - (int64_t)c * CH) : CH;
#pragma unroll
            for (int ta = 0; ta < NTT; ++ta) {
                const int t = 16 * ta + l16 < nv ? 16 * ta + l16 : nv - 1;
                const int64_t row = ((t0 + (int64_t)c * CH + t) * H + h) * DV;
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt)
                    zz[ta][vt] = *reinterpret_cast<const T4*>(gz + row + vcol0 + 16 * vt + 4 * g4);
            }
        }
    };

    // outputs of the previous chunk, stored in the middle of the next one so
    // that the wait at the top of a chunk never waits for them
    using T4s = T4;
    T4s yd[NTT][NVT];
    int64_t yd_row0 = 0;
    int yd_nvalid = 0;
    auto store_y = [&]() {
#pragma unroll
        for (int ta = 0; ta < NTT; ++ta) {
            const int t = 16 * ta + l16;
            if (t < yd_nvalid) {
                const int64_t row = (yd_row0 + (int64_t)t * H) * DV;   // token t, head h
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt)
                    *reinterpret_cast<T4s*>(gy + row + vcol0 + 16 * vt + 4 * g4) = yd[ta][vt];
            }
        }
    };

    // checkpoint parameters, read once: kernel-argument loads inside the loop
    // would share the LDS wait counter and make every fragment read wait for
    // all the others
    float* ckpt = p.ckpt;
    int ck_every = p.ckpt_every > 0 ? p.ckpt_every : 1;
    int64_t ck_cap = p.ckpt_cap, ck_base = ckpt ? (int64_t)p.ckpt_off[n] : 0;
    asm volatile("" : "+s"(ckpt), "+s"(ck_every), "+s"(ck_cap), "+s"(ck_base));
    if (nch > 0) {
        if constexpr (!C::LW) stage(0, 0, J_0{}, J_E{});
        load_uz(0);
    }
    for (int c = 0; c < nch; ++c) {
        const char* buf = smem + (c % C::NBUF) * C::BUF;
        const int nb = (c + 1) % C::NBUF;
        const int cn = c + 1 < nch ? c + 1 : c;   // the last chunk refetches its own (harmless)
        wait_vmcnt<0>();                           // chunk c (and U^T, z) of this wave
        T4 utc[NTT][NVT], zzc[NTT][NVT];
#pragma unroll
        for (int ta = 0; ta < NTT; ++ta)
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) {
                if constexpr (!C::LW) {
                    utc[ta][vt] = ut[ta][vt];
                    zzc[ta][vt] = zz[ta][vt];
                }
            }
        if constexpr (C::LW && !C::AUG) {
            if (gz) {   // this wave's z rows of chunk c into the z tile
                char* zt = smem + C::O_Z + (c % 2) * C::ZT;
                if constexpr (ZJW >= 1) *reinterpret_cast<uint4*>(zt + wave * 1024 + 16 * lane) = zrow0;
                if constexpr (ZJW >= 2) *reinterpret_cast<uint4*>(zt + (NW + wave) * 1024 + 16 * lane) = zrow1;
            }
        }
        const int nvalid = len - (int64_t)c * CH < CH ? (int)(len - (int64_t)c * CH) : CH;
        // every wave's part of chunk c has landed, and every wave is done with
        // the buffer the next chunk goes to
        barrier_keep_loads();
        if constexpr (C::LW) {
#pragma unroll
            for (int ta = 0; ta < NTT; ++ta)
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt)
                    utc[ta][vt] = *reinterpret_cast<const T4*>(buf + C::NF * 1024 +
                                                               ((wave * NVT + vt) * NTT + ta) * C::UTT +
                                                               lane * 4 * (int)sizeof(T));
            if (!C::AUG && gz) {
                const char* zt = smem + C::O_Z + (c % 2) * C::ZT;
#pragma unroll
                for (int ta = 0; ta < NTT; ++ta)
#pragma unroll
                    for (int vt = 0; vt < NVT; ++vt)
                        zzc[ta][vt] = *reinterpret_cast<const T4*>(zt + zy_off(ta, vt));
                // the next chunk's z rows: in flight for the whole of this chunk
                if constexpr (!C::AUG) load_zrows(cn);
            }
        }

        // Delta = U + Wn S
        Frag sf[NKC][NVT];
#pragma unroll
        for (int s = 0; s < NKC; ++s)
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt)
                sf[s][vt] = K::from_acc(S[s * TPB][vt], S[s * TPB + TPB - 1][vt]);
        f32x4_t D[NTT][NVT];
#pragma unroll
        for (int ta = 0; ta < NTT; ++ta)
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) D[ta][vt] = ident ? f32x4_t{0.f, 0.f, 0.f, 0.f} : to_f32x4(utc[ta][vt]);
        // With one value tile per wave, each phase reads all its fragments
        // before its first product, so that the reads overlap one another
        // instead of each product waiting for its own (two tiles have no
        // registers for that).
        constexpr bool PRE = NVT == 1;
        if constexpr (PRE) {
            Frag wf[NKC][NTT];
#pragma unroll
            for (int s = 0; s < NKC; ++s)
#pragma unroll
                for (int ta = 0; ta < NTT; ++ta) wf[s][ta] = frag(buf, C::F_W + s * NTT + ta);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < NKC; ++s)
#pragma unroll
                for (int ta = 0; ta < NTT; ++ta) D[ta][0] = K::mma(wf[s][ta], sf[s][0], D[ta][0]);
        } else {
#pragma unroll
            for (int s = 0; s < NKC; ++s)
#pragma unroll
                for (int ta = 0; ta < NTT; ++ta) {
                    const Frag wf = frag(buf, C::F_W + s * NTT + ta);
#pragma unroll
                    for (int vt = 0; vt < NVT; ++vt) D[ta][vt] = K::mma(wf, sf[s][vt], D[ta][vt]);
                }
        }
        if constexpr (!C::AUG) {
            if constexpr (C::LW) {
                if (c > 0) store_yrows(c - 1);   // rows of the previous chunk's outputs
            } else if (yd_nvalid > 0) {
                store_y();
            }
        }
        if constexpr (C::NBUF == 2 && !C::LW) stage(cn, nb, J_0{}, J_H{});
        Frag df[NKT][NVT];
#pragma unroll
        for (int u = 0; u < NKT; ++u)
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) {
                const int t1 = u * TPB + TPB - 1;
                df[u][vt] = K::from_acc(D[u * TPB][vt], t1 < NTT ? D[t1 < NTT ? t1 : 0][vt]
                                                                 : f32x4_t{0.f, 0.f, 0.f, 0.f});
            }

        if constexpr (C::LW) barrier_keep_loads();   // group 2 of chunk c (gam, Kh^T, Qt, Pm) has landed
        // S <- gam * S + Kh^T Delta
        const float* gbuf = reinterpret_cast<const float*>(buf + C::F_G * 1024);
        if constexpr (PRE) {
            Frag kf[NCT][NKT];
            f32x4_t gm[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                gm[ct] = *reinterpret_cast<const f32x4_t*>(gbuf + 16 * ct + 4 * g4);
#pragma unroll
                for (int u = 0; u < NKT; ++u) kf[ct][u] = frag(buf, C::F_K + ct * NKT + u);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                S[ct][0] *= gm[ct];
#pragma unroll
                for (int u = 0; u < NKT; ++u) S[ct][0] = K::mma(kf[ct][u], df[u][0], S[ct][0]);
            }
        } else {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const f32x4_t gm = *reinterpret_cast<const f32x4_t*>(gbuf + 16 * ct + 4 * g4);
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt) S[ct][vt] *= gm;
#pragma unroll
                for (int u = 0; u < NKT; ++u) {
                    const Frag kf = frag(buf, C::F_K + ct * NKT + u);
#pragma unroll
                    for (int vt = 0; vt < NVT; ++vt) S[ct][vt] = K::mma(kf, df[u][vt], S[ct][vt]);
                }
            }
        }
        if constexpr (C::NBUF == 2) {
            if constexpr (!C::LW) stage(cn, nb, J_H{}, J_E{});
            if constexpr (!C::LW) load_uz(cn);
        }
        if constexpr (!C::AUG) {
            // prefix-cache checkpoint: the state after this chunk
            if (ckpt && (c + 1) % ck_every == 0 && (int64_t)(c + 1) * CH <= len) {
                const int64_t row = ck_base + (c + 1) / ck_every - 1;
                if (row < ck_cap) {
                    // global address space: a generic store would also count on the
                    // LDS wait counter
                    __attribute__((address_space(1))) float* dst =
                        (__attribute__((address_space(1))) float*)(ckpt + (row * H + h) * DK * (int64_t)DV);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                        for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                dst[(16 * ct + 4 * g4 + i) * DV + colw + 16 * vt + l16] = S[ct][vt][i];
                }
            }
        }

        if constexpr (!C::AUG) {
            // O^T = S_old^T Qt^T + Delta^T Pm^T, then the gate
            f32x4_t O[NVT][NTT];
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
                for (int ta = 0; ta < NTT; ++ta) O[vt][ta] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if constexpr (PRE) {
                Frag qf[NKC][NTT], pf[NTT][NKT];
#pragma unroll
                for (int s = 0; s < NKC; ++s)
#pragma unroll
                    for (int ta = 0; ta < NTT; ++ta) qf[s][ta] = frag(buf, C::F_Q + s * NTT + ta);
#pragma unroll
                for (int ta = 0; ta < NTT; ++ta)
#pragma unroll
                    for (int u = 0; u < NKT; ++u)
                        if (u * KB <= 16 * ta + 15) pf[ta][u] = frag(buf, C::F_P + pm_frag_index(ta, u, NKT, KB));
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int s = 0; s < NKC; ++s)
#pragma unroll
                    for (int ta = 0; ta < NTT; ++ta) O[0][ta] = K::mma(sf[s][0], qf[s][ta], O[0][ta]);
#pragma unroll
                for (int ta = 0; ta < NTT; ++ta)
#pragma unroll
                    for (int u = 0; u < NKT; ++u)
                        if (u * KB <= 16 * ta + 15) O[0][ta] = K::mma(df[u][0], pf[ta][u], O[0][ta]);
            } else {
#pragma unroll
                for (int s = 0; s < NKC; ++s)
#pragma unroll
                    for (int ta = 0; ta < NTT; ++ta) {
                        const Frag qf = frag(buf, C::F_Q + s * NTT + ta);
#pragma unroll
                        for (int vt = 0; vt < NVT; ++vt) O[vt][ta] = K::mma(sf[s][vt], qf, O[vt][ta]);
                    }
#pragma unroll
                for (int ta = 0; ta < NTT; ++ta)
#pragma unroll
                    for (int u = 0; u < NKT; ++u)
                        if (u * KB <= 16 * ta + 15) {
                            const Frag pf = frag(buf, C::F_P + pm_frag_index(ta, u, NKT, KB));
#pragma unroll
                            for (int vt = 0; vt < NVT; ++vt) O[vt][ta] = K::mma(df[u][vt], pf, O[vt][ta]);
                        }
            }
#pragma unroll
            for (int ta = 0; ta < NTT; ++ta)
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt) {
                    f32x4_t o = O[vt][ta];
                    if (gz) {
                        const f32x4_t zf = to_f32x4(zzc[ta][vt]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) o[i] *= sigmoid(zf[i]);
                    }
                    if constexpr (C::LW)
                        *reinterpret_cast<T4*>(smem + C::O_Y + (c % 2) * C::ZT + zy_off(ta, vt)) = from_f32x4<T>(o);
                    else
                        yd[ta][vt] = from_f32x4<T>(o);
                }
            yd_row0 = (t0 + (int64_t)c * CH) * H + h;
            yd_nvalid = nvalid;
        }
        if constexpr (C::NBUF == 1) {
            barrier_keep_loads();                  // buffer free for the next chunk
            if (c + 1 < nch) {
                stage(c + 1, 0, J_0{}, J_E{});
                load_uz(c + 1);
            }
        }
    }
    if constexpr (!C::AUG && !C::LW) {
        if (yd_nvalid > 0) store_y();             // outputs of the last chunk
    }
    if constexpr (!C::AUG && C::LW) {
        if (nch > 0) {
            barrier_keep_loads();                 // every wave's outputs of the last chunk are in LDS
            store_yrows(nch - 1);
        }
    }

    // ---- final state ---------------------------------------------------------
    if (p.sfin && n >= p.final_seq_lo) {
        const int64_t sb = ((int64_t)(n - p.final_seq_lo) * H + h) * DK * (int64_t)dvt;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) {
                const int col = colw + 16 * vt + l16;
#pragma unroll
                for (int i = 0; i < 4; ++i) p.sfin[sb + (int64_t)(16 * ct + 4 * g4 + i) * dvt + col] = S[ct][vt][i];
            }
    }
}

// Per-sequence plan: chunk offsets, a longest-first order, checkpoint offsets
// (each output optional).  One workgroup; prefix sums in rounds of 256.
__global__ __launch_bounds__(256) void varlen_plan_kernel(int N, const int32_t* __restrict__ cu, int64_t T_total,
                                                          int CH, int ckpt_interval,
                                                          int32_t* __restrict__ chunk_off,
                                                          int32_t* __restrict__ order,
                                                          int32_t* __restrict__ ckpt_off) {
    __shared__ int buf[2][256];
    const int tid = threadIdx.x;
    auto seq_len = [&](int i) -> int64_t {
        if (!cu) return T_total;
        const int64_t l = (int64_t)cu[i + 1] - cu[i];
        return l > 0 ? l : 0;
    };
    int carry0 = 0, carry1 = 0;
    for (int base = 0; base < N; base += 256) {
        const int i = base + tid;
        int x0 = 0, x1 = 0;
        if (i < N) {
            const int64_t l = seq_len(i);
            x0 = (int)((l + CH - 1) / CH);
            x1 = ckpt_interval > 0 ? (int)(l / ckpt_interval) : 0;
        }
        buf[0][tid] = x0;
        buf[1][tid] = x1;
        __syncthreads();
        for (int d = 1; d < 256; d <<= 1) {
            const int y0 = tid >= d ? buf[0][tid - d] : 0;
            const int y1 = tid >= d ? buf[1][tid - d] : 0;
            __syncthreads();
            buf[0][tid] += y0;
            buf[1][tid] += y1;
            __syncthreads();
        }
        if (i < N) {
            if (chunk_off) chunk_off[i] = carry0 + buf[0][tid] - x0;
            if (ckpt_off) ckpt_off[i] = carry1 + buf[1][tid] - x1;
        }
        carry0 += buf[0][255];
        carry1 += buf[1][255];
        __syncthreads();
    }
    if (tid == 0) {
        if (chunk_off) chunk_off[N] = carry0;
        if (ckpt_off) ckpt_off[N] = carry1;
    }
    if (!order) return;
    for (int i = tid; i < N; i += 256) {
        int rank = i;
        if (N <= 1024) {
            const int64_t li = seq_len(i);
            rank = 0;
            for (int j = 0; j < N; ++j) {
                const int64_t lj = seq_len(j);
                rank += (lj > li) || (lj == li && j < i);
            }
        }
        order[rank] = i;
    }
}

// ---------------------------------------------------------------------------
template <class C>
static hipError_t launch_state_cfg(const TwoPassArgs& a, const int32_t* chunk_off, const int32_t* order) {
    StateParams p;
    p.chunk_cap = (int)a.chunk_cap;
    p.H = a.H;
    p.num_seqs = a.num_seqs;
    p.nchains = a.num_seqs * a.H;
    p.dvt = C::AUG ? a.dk + a.dv : a.dv;
    p.nvg = p.dvt / C::CW;
    p.final_seq_lo = a.final_seq_lo;
    p.cps = (int)((a.seg_len + a.chunk - 1) / a.chunk);
    p.T_total = a.T_total;
    p.seg_len = a.seg_len;
    p.cu_seqlens = a.cu_seqlens;
    p.chunk_off = chunk_off;
    p.order = order;
    p.z = a.z;
    p.y = a.y;
    p.s0 = a.initial_state;
    p.sfin = a.final_state;
    p.ws = a.bufs;
    p.ckpt = a.ckpt;
    p.ckpt_off = a.ckpt_off;
    p.ckpt_every = a.ckpt_every > 0 ? a.ckpt_every : 1;
    p.ckpt_cap = a.ckpt_cap;
    if (p.nchains == 0) return hipSuccess;
    auto kern = chunk_state_kernel<C>;
    if (C::BYTES > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute((const void*)kern,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, C::BYTES);
        if (e != hipSuccess) return e;
    }
    const long nblk = (long)((p.nchains + 7) / 8) * 8 * p.nvg;
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(C::NTHR), C::BYTES, (hipStream_t)a.stream, p);
    return hipGetLastError();
}

template <class E, int DK, int CH, int MODE>
static hipError_t launch_state_nvt(const TwoPassArgs& a, const int32_t* co, const int32_t* ord) {
    // One value tile per wave wherever loader waves apply, whatever the
    // number of chains (on the 16-sequence varlen layer 2.84 ms against 3.04
    // with two tiles); the transition pairs, with dk + dv columns a chain,
    // keep the choice made from the chain count (two tiles: 0.74 ms against
    // 1.07 for 1024 chains).
    using C1 = StCfg<E, DK, DK, CH, 1, MODE>;
    if (a.nvt == 1 || (C1::LW && MODE != kModePairs)) return launch_state_cfg<C1>(a, co, ord);
    return launch_state_cfg<StCfg<E, DK, DK, CH, 2, MODE>>(a, co, ord);
}

template <class E, int DK, int CH>
static hipError_t launch_state_mode(const TwoPassArgs& a, const int32_t* co, const int32_t* ord) {
    switch (a.mode) {
        case kModeSeq: return launch_state_nvt<E, DK, CH, kModeSeq>(a, co, ord);
        case kModeVarlen: return launch_state_nvt<E, DK, CH, kModeVarlen>(a, co, ord);
        case kModePairs: return launch_state_nvt<E, DK, CH, kModePairs>(a, co, ord);
        default: return launch_state_nvt<E, DK, CH, kModeFinish>(a, co, ord);
    }
}

template <class E, int DK>
static hipError_t launch_state_dk(const TwoPassArgs& a, const int32_t* co, const int32_t* ord) {
    if (a.chunk == 64) return launch_state_mode<E, DK, 64>(a, co, ord);
    if (a.chunk == 32) return launch_state_mode<E, DK, 32>(a, co, ord);
    return launch_state_mode<E, DK, 16>(a, co, ord);
}

hipError_t launch_chunk_state(const TwoPassArgs& a, const int32_t* chunk_off, const int32_t* order) {
    if (a.dtype == 0)
        return a.dk == 128 ? launch_state_dk<BF16, 128>(a, chunk_off, order)
                           : launch_state_dk<BF16, 64>(a, chunk_off, order);
    return a.dk == 128 ? launch_state_dk<F32, 128>(a, chunk_off, order)
                       : launch_state_dk<F32, 64>(a, chunk_off, order);
}

hipError_t launch_varlen_plan(int num_seqs, const int32_t* cu_seqlens, int64_t T_total, int chunk,
                              int ckpt_interval, int32_t* chunk_off, int32_t* order, int32_t* ckpt_off,
                              void* stream) {
    hipLaunchKernelGGL(varlen_plan_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, num_seqs, cu_seqlens,
                       T_total, chunk, ckpt_interval, chunk_off, order, ckpt_off);
    return hipGetLastError();
}

}  // namespace kda
