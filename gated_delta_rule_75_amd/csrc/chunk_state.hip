// State scan: carries the state of every (sequence, head) through its chunks
// with the per-chunk products the preparation kernel stored (twopass.h):
//     Delta = U + Wn S,   O = Qt S + Pm Delta,   S <- gam * S + Kh^T Delta,
//     y = O * sigmoid(z),
// where U = T V is formed here, from T = L^{-1} diag(beta) and the chunk's v.
//
// State columns evolve independently.  A workgroup of NW waves owns
// 16 NVT NW consecutive columns of one (sequence, head); each wave owns
// 16 NVT of them and keeps its part of S and Delta in MFMA accumulator tiles,
// fed back as operands straight from the lanes that hold them (the k-block
// order of twopass.h).  The chunk operands every wave needs (Wn, Qt, Kh^T,
// Pm, T, gam) and the workgroup's rows of v are copied once per workgroup
// into LDS, double-buffered so chunk c+1 streams in while chunk c is
// computed.  In LDS each operand fragment (16 rows x one k-block) is stored
// in lane order, 16 bytes per lane, so that every wave reads a fragment with
// one conflict-free 16-byte access per lane.  Without loader waves (below),
// z, private to a wave, goes straight to registers one chunk ahead.
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
// v rows fit in LDS (one value tile per wave), four extra waves do all the
// staging of later chunks while chunk c is computed and meet the compute
// waves at its barriers (two per chunk: one once v, T and Wn, the operands of
// Delta, are in; one before the state update, once the rest is).  v, T and Wn
// go out one and a half chunks ahead, into the slots of the buffer whose
// chunk has just passed its middle barrier; the rest one chunk ahead.  A wave that issues a 1 KiB copy stalls until
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
    int chunk_cap;          // bound on the global chunk count
    int slab_lo, slab_hi;   // global chunks whose products the workspace holds
    int rect_w, rect_c0, rect_s0, rect_s1;   // or a rectangle of segments x chunks (rect_w > 0)
    int first_slab;         // chains without chunks run here
    float* carry;           // state between slabs, [num_seqs, H, dk, dvt]
    int64_t T_total, seg_len;
    const int32_t* cu_seqlens;
    const int32_t* chunk_off;
    const int32_t* order;
    const void* v;
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

template <typename E_, int DK_, int DV_, int CH_, int NVT_, int MODE_, int NW_ = 4>
struct StCfg {
    using E = E_;
    using K = KBlk<E_>;
    using T = typename K::T;
    static constexpr int DK = DK_, DV = DV_, CH = CH_, NVT = NVT_, MODE = MODE_;
    static constexpr bool AUG = MODE_ == kModePairs;
    static constexpr int NW = NW_;                      // compute waves
    static constexpr int CW = 16 * NVT * NW;            // state columns per workgroup
    static constexpr int NTT = CH / 16, NCT = DK / 16;
    static constexpr int KB = K::KB, TPB = K::TPB;
    static constexpr int NKC = DK / KB;                 // k-blocks over channels
    static constexpr int CP = (CH + KB - 1) / KB * KB;
    static constexpr int NKT = CP / KB;                 // k-blocks over tokens
    static_assert(NKC * TPB == NCT, "channel k-blocks");
    static constexpr int NPM = pm_frags(NTT, NKT, KB);  // stored fragments of Pm
    // fragment index ranges in an LDS buffer (1 KiB each)
    // The KCP pairs with two value tiles a wave mix their columns: waves
    // 0 .. NW/2-1 take transition columns and the others value columns, so
    // each workgroup needs v for half its columns, and T and the v rows sit
    // in one region of their own (restaged mid-chunk) while the rest is
    // double-buffered: with four waves (half of a chain's columns) 80 KB, two
    // workgroups a CU; with eight (all of them at dk = 128) 88 KB, one.
    static constexpr bool MIX = AUG && NVT == 2;
    static constexpr int F_W = 0, N_W = NKC * NTT;
    static constexpr int N_T = NPM;                     // L^{-1} diag(beta), operand of U = T V
    static constexpr int F_T0 = F_W + N_W;              // T beside Wn (loader group 1: v, Wn, T)
    static constexpr int F_Q = MIX ? F_T0 : F_T0 + N_T, N_Q = AUG ? 0 : NKC * NTT;
    static constexpr int F_K = F_Q + N_Q, N_K = NCT * NKT;
    static constexpr int F_P = F_K + N_K, N_P = AUG ? 0 : NPM;
    static constexpr int F_G = F_P + N_P;               // gam: dk fp32, repeated to fill 1 KiB
    static constexpr int NFB = F_G + 1;                 // fragments held in a buffer
    static constexpr int F_T = MIX ? NFB : F_T0;        // MIX: T after those, in its own region
    static constexpr int NF = NFB + (MIX ? N_T : 0);
    static constexpr int FPW = (NFB + NW - 1) / NW;     // buffered fragment loads per wave
    // rows of v for the workgroup's columns, after the fragments: [CH][CW]
    // row-major, the 16-byte units of row t stored at unit x ^ vswz(t), so
    // that the rows one k-block spreads over the four lane groups of a
    // fragment read land in different banks.  Copied by the loader waves, or
    // without them by the compute waves beside their share of the fragments
    static constexpr int VCOLS = MIX ? CW / 2 : CW;     // value columns of a workgroup
    static constexpr int VRB = VCOLS * (int)sizeof(T);  // bytes of one row
    static constexpr int VTB = CH * VRB;
    static constexpr int VRPC = 1024 / VRB;             // rows per 1 KiB copy
    static_assert(VTB % 1024 == 0 && 1024 % VRB == 0, "v rows in whole 1 KiB copies");
    // z and y tiles of the workgroup's columns, [CH][CW] row-major in LDS with
    // the 16-byte units of row t stored at unit x ^ (t % ZXR), which spreads
    // the 16 rows a wave's fragment access touches over the banks
    static constexpr int ZRB = CW * (int)sizeof(T);        // bytes of one token row
    static constexpr int ZXR = ZRB / 16;                   // 16-byte units per row
    static constexpr int ZT = AUG ? 0 : CH * ZRB;          // bytes of a z or y tile
    // loader waves (with two value tiles per wave the compute waves' registers
    // are at the 256 limit already; they keep staging their own operands);
    // the z and y rows go in whole 1 KiB copies per compute wave
    static constexpr bool LW = NVT == 1 && ZT % (1024 * NW) == 0 && 2 * (NF * 1024 + VTB) + 2 * ZT <= 160 * 1024;
    static constexpr int BUF = NFB * 1024 + (MIX ? 0 : VTB);
    static constexpr int NVC = VTB / 1024;              // v-row copies per chunk
    static constexpr int VPW = (NVC + NW - 1) / NW;     // of them per compute wave (no loader waves)
    // double buffers unless the pairs, whose workgroups fit two to a CU in
    // registers, would then lose that: one buffer each, and the other
    // workgroup of the CU overlaps the copies instead
    static constexpr int NBUF = LW || MIX ? 2 : AUG && 2 * BUF > 80 * 1024 && BUF <= 80 * 1024 ? 1
                                              : 2 * BUF <= 150 * 1024 ? 2 : 1;
    // with LW: one z tile and one y tile.  The z rows of chunk c are written
    // at its top, after every wave has passed the second barrier of chunk c-1
    // and so has read its z of chunk c-1; the outputs of chunk c are written
    // after its second barrier, by which every wave has stored chunk c-1's
    // rows out of the tile
    static constexpr int O_Z = NBUF * BUF;
    static constexpr int O_Y = O_Z + ZT;
    static constexpr int O_TV = NBUF * BUF;                // MIX: T fragments, then the v rows
    static constexpr int BYTES = NBUF * BUF + (LW ? 2 * ZT : 0) + (MIX ? N_T * 1024 + VTB : 0);
    static_assert(BYTES <= 160 * 1024, "LDS");
    static_assert(!MIX || sizeof(T) == 4 || NW != 4 || BYTES <= 80 * 1024, "two pairs workgroups a CU");
    // loader waves: four (with the copies dealt round-robin, two, three and
    // four loaders reach 324, 317 and 314 us on the 96-head layer)
    static constexpr int NLW = LW ? 4 : 0;
    static constexpr int NCOPY = NF + NVC;                   // 1 KiB copies per chunk (LW)
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

// 16-byte unit swizzle of a v row in LDS: the KPL-row groups that the four
// lane groups of a fragment read fall on different units
template <class C>
__device__ __forceinline__ int vswz(int row) {
    return ((row / (C::KB / 4)) & 3) * (int)sizeof(typename C::T);
}

// 16 bytes as a native vector (arrays of it stay in registers)
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

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
    // stay inside T_total and the chunk bound whatever the offsets say
    if (t0 >= p.T_total) len = 0;
    else if (t0 + len > p.T_total) len = p.T_total - t0;
    int nch = len > 0 ? (int)((len + CH - 1) / CH) : 0;
    if (cbase + nch > p.chunk_cap) nch = cbase < p.chunk_cap ? p.chunk_cap - cbase : 0;
    const int dvt = p.dvt;
    // the chain's chunks [cb, ce) inside this slab; the chain is then shifted so
    // that its window starts at chunk 0 (tokens t0.., workspace block cws + c)
    const int64_t len_chain = len;
    int cb = 0, ce = nch;
    const bool rect = p.rect_w > 0;
    const bool mine = !rect || (n >= p.rect_s0 && n < p.rect_s1);
    if (rect) {
        cb = mine ? (p.rect_c0 < nch ? p.rect_c0 : nch) : nch;
        ce = mine ? (p.rect_c0 + p.rect_w < nch ? p.rect_c0 + p.rect_w : nch) : 0;
    } else {
        if (p.slab_lo > cbase) cb = p.slab_lo - cbase < nch ? p.slab_lo - cbase : nch;
        if (p.slab_hi < cbase + nch) ce = p.slab_hi > cbase ? p.slab_hi - cbase : 0;
    }
    if (ce <= cb) {
        if (nch > 0 || !p.first_slab || !mine) return;   // nothing of this chain in the slab
        cb = ce = 0;
    }
    const bool from_start = cb == 0, to_end = ce == nch;
    t0 += (int64_t)cb * CH;
    len = len - (int64_t)cb * CH < (int64_t)(ce - cb) * CH ? len - (int64_t)cb * CH : (int64_t)(ce - cb) * CH;
    const int ck0 = cb;                      // chunks of the chain before the window
    // workspace block of the window's first chunk
    const int cws = rect ? (n - p.rect_s0) * p.rect_w + cb - p.rect_c0 : cbase + cb - p.slab_lo;
    nch = ce - cb;
    // first value tile (16 columns of v / U) of the workgroup; negative for
    // the transition columns of mode 2, whose waves take no values
    const int vt_wg = C::MIX ? vg * C::VCOLS / 16 : (vg * C::CW - (C::AUG ? DK : 0)) / 16;
    const T* gv = static_cast<const T*>(p.v);

    if constexpr (C::LW) {
        if (wave >= NW) {
            // ---- loader waves: the operands of later chunks into LDS while chunk c is computed ----
            constexpr int FB = 64 * KPL * (int)sizeof(T);   // bytes of one fragment (1 KiB)
            static_assert(FB == 1024, "fragment size");
            const char* wn = static_cast<const char*>(p.ws.wn) + 16 * lane;
            const char* qt = static_cast<const char*>(p.ws.qt) + 16 * lane;
            const char* kh = static_cast<const char*>(p.ws.kht) + 16 * lane;
            const char* pm = static_cast<const char*>(p.ws.pm) + 16 * lane;
            const char* gm = reinterpret_cast<const char*>(p.ws.gam) + 16 * (lane % (DK / 4));
            const char* tt = static_cast<const char*>(p.ws.tt) + 16 * lane;
            // v rows: lane l of copy j holds row j VRPC + l / units, its
            // 16-byte unit x stored at x ^ vswz(row); the columns of a
            // transition workgroup (mode 2) take no values: any valid row
            constexpr int VU = C::VRB / 16;                    // units per row
            const int vrow_l = lane / VU, vx = lane % VU;
            const int vcol_wg = vt_wg > 0 ? 16 * vt_wg : 0;
            // copy j of a chunk (1 KiB): the v rows first (private to the
            // workgroup, so never in L2 already), then Wn, T, gam, Kh^T, Qt, Pm;
            // LDS slot k of copy j: fragment k, or v-row copy k - NF.  The copies
            // are dealt to the loaders in turn.  Group 1 (v, Wn, T: the operands
            // of Delta, read before the middle barrier) and group 2 (gam, Kh^T,
            // Qt, Pm, read after it) go straight into LDS:
            //   after the middle barrier of chunk c, group 2 of chunk c+1 into
            //   buffer (c+1) % 2, then group 1 of chunk c+2 into the group-1
            //   slots of buffer c % 2, which every compute wave has finished
            //   reading by that barrier.
            // Group 1 then has one and a half chunks to land, group 2 one.  The
            // waits count copies, which relies on vector memory operations
            // completing in issue order.
            constexpr int NU = C::NCOPY - C::NF;
            constexpr int NG1 = NU + C::N_W + C::N_T;
            auto src_of = [&](int c, int k) __attribute__((always_inline)) -> const char* {
                const int64_t wsb = (int64_t)(cws + c) * H + h;
                if (k < C::F_T0) return wn + wsb * (int64_t)(CH * DK * sizeof(T)) + (k - C::F_W) * FB;
                if (k < C::F_Q) return tt + wsb * (int64_t)(C::NPM * FB) + (k - C::F_T0) * FB;
                if (k < C::F_K) return qt + wsb * (int64_t)(CH * DK * sizeof(T)) + (k - C::F_Q) * FB;
                if (k < C::F_P) return kh + wsb * (int64_t)(DK * CP * sizeof(T)) + (k - C::F_K) * FB;
                if (k < C::F_G) return pm + wsb * (int64_t)(C::NPM * FB) + (k - C::F_P) * FB;
                if (k == C::F_G) return gm + wsb * (int64_t)(DK * sizeof(float));
                // v row of this lane (rows past the chunk's end repeat its last one)
                const int nv = len - (int64_t)c * CH < CH ? (int)(len - (int64_t)c * CH) : CH;
                int row = (k - C::NF) * C::VRPC + vrow_l;
                row = row < nv ? row : nv - 1;
                return reinterpret_cast<const char*>(gv + ((t0 + (int64_t)c * CH + row) * H + h) * DV + vcol_wg) +
                       16 * (vx ^ vswz<C>(row));
            };
            // the loader's program, with its index LI a constant, so that each
            // copy's slot and source array fold at compile time
            auto loader = [&](auto LI) __attribute__((always_inline)) {
                constexpr int li = decltype(LI)::value;
                constexpr auto kslot = [](int j) -> int {
                    if (j < NU) return C::NF + j;                     // v rows
                    j -= NU;
                    if (j < C::N_W + C::N_T) return C::F_W + j;       // Wn, then T
                    j -= C::N_W + C::N_T;
                    if (j == 0) return C::F_G;
                    if (j <= C::N_K) return C::F_K + j - 1;
                    if (j <= C::N_K + C::N_Q) return C::F_Q + j - 1 - C::N_K;
                    return C::F_P + j - 1 - C::N_K - C::N_Q;
                };
                // copies of this loader in group 1 and in group 2
                constexpr int N1 = (NG1 - li + C::NLW - 1) / C::NLW;
                constexpr int N2 = (C::NCOPY - li + C::NLW - 1) / C::NLW - N1;
                static_assert(N1 + N2 <= 63, "vmcnt range");
                auto copy_g1 = [&](int c, int b) __attribute__((always_inline)) {
                    char* buf = smem + b * C::BUF;
#pragma unroll
                    for (int j = 0; j < NG1; ++j)
                        if (j % C::NLW == li) lds_dma16(src_of(c, kslot(j)), buf + kslot(j) * 1024);
                };
                auto copy_g2 = [&](int c, int b) __attribute__((always_inline)) {
                    char* buf = smem + b * C::BUF;
#pragma unroll
                    for (int j = NG1; j < C::NCOPY; ++j)
                        if (j % C::NLW == li) lds_dma16(src_of(c, kslot(j)), buf + kslot(j) * 1024);
                };
                // the waits below count on this issue order, which the
                // scheduling barriers keep
                if (nch > 0) {
                    copy_g1(0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    copy_g2(0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    if (nch > 1) copy_g1(1, 1);
                }
                for (int c = 0; c < nch; ++c) {
                    // group 1 of chunk c has landed (group 2 of c and group 1 of c+1 may be in flight)
                    if (c + 1 < nch) wait_vmcnt<N1 + N2>();
                    else wait_vmcnt<N2>();
                    barrier_keep_loads();       // group 1 of chunk c is in LDS; the compute waves are done with chunk c-1
                    if (c + 1 < nch) wait_vmcnt<N1>();   // group 2 of chunk c (group 1 of c+1 may be in flight)
                    else wait_vmcnt<0>();
                    barrier_keep_loads();       // group 2 of chunk c is in LDS
                    if (c + 1 < nch) copy_g2(c + 1, (c + 1) % 2);
                    __builtin_amdgcn_sched_barrier(0);
                    if (c + 2 < nch) copy_g1(c + 2, c % 2);
                }
            };
            static_assert(C::NLW == 4, "loader count");
            switch (wave - NW) {
                case 0: loader(std::integral_constant<int, 0>{}); break;
                case 1: loader(std::integral_constant<int, 1>{}); break;
                case 2: loader(std::integral_constant<int, 2>{}); break;
                default: loader(std::integral_constant<int, 3>{}); break;
            }
            if constexpr (!C::AUG) {
                if (nch > 0) barrier_keep_loads();   // matches the compute waves' last y hand-off
            }
            return;
        }
    }

    // first state column of the wave (MIX: the first half of the waves on
    // transition columns, the second half on value columns)
    const int colw = !C::MIX ? vg * C::CW + wave * 16 * NVT
                   : wave < NW / 2 ? vg * C::VCOLS + wave * 16 * NVT
                                   : DK + vg * C::VCOLS + (wave - NW / 2) * 16 * NVT;
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
    // entering state: the initial state at the chain's first chunk (zeros, or
    // [I | 0] for the pairs), the carry of the previous slab otherwise
    const float* sinit = from_start ? (C::AUG ? nullptr : p.s0) : p.carry;
    if (sinit) {
        const float* s0 = sinit + ((int64_t)n * H + h) * DK * (int64_t)dvt;
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
        f = f < C::NFB ? f : C::NFB - 1;   // the last wave repeats its last fragment
        constexpr int FB = 64 * KPL * (int)sizeof(T);   // bytes of one fragment
        if (f < C::F_T0) {
            fbase[j] = static_cast<const char*>(p.ws.wn);
            fstride[j] = (int64_t)CH * DK * sizeof(T);
            foff[j] = (f - C::F_W) * FB;
        } else if (f < C::F_T0 + C::N_T && !C::MIX) {
            fbase[j] = static_cast<const char*>(p.ws.tt);
            fstride[j] = (int64_t)C::NPM * FB;
            foff[j] = (f - C::F_T0) * FB;
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
    // v-row copies wave + NW j of chunk c (no loader waves): lane l holds row
    // copy * VRPC + l / units, its unit x stored at x ^ vswz(row)
    auto stage_v = [&](int c, int b) {
        if (vt_wg < 0) return;                     // transition columns: no values
        constexpr int VU = C::VRB / 16;
        const int nv = len - (int64_t)c * CH < CH ? (int)(len - (int64_t)c * CH) : CH;
        char* buf = C::MIX ? smem + C::O_TV + C::N_T * 1024 : smem + b * C::BUF + C::NFB * 1024;
#pragma unroll
        for (int j = 0; j < C::VPW; ++j) {
            const int cp = wave + NW * j;
            if (cp < C::NVC) {
                int row = cp * C::VRPC + lane / VU;
                row = row < nv ? row : nv - 1;
                lds_dma16(reinterpret_cast<const char*>(gv + ((t0 + (int64_t)c * CH + row) * H + h) * DV + 16 * vt_wg) +
                              16 * ((lane % VU) ^ vswz<C>(row)),
                          buf + cp * 1024);
            }
        }
    };
    // fragments [J0, J1) of this wave's share of chunk c into LDS buffer b
    // (with J0 = 0 also its v-row copies, except with MIX)
    auto stage = [&](int c, int b, auto J0, auto J1) {
        const int64_t wsb = (int64_t)(cws + c) * H + h;
        char* buf = smem + b * C::BUF;
        if constexpr (decltype(J0)::value == 0 && !C::MIX) stage_v(c, b);
#pragma unroll
        for (int j = decltype(J0)::value; j < decltype(J1)::value; ++j) {
            const int f = wave + NW * j < C::NFB ? wave + NW * j : C::NFB - 1;
            lds_dma16(fbase[j] + wsb * fstride[j] + foff[j], buf + f * 1024);
        }
    };
    // MIX: T fragments and v rows of chunk c into their own region
    auto stage_tv = [&](int c) {
        const int64_t wsb = (int64_t)(cws + c) * H + h;
        const char* tsrc = static_cast<const char*>(p.ws.tt) + wsb * (int64_t)(C::NPM * 1024) + 16 * lane;
#pragma unroll
        for (int f = wave; f < C::N_T; f += NW) lds_dma16(tsrc + f * 1024, smem + C::O_TV + f * 1024);
        stage_v(c, 0);
    };
    // fragment i of T for buffer buf
    auto tfrag = [&](const char* buf, int i) -> Frag {
        const char* at = C::MIX ? smem + C::O_TV + i * 1024 : buf + (C::F_T + i) * 1024;
        return *reinterpret_cast<const Frag*>(at + 16 * lane);
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
    u32x4_t zrow[ZJW > 0 ? ZJW : 1];   // rows in flight (copies wave, wave + NW, ...)
    auto zrow_src = [&](int c, int jj) -> const u32x4_t* {
        const int nv = len - (int64_t)c * CH < CH ? (int)(len - (int64_t)c * CH) : CH;
        int t, x;
        zpos(jj * NW + wave, t, x);
        t = t < nv ? t : nv - 1;
        return reinterpret_cast<const u32x4_t*>(
            reinterpret_cast<const char*>(gz + ((t0 + (int64_t)c * CH + t) * H + h) * DV + vcw) + 16 * x);
    };
    auto load_zrows = [&](int c) {
#pragma unroll
        for (int jj = 0; jj < ZJW; ++jj) zrow[jj] = *zrow_src(c, jj);
    };
    auto store_yrows = [&](int c) {
        const char* yt = smem + C::O_Y;
        const int nv = len - (int64_t)c * CH < CH ? (int)(len - (int64_t)c * CH) : CH;
#pragma unroll
        for (int jj = 0; jj < ZJW; ++jj) {
            const int j = jj * NW + wave;
            int t, x;
            zpos(j, t, x);
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(yt + j * 1024 + 16 * lane);
            // written once, read by nobody here: stored past the caches
            if (t < nv)
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(
                    gy + ((t0 + (int64_t)c * CH + t) * H + h) * DV + vcw) + 16 * x));
        }
    };
    // B operand of U = T V for value tile vt of the wave: lane (group g4,
    // column l16) holds v at the KPL tokens u KB + g4 KPL + e of k-block u, in
    // the order the T fragments were stored (tokens past the chunk are zero in
    // T; those past C give zeros here, those past the data repeat the last row)
    auto vfrag_elem = [&](int u, int e) { return u * KB + g4 * KPL + e; };
    // without loader waves: z of the wave's columns, one chunk ahead in registers
    T4 zz[NTT][NVT];
    auto load_uz = [&](int c) {
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
        if constexpr (C::MIX) stage_tv(0);
        load_uz(0);
    }
    for (int c = 0; c < nch; ++c) {
        const char* buf = smem + (c % C::NBUF) * C::BUF;
        const int nb = (c + 1) % C::NBUF;
        const int cn = c + 1 < nch ? c + 1 : c;   // the last chunk refetches its own (harmless)
        wait_vmcnt<0>();                           // chunk c (and v, z) of this wave
        T4 zzc[NTT][NVT];
        Frag vfc[NVT][NKT];
        if constexpr (!C::LW) {
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
                for (int ta = 0; ta < NTT; ++ta) zzc[ta][vt] = zz[ta][vt];
        }
        if constexpr (C::LW && !C::AUG) {
            if (gz) {   // this wave's z rows of chunk c into the z tile
                char* zt = smem + C::O_Z;
#pragma unroll
                for (int jj = 0; jj < ZJW; ++jj)
                    *reinterpret_cast<u32x4_t*>(zt + (jj * NW + wave) * 1024 + 16 * lane) = zrow[jj];
            }
        }
        const int nvalid = len - (int64_t)c * CH < CH ? (int)(len - (int64_t)c * CH) : CH;
        // every wave's part of chunk c has landed, and every wave is done with
        // the buffer the next chunk goes to
        barrier_keep_loads();
        // the KCP pairs have no output phase to hide their copies behind: all
        // of the next chunk's fragments go out now, a whole chunk ahead
        if constexpr (C::AUG && C::NBUF == 2 && !C::LW) stage(cn, nb, J_0{}, J_E{});
        // the wave's v fragments from the v rows of the chunk
        if (!ident) {
            const char* vt_rows = C::MIX ? smem + C::O_TV + C::N_T * 1024 : buf + C::NFB * 1024;
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
                for (int u = 0; u < NKT; ++u)
#pragma unroll
                    for (int e = 0; e < KPL; ++e) {
                        const int row = vfrag_elem(u, e);
                        const int wv = C::MIX ? wave - NW / 2 : wave;   // the wave's place among the value columns
                        const int cb = (wv * 16 * NVT + 16 * vt + l16) * (int)sizeof(T);
                        const T x = row < CH ? *reinterpret_cast<const T*>(vt_rows + row * C::VRB +
                                                                           ((cb / 16) ^ vswz<C>(row)) * 16 + cb % 16)
                                             : from_f32<T>(0.f);
                        K::set(vfc[vt][u], e, x);
                    }
        }
        if constexpr (C::LW) {
            if (!C::AUG && gz) {
                const char* zt = smem + C::O_Z;
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
        // U = T V (T lower triangular: k-blocks on or below the diagonal tile)
        f32x4_t D[NTT][NVT];
#pragma unroll
        for (int ta = 0; ta < NTT; ++ta)
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) D[ta][vt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (!ident) {
#pragma unroll
            for (int ta = 0; ta < NTT; ++ta)
#pragma unroll
                for (int u = 0; u < NKT; ++u)
                    if (u * KB <= 16 * ta + 15) {
                        const Frag tf = tfrag(buf, pm_frag_index(ta, u, NKT, KB));
#pragma unroll
                        for (int vt = 0; vt < NVT; ++vt) D[ta][vt] = K::mma(tf, vfc[vt][u], D[ta][vt]);
                    }
        }
        // With one value tile per wave, each phase reads all its fragments
        // before its first product, so that the reads overlap one another
        // instead of each product waiting for its own (two tiles have no
        // registers for that).
        constexpr bool PRE = NVT == 1;
        // the output phase keeps the bf16/fp32 copy of the old state alive
        // beside its fragments: with fp32 operands and eight waves a
        // workgroup (256 registers) they are read as they are used instead
        constexpr bool PRE_O = PRE && !(C::LW && sizeof(T) == 4 && NKC * NTT > 8);
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
        if constexpr (C::MIX) {
            barrier_keep_loads();                  // every wave is done with T and v of chunk c
            if (c + 1 < nch) stage_tv(c + 1);
        }
        if constexpr (C::NBUF == 2 && !C::LW && !C::AUG) stage(cn, nb, J_0{}, J_H{});
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
            if constexpr (!C::LW && !C::AUG) stage(cn, nb, J_H{}, J_E{});
            if constexpr (!C::LW) load_uz(cn);
        }
        if constexpr (!C::AUG) {
            // prefix-cache checkpoint: the state after this chunk
            if (ckpt && (ck0 + c + 1) % ck_every == 0 && (int64_t)(ck0 + c + 1) * CH <= len_chain) {
                const int64_t row = ck_base + (ck0 + c + 1) / ck_every - 1;
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
            if constexpr (PRE_O) {
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
                        *reinterpret_cast<T4*>(smem + C::O_Y + zy_off(ta, vt)) = from_f32x4<T>(o);
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

    // ---- final state, or the carry to the next slab ----------------------------
    float* sout = nullptr;
    if (!to_end) sout = p.carry + ((int64_t)n * H + h) * DK * (int64_t)dvt;
    else if (p.sfin && n >= p.final_seq_lo) sout = p.sfin + ((int64_t)(n - p.final_seq_lo) * H + h) * DK * (int64_t)dvt;
    if (sout) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) {
                const int col = colw + 16 * vt + l16;
#pragma unroll
                for (int i = 0; i < 4; ++i) sout[(int64_t)(16 * ct + 4 * g4 + i) * dvt + col] = S[ct][vt][i];
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
    p.slab_lo = (int)a.slab_lo;
    p.slab_hi = (int)a.slab_hi;
    p.rect_w = a.rect_w;
    p.rect_c0 = a.rect_c0;
    p.rect_s0 = a.rect_s0;
    p.rect_s1 = a.rect_s1;
    p.first_slab = a.rect_w > 0 ? a.rect_c0 == 0 : a.slab_lo == 0;
    p.carry = a.carry;
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
    p.v = a.v;
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
        const hipError_t e = ensure_lds_limit((const void*)kern, (int)C::BYTES);
        if (e != hipSuccess) return e;
    }
    const long nblk = (long)((p.nchains + 7) / 8) * 8 * p.nvg;
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(C::NTHR), C::BYTES, (hipStream_t)a.stream, p);
    return hipGetLastError();
}

// The configuration a call runs with, handed to f as a value of its type.
// One value tile per wave wherever loader waves apply, whatever the number of
// chains (on the 16-sequence varlen layer 2.84 ms against 3.04 with two
// tiles); the transition pairs, with dk + dv columns a chain, keep the choice
// made from the chain count (two tiles: 0.74 ms against 1.07 for 1024
// chains), at bf16 and dk = 128 with all 256 columns of a chain in one
// workgroup of eight compute waves.
template <class E, int DK, int CH, int MODE, class F>
static auto with_state_nvt(const TwoPassArgs& a, F&& f) {
    using C1 = StCfg<E, DK, DK, CH, 1, MODE>;
    if (a.nvt == 1 || (C1::LW && MODE != kModePairs)) return f(C1{});
    if constexpr (MODE == kModePairs && DK == 128 && sizeof(typename E::T) == 2)
        return f(StCfg<E, DK, DK, CH, 2, MODE, kPairsWaves>{});
    else
        return f(StCfg<E, DK, DK, CH, 2, MODE>{});
}

template <class E, int DK, int CH, class F>
static auto with_state_mode(const TwoPassArgs& a, F&& f) {
    switch (a.mode) {
        case kModeSeq: return with_state_nvt<E, DK, CH, kModeSeq>(a, f);
        case kModeVarlen: return with_state_nvt<E, DK, CH, kModeVarlen>(a, f);
        case kModePairs: return with_state_nvt<E, DK, CH, kModePairs>(a, f);
        default: return with_state_nvt<E, DK, CH, kModeFinish>(a, f);
    }
}

template <class E, int DK, class F>
static auto with_state_dk(const TwoPassArgs& a, F&& f) {
    if (a.chunk == 64) return with_state_mode<E, DK, 64>(a, f);
    if (a.chunk == 32) return with_state_mode<E, DK, 32>(a, f);
    return with_state_mode<E, DK, 16>(a, f);
}

template <class F>
static auto with_state_cfg(const TwoPassArgs& a, F&& f) {
    if (a.dtype == 0) return a.dk == 128 ? with_state_dk<BF16, 128>(a, f) : with_state_dk<BF16, 64>(a, f);
    return a.dk == 128 ? with_state_dk<F32, 128>(a, f) : with_state_dk<F32, 64>(a, f);
}

hipError_t launch_chunk_state(const TwoPassArgs& a, const int32_t* chunk_off, const int32_t* order) {
    return with_state_cfg(a, [&](auto c) { return launch_state_cfg<decltype(c)>(a, chunk_off, order); });
}

void state_geometry(const TwoPassArgs& a, int* wg_per_chain, int* wg_per_cu) {
    with_state_cfg(a, [&](auto c) {
        using C = decltype(c);
        const int cols = C::AUG ? a.dk + a.dv : a.dv;
        *wg_per_chain = cols / C::CW > 0 ? cols / C::CW : 1;
        // eight waves a CU at the scan's register count, and the LDS
        const int by_waves = 8 / (C::NW + C::NLW), by_lds = (int)((160 * 1024) / C::BYTES);
        *wg_per_cu = by_waves < by_lds ? (by_waves > 0 ? by_waves : 1) : (by_lds > 0 ? by_lds : 1);
        return 0;
    });
}

hipError_t launch_varlen_plan(int num_seqs, const int32_t* cu_seqlens, int64_t T_total, int chunk,
                              int ckpt_interval, int32_t* chunk_off, int32_t* order, int32_t* ckpt_off,
                              void* stream) {
    hipLaunchKernelGGL(varlen_plan_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, num_seqs, cu_seqlens,
                       T_total, chunk, ckpt_interval, chunk_off, order, ckpt_off);
    return hipGetLastError();
}

}  // namespace kda
