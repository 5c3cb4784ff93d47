// Two-pass chunked form of the KDA recurrence: shared definitions of the
// chunk-preparation kernel (chunk_prep.hip) and the state-scan kernel
// (chunk_state.hip).
//
// Unrolling a chunk of C tokens that starts from state S (recurrence of page
// "Exercices", Niveau 2 Q7; the pages cite the blocked "UT transform" form
// without printing it, so it is derived here), with G_t the in-chunk running
// sum of g and A_tj = sum_c k_tc k_jc e^{G_tc - G_jc} (j < t):
//     Delta = U - W S                       W = Tb (K e^G)
//     O     = Qt S + Pm Delta               U = Tb V
//     S    <- gam * S + Kh^T Delta          Tb = L^{-1} diag(beta), L = I + diag(beta) A
// with Qt = scale Q e^G, Pm_tj = scale sum_c q_tc k_jc e^{G_tc - G_jc} (j <= t),
// Kh = K e^{G_C - G} and gam = e^{G_C}.  Everything except the three
// S-products depends on the chunk alone, so the preparation kernel forms it
// for every (chunk, head) at once, and the scan kernel carries the state
// through the chunks of a sequence with three small products per chunk.
// U = Tb V is left to the scan kernel, off the state's path: it needs only
// the C x C triangle Tb beside v itself, so the preparation kernel neither
// reads v nor writes a C x dv product per chunk.
//
// Workspace arrays, one block per (chunk, head), chunk-major ("chunk" is the
// global chunk index over all sequences):
//   Wn   -W      [C x dk]    rows t, reduction over channels
//   Qt           [C x dk]    rows t, reduction over channels
//   KhT  Kh^T    [dk x CP]   rows c, reduction over tokens
//   Pm           [C x CP]    rows t, reduction over tokens j (zero for j > t);
//                            only the fragments on or below the diagonal
//   Tb           [C x CP]    rows t, reduction over tokens j (zero for j > t);
//                            the same fragments as Pm, k in natural order
//   gam          [dk] fp32
// CP is C rounded up to a whole k-block (tokens past C are zero).  The
// operand matrices are stored as MFMA fragments: a fragment is 16 rows x one
// k-block, 64 lanes x 16 bytes in lane order, lane l = (row % 16) + 16 * slot
// holding the k-block positions [slot * KB/4, (slot + 1) * KB/4) of its row
// (positions in the k-block order below).  A fragment is then one contiguous
// 1 KiB read, and the lanes of a wave read it with one 16-byte access each.
// Tb's fragments keep the natural k order (lane group g holds k-block
// positions g KB/4 ..): both operands of U = Tb V come from memory, so no
// accumulator order constrains them.
//
// k-block order.  The scan kernel keeps S and Delta in MFMA accumulator tiles,
// where lane l holds rows 4*(l/16)+i (i < 4) of column l%16, and feeds them
// back as MFMA operands without moving data between lanes.  A reduction is
// free to visit its k indices in any order as long as both operands agree, so
// an operand fragment is built from the lane's own accumulator values: for
// bf16 (v_mfma_f32_16x16x32_bf16, 8 k values per lane) slot j < 4 of lane
// group g is row 4g+j of the first 16-row tile and slot j >= 4 row 4g+j-4 of
// the second, i.e. logical index l of a 32-wide k-block sits at position
// 8*((l%16)/4) + 4*(l/16) + l%4.  The preparation kernel stores the
// memory-side operands in that order, so each lane fetches its 8 values with
// one 16-byte load.  fp32 (v_mfma_f32_16x16x4f32, 1 k value per lane) issues
// four MFMAs per 16-wide k-block, MFMA i taking row 4g+i, which is the
// natural order.
#pragma once

#include "common.h"

namespace kda {

template <typename E> struct KBlk;

template <> struct KBlk<BF16> {
    using T = __bf16;
    using Frag = bf16x8_t;
    static constexpr int KB = 32;   // k indices per block
    static constexpr int TPB = 2;   // accumulator tiles per block
    static __device__ __forceinline__ int pos(int l) {
        return 8 * ((l & 15) >> 2) + 4 * ((l >> 4) & 1) + (l & 3) + (l & ~31);
    }
    static __device__ __forceinline__ f32x4_t mma(Frag a, Frag b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ Frag from_acc(f32x4_t lo, f32x4_t hi) {
        Frag f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[i] = (__bf16)lo[i];
            f[4 + i] = (__bf16)hi[i];
        }
        return f;
    }
    static __device__ __forceinline__ Frag zero() {
        Frag f;
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (__bf16)0.f;
        return f;
    }
    static __device__ __forceinline__ void set(Frag& f, int e, T x) { f[e] = x; }
};

template <> struct KBlk<F32> {
    using T = float;
    using Frag = f32x4_t;
    static constexpr int KB = 16;
    static constexpr int TPB = 1;
    static __device__ __forceinline__ int pos(int l) { return l; }
    static __device__ __forceinline__ f32x4_t mma(Frag a, Frag b, f32x4_t c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
        return c;
    }
    static __device__ __forceinline__ Frag from_acc(f32x4_t lo, f32x4_t) { return lo; }
    static __device__ __forceinline__ Frag zero() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }
    static __device__ __forceinline__ void set(Frag& f, int e, T x) { f[e] = x; }
};

// Element offset, inside one array block, of element (row, k) of an operand
// matrix stored as fragments; fidx is the fragment of (row / 16, k / KB).
template <class K>
__device__ __forceinline__ int frag_elem(int fidx, int row, int k) {
    constexpr int KPL = K::KB / 4;
    const int p = K::pos(k % K::KB);
    return fidx * 64 * KPL + ((row & 15) + 16 * (p / KPL)) * KPL + p % KPL;
}

// Fragments of Pm, on or below the diagonal: (token tile ta, k-block u) with
// u * KB <= 16 ta + 15, numbered in (ta, u) order.
__host__ __device__ constexpr int pm_frags(int ntt, int nkt, int kb) {
    int n = 0;
    for (int ta = 0; ta < ntt; ++ta)
        for (int u = 0; u < nkt; ++u) n += (u * kb <= 16 * ta + 15) ? 1 : 0;
    return n;
}
__host__ __device__ constexpr int pm_frag_index(int ta, int u, int nkt, int kb) {
    int n = 0;
    for (int a = 0; a < ta; ++a)
        for (int v = 0; v < nkt; ++v) n += (v * kb <= 16 * a + 15) ? 1 : 0;
    return n + u;
}

// Host-side sizes of the workspace arrays (elements per (chunk, head) block).
struct TwoPassDims {
    int dk, dv, C, CP;
    size_t esz;  // bytes per element of the operand arrays
    size_t wn() const { return (size_t)C * dk; }
    size_t qt() const { return (size_t)C * dk; }
    size_t kht() const { return (size_t)dk * CP; }
    size_t pm() const { return (size_t)pm_frags(C / 16, CP / (esz == 2 ? 32 : 16), esz == 2 ? 32 : 16) * 64 *
                               (esz == 2 ? 8 : 4); }
    size_t tt() const { return pm(); }
    size_t gam() const { return (size_t)dk; }
    // bytes of one (chunk, head) block over all arrays
    size_t block_bytes() const { return (wn() + qt() + kht() + pm() + tt()) * esz + gam() * 4; }
};

inline TwoPassDims twopass_dims(int dtype, int dk, int dv, int chunk) {
    const int kb = dtype == 0 ? 32 : 16;
    TwoPassDims d;
    d.dk = dk;
    d.dv = dv;
    d.C = chunk;
    d.CP = (chunk + kb - 1) / kb * kb;
    d.esz = dtype == 0 ? 2 : 4;
    return d;
}

// Device pointers of the workspace arrays.
struct TwoPassBufs {
    void *wn, *qt, *kht, *pm, *tt;
    float* gam;
};

}  // namespace kda
