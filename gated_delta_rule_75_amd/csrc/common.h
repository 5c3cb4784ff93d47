// Device helpers shared by the libkda kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Element types.  Global tensors q, k, v, z, y are bf16 or fp32.  MFMA operand
// tiles in LDS use the same element type: bf16 feeds v_mfma_f32_16x16x32_bf16
// (8 consecutive k per lane), fp32 feeds v_mfma_f32_16x16x4_f32 (1 k per lane).
// Both produce the 16x16 fp32 tile in the same lane layout: lane l holds rows
// 4*(l/16)+i, i<4, of column l%16.
// ---------------------------------------------------------------------------
struct BF16 {
    using T = __bf16;
    using Frag = bf16x8_t;
    static constexpr int KPL = 8;         // k elements per lane per MFMA
    static constexpr int KSTEP = 32;      // k depth of one MFMA
    static __device__ __forceinline__ f32x4_t mma(Frag a, Frag b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

struct F32 {
    using T = float;
    using Frag = float;
    static constexpr int KPL = 1;
    static constexpr int KSTEP = 4;
    static __device__ __forceinline__ f32x4_t mma(Frag a, Frag b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// Fragment element access (k index within the lane's KPL elements).
template <typename E>
__device__ __forceinline__ float frag_get(const typename E::Frag& f, int i);
template <>
__device__ __forceinline__ float frag_get<BF16>(const bf16x8_t& f, int i) { return (float)f[i]; }
template <>
__device__ __forceinline__ float frag_get<F32>(const float& f, int) { return f; }

template <typename E>
__device__ __forceinline__ void frag_set(typename E::Frag& f, int i, float x);
template <>
__device__ __forceinline__ void frag_set<BF16>(bf16x8_t& f, int i, float x) { f[i] = (__bf16)x; }
template <>
__device__ __forceinline__ void frag_set<F32>(float& f, int, float x) { f = x; }

// Operand fragment of a 16 x KSTEP tile stored row-major in LDS with pitch ld
// (elements): rows r0 .. r0+15, k columns k0 .. k0+KSTEP-1.  Used for both A
// (rows = output rows) and B (rows = output columns, i.e. B stored transposed).
template <typename E>
__device__ __forceinline__ typename E::Frag lds_frag(const typename E::T* base, int ld, int r0,
                                                     int k0, int lane) {
    const typename E::T* p = base + (r0 + (lane & 15)) * ld + k0 + E::KPL * (lane >> 4);
    return *reinterpret_cast<const typename E::Frag*>(p);
}

// Fragment of a reduction shorter than one MFMA (klim < KSTEP, klim a
// multiple of KPL): lanes whose k range starts at or past klim supply zeros.
template <typename E, int KLIM>
__device__ __forceinline__ typename E::Frag lds_frag_lim(const typename E::T* base, int ld, int r0,
                                                         int k0, int lane) {
    if constexpr (KLIM % E::KSTEP == 0) return lds_frag<E>(base, ld, r0, k0, lane);
    typename E::Frag f;
    if (k0 + E::KPL * (lane >> 4) < KLIM) {
        f = lds_frag<E>(base, ld, r0, k0, lane);
    } else {
#pragma unroll
        for (int i = 0; i < E::KPL; ++i) frag_set<E>(f, i, 0.f);
    }
    return f;
}

// Same fragment with every element multiplied by a per-k factor table (fp32,
// indexed by absolute k).
template <typename E>
__device__ __forceinline__ typename E::Frag lds_frag_scaled(const typename E::T* base, int ld,
                                                            int r0, int k0, int lane,
                                                            const float* kscale) {
    typename E::Frag f = lds_frag<E>(base, ld, r0, k0, lane);
    const int kb = k0 + E::KPL * (lane >> 4);
#pragma unroll
    for (int i = 0; i < E::KPL; ++i) frag_set<E>(f, i, frag_get<E>(f, i) * kscale[kb + i]);
    return f;
}

// Global element loads/stores of bf16 / fp32 tensors.
__device__ __forceinline__ float gload(const __bf16* p) { return (float)*p; }
__device__ __forceinline__ float gload(const float* p) { return *p; }
__device__ __forceinline__ void gstore(__bf16* p, float x) { *p = (__bf16)x; }
__device__ __forceinline__ void gstore(float* p, float x) { *p = x; }

// Two consecutive elements (4-byte aligned for bf16, 8-byte for fp32).
__device__ __forceinline__ f32x2_t gload2(const __bf16* p) {
    bf16x2_t v = *reinterpret_cast<const bf16x2_t*>(p);
    return f32x2_t{(float)v[0], (float)v[1]};
}
__device__ __forceinline__ f32x2_t gload2(const float* p) {
    return *reinterpret_cast<const f32x2_t*>(p);
}

__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }
// 2^x in one v_exp_f32
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float sigmoid(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// 16 bytes per lane from global memory straight into LDS: lane i writes
// lds + 16 i.  (A __device__ wrapper: the builtin written directly in a
// kernel template hides the kernel from the host compilation pass.)
__device__ __forceinline__ void lds_dma16(const void* src, void* lds) {
    __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

// s_waitcnt vmcnt(n) (n < 64), other counters left alone
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that leaves global loads and stores in flight.
// __syncthreads() waits for every outstanding vector-memory operation (its
// fence covers global stores and direct-to-LDS copies too); kernels whose
// waves share data only through LDS need just their LDS operations finished.
// Pending LDS reads finish first, so no wave still reads a buffer that
// another wave overwrites after the barrier; the empty asm statements keep
// the compiler from moving memory accesses across it.  A caller that needs a
// global-to-LDS copy to have landed waits for it (s_waitcnt vmcnt) first.
__device__ __forceinline__ void barrier_keep_loads() {
    // no instruction is scheduled across it either (work placed after a
    // barrier in the source stays after it, and the reverse)
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Sum over each row of 16 consecutive lanes, the total in every lane of the
// row: DPP quad permutations [1,0,3,2] and [2,3,0,1] for lane distances 1
// and 2, then the half-row and row mirrors for 4 and 8.  Four VALU adds and
// no LDS traffic (a __shfl_xor is an LDS permute); every lane adds the same
// pairs in the same order, so all of them hold the same bits.  Each pattern
// reads a lane of the same row, so the zero fill for out-of-range lanes never
// applies; requesting it lets the compiler fold the move into the add
// (v_add_f32_dpp).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
    x += dpp_mov<0x141>(x);   // row_half_mirror
    x += dpp_mov<0x140>(x);   // row_mirror
    return x;
}

// Fused input step: unit q and k as x / sqrt(sum x^2 + kNormEps), the
// log-decay g = kGMin * sigmoid(a) in (kGMin, 0), beta = sigmoid(b).
constexpr float kGMin = -5.0f;
constexpr float kNormEps = 1e-6f;
__device__ __forceinline__ float decay_gate(float a) { return kGMin * sigmoid(a); }

}  // namespace kda
