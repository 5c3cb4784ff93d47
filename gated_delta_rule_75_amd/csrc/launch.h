// Host-side launch descriptors shared by the C ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "twopass.h"

namespace kda {

struct DecodeArgs {
    int dtype;  // 0 bf16, 1 fp32
    int N, H, dk, dv;
    float scale;
    const void *q, *k, *v;
    const void *g, *beta;  // fp32 g, beta; fused: pre-activations a, b in the storage dtype
    bool fused;            // raw q, k (normalised in the kernel) and gate pre-activations
    const void* z;
    float* state;
    void* y;
    void* stream;
};

// Modes of the state scan.  Distinct instantiations keep the profiler
// statistics of the different call sites apart.
enum ScanMode : int {
    kModeSeq = 0,     // one sequence, or equal segments (no offsets array)
    kModeVarlen = 1,  // packed sequences given by cu_seqlens
    kModePairs = 2,   // KCP segment pairs: augmented state [I | 0], values [0 | v], no outputs
    kModeFinish = 3,  // KCP outputs of every segment from its entering state
};

struct TwoPassArgs {
    int dtype;  // 0 bf16, 1 fp32
    int H, dk, dv, chunk;
    float scale;
    int num_seqs;
    int64_t T_total;
    const int32_t* cu_seqlens;  // device offsets, or NULL: sequence n spans
    int64_t seg_len;            //   [n*seg_len, min((n+1)*seg_len, T_total))
    const void *q, *k, *v;
    const void *g, *beta;        // fp32 g, beta; fused: pre-activations a, b in the storage dtype
    bool fused;                  // raw q, k (normalised in the kernel) and gate pre-activations
    bool pairs_only;             // preparation: only the products the KCP pairs read (no Qt, P)
    const void* z;
    const float* initial_state;  // [num_seqs, H, dk, dv] or NULL
    float* final_state;          // see final_seq_lo; mode 2: [num_seqs, H, dk, dk + dv]
    int final_seq_lo;            // only sequences n >= final_seq_lo write final_state[n - lo]
    void* y;                     // NULL only in mode 2
    int mode;                    // ScanMode
    int nvt;                     // 16-column value tiles per scan wave (1 or 2)
    TwoPassBufs bufs;            // chunk products (workspace)
    int64_t chunk_cap;           // bound on the global chunk count of the call
    // Time slab: the workspace arrays hold the products of global chunks
    // [slab_lo, slab_hi) only.  A chain then runs just its chunks inside the
    // slab: from its initial state when the slab holds its first chunk, else
    // from carry[n]; into its final state when the slab holds its last chunk,
    // else into carry[n].  Chains with no chunks at all run in the first slab.
    // One slab [0, chunk_cap) with no carry covers the whole call.
    int64_t slab_lo, slab_hi;
    // Rectangular slab (equal segments only, cu_seqlens NULL; rect_w > 0):
    // chunks [rect_c0, rect_c0 + rect_w) of segments [rect_s0, rect_s1), in
    // workspace block ((n - rect_s0) rect_w + c - rect_c0) H + h; slab_lo and
    // slab_hi are then unused.  Empty segments run in the part with rect_c0 = 0.
    int rect_w, rect_c0, rect_s0, rect_s1;
    float* carry;                // [num_seqs, H, dk, dv] (mode 2: dk + dv columns), or NULL
    // prefix-cache checkpoints (modes 0 and 1): the state after every
    // ckpt_every chunks of a sequence, at row ckpt_off[n] + j of ckpt
    float* ckpt;                 // [capacity, H, dk, dv] or NULL
    const int32_t* ckpt_off;     // device [num_seqs + 1]
    int ckpt_every;
    int64_t ckpt_cap;
    void* stream;
};

bool prefill_supported(int dtype, int dk, int dv, int chunk);

// Raise a kernel's dynamic-LDS limit to `bytes`, once per (device, kernel):
// later calls on the same device return at once.
hipError_t ensure_lds_limit(const void* kern, int bytes);
// Compute units of the current device, queried once per device.
hipError_t device_cu_count(int* cus);

// Per-sequence plan, each output optional: chunk offsets ([num_seqs + 1]),
// a longest-first order ([num_seqs]) and checkpoint offsets ([num_seqs + 1],
// floor(len / ckpt_interval) rows per sequence).  cu_seqlens NULL means one
// sequence of T_total tokens.
hipError_t launch_varlen_plan(int num_seqs, const int32_t* cu_seqlens, int64_t T_total, int chunk,
                              int ckpt_interval, int32_t* chunk_off, int32_t* order, int32_t* ckpt_off,
                              void* stream);
// Products of every (chunk, head) into a.bufs; nchunks bounds the chunk count
// (chunk_off, when given, holds the exact offsets).
hipError_t launch_chunk_prep(const TwoPassArgs& a, const int32_t* chunk_off, int64_t nchunks);
// The sequential pass over the chunks of every (sequence, head).
hipError_t launch_chunk_state(const TwoPassArgs& a, const int32_t* chunk_off, const int32_t* order);
// Workgroups a chain of the state scan takes, and how many of them fit on a
// CU at once, for the configuration launch_chunk_state picks for `a`.
void state_geometry(const TwoPassArgs& a, int* wg_per_chain, int* wg_per_cu);
// compute waves of a KCP pairs workgroup at bf16, dk = 128: all dk + dv
// columns of a chain in one workgroup
constexpr int kPairsWaves = 8;

hipError_t launch_decode(const DecodeArgs& a);
// Td draft tokens per request (inputs [N, Td, H, d]) against the resident
// states: outputs of all of them (a.y, optional) and the state after the first
// accepted[n] written back (accepted optional).
hipError_t launch_replay(const DecodeArgs& a, int Td, const int32_t* accepted);

// KCP phase 2: starts[s] = M_{s-1} starts[s-1] + Sloc_{s-1}, starts[0] = S0,
// through kcp_group_len(nseg)-segment groups: group_pairs [G][H][dk][dk+dv]
// and group_starts [G][H][dk][dv] are scratch (G = ceil(nseg / L)).
int kcp_group_len(int nseg);
hipError_t launch_kcp_scan(int H, int dk, int dv, int nseg, const float* pairs,
                           const float* initial_state, float* starts, float* group_pairs,
                           float* group_starts, hipStream_t stream);

}  // namespace kda
