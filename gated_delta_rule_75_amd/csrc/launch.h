// Host-side launch descriptors shared by the C ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

struct DecodeArgs {
    int dtype;  // 0 bf16, 1 fp32
    int N, H, dk, dv;
    float scale;
    const void *q, *k, *v;
    const float *g, *beta;
    const void* z;
    float* state;
    void* y;
    void* stream;
};

struct PrefillArgs {
    int dtype;  // 0 bf16, 1 fp32
    int H, dk, dv, chunk;
    float scale;
    int num_seqs;
    int64_t T_total;
    const int32_t* cu_seqlens;  // device offsets, or NULL: sequence n spans
    int64_t seg_len;            //   [n*seg_len, min((n+1)*seg_len, T_total))
    const void *q, *k, *v;
    const float *g, *beta;
    const void* z;
    const float* initial_state;  // [num_seqs, H, dk, dv] or NULL
    float* final_state;          // see final_seq_lo and mode 2
    int final_seq_lo;            // only sequences n >= final_seq_lo write final_state[n - lo]
    void* y;                     // NULL only in mode 2
    int mode;                    // 0 one sequence / equal segments, 1 varlen (cu_seqlens),
                                 // 2 KCP pairs: value width dk + dv, identity start on the first
                                 //   dk columns, final_state gets [num_seqs, H, dk, dk + dv],
                                 // 3 KCP segment outputs
    int vs;                      // value-slice width per workgroup (0 = library choice)
    void* stream;
};

bool prefill_supported(int dtype, int dk, int dv, int chunk);
hipError_t launch_prefill(const PrefillArgs& a);
hipError_t launch_decode(const DecodeArgs& a);

// KCP phase 2: starts[s] = M_{s-1} starts[s-1] + Sloc_{s-1}, starts[0] = S0.
hipError_t launch_kcp_scan(int H, int dk, int dv, int nseg, const float* pairs,
                           const float* initial_state, float* starts, float* final_state,
                           hipStream_t stream);

}  // namespace kda
