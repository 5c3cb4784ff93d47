// C ABI of libkda: argument validation, workspace sizing and dispatch to the
// HIP kernels.  Every check runs before anything is enqueued.
#include "../../include/kda.h"

#include <hip/hip_runtime.h>

#include "launch.h"

namespace {

constexpr int kVersion = 1 * 10000 + 0 * 100 + 0;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elt_align(kda_dtype dt) { return dt == KDA_BF16 ? 4 : 8; }

bool head_shape_ok(int dk, int dv) { return (dk == 64 && dv == 64) || (dk == 128 && dv == 128); }

kda_status from_hip(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Byte sizes of the KCP workspace parts.
void kcp_parts(int H, int dk, int dv, int nseg, size_t* pairs, size_t* starts) {
    *pairs = round_up((size_t)nseg * H * dk * (size_t)(dk + dv) * sizeof(float), 256);
    *starts = round_up((size_t)nseg * H * dk * (size_t)dv * sizeof(float), 256);
}

}  // namespace

extern "C" {

int kda_version(void) { return kVersion; }

const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
        case KDA_ERR_WORKSPACE_TOO_SMALL: return "KDA_ERR_WORKSPACE_TOO_SMALL";
        case KDA_ERR_HIP: return "KDA_ERR_HIP";
    }
    return "KDA_ERR_UNKNOWN";
}

kda_status kda_chunk_fwd(kda_dtype dt, int H, int dk, int dv, int chunk, float scale,
                         int num_seqs, int64_t T_total, const int32_t* cu_seqlens,
                         const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const void* z, const float* initial_state,
                         float* final_state, void* y, void* stream) {
    if (dt != KDA_BF16 && dt != KDA_F32) return KDA_ERR_INVALID_ARGUMENT;
    if (H <= 0 || num_seqs <= 0 || T_total < 0) return KDA_ERR_INVALID_ARGUMENT;
    if (!cu_seqlens && num_seqs != 1) return KDA_ERR_INVALID_ARGUMENT;
    if ((int64_t)num_seqs * H > (int64_t)1 << 28) return KDA_ERR_INVALID_ARGUMENT;
    if (!head_shape_ok(dk, dv)) return KDA_ERR_UNSUPPORTED;
    if (!kda::prefill_supported((int)dt, dk, dv, chunk)) return KDA_ERR_UNSUPPORTED;
    if (T_total > 0 && (!q || !k || !v || !g || !beta || !y)) return KDA_ERR_INVALID_ARGUMENT;
    const size_t ea = elt_align(dt);
    if (!aligned(q, ea) || !aligned(k, ea) || !aligned(v, ea) || !aligned(z, ea) ||
        !aligned(y, ea) || !aligned(g, 8) || !aligned(beta, 4) || !aligned(cu_seqlens, 4) ||
        !aligned(initial_state, 16) || !aligned(final_state, 16))
        return KDA_ERR_INVALID_ARGUMENT;
    kda::PrefillArgs a{};
    a.dtype = (int)dt;
    a.H = H;
    a.dk = dk;
    a.dv = dv;
    a.chunk = chunk;
    a.scale = scale;
    a.num_seqs = num_seqs;
    a.T_total = T_total;
    a.cu_seqlens = cu_seqlens;
    a.seg_len = T_total;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.z = z;
    a.initial_state = initial_state;
    a.final_state = final_state;
    a.final_seq_lo = 0;
    a.y = y;
    a.mode = cu_seqlens ? 1 : 0;
    a.vs = 0;
    a.stream = stream;
    return from_hip(kda::launch_prefill(a));
}

size_t kda_kcp_workspace_size(int H, int dk, int dv, int num_segments) {
    if (H <= 0 || num_segments <= 0 || !head_shape_ok(dk, dv)) return 0;
    size_t pairs, starts;
    kcp_parts(H, dk, dv, num_segments, &pairs, &starts);
    return pairs + starts;
}

kda_status kda_kcp_scan(kda_dtype dt, int H, int dk, int dv, int chunk, float scale, int64_t T,
                        int num_segments, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, const void* z,
                        const float* initial_state, float* final_state, void* y,
                        void* workspace, size_t workspace_bytes, void* stream) {
    if (dt != KDA_BF16 && dt != KDA_F32) return KDA_ERR_INVALID_ARGUMENT;
    if (H <= 0 || num_segments <= 0 || T < num_segments) return KDA_ERR_INVALID_ARGUMENT;
    if (!head_shape_ok(dk, dv)) return KDA_ERR_UNSUPPORTED;
    if (!kda::prefill_supported((int)dt, dk, dv, chunk)) return KDA_ERR_UNSUPPORTED;
    if (!q || !k || !v || !g || !beta || !y || !workspace) return KDA_ERR_INVALID_ARGUMENT;
    const size_t ea = elt_align(dt);
    if (!aligned(q, ea) || !aligned(k, ea) || !aligned(v, ea) || !aligned(z, ea) ||
        !aligned(y, ea) || !aligned(g, 8) || !aligned(beta, 4) || !aligned(workspace, 256) ||
        !aligned(initial_state, 16) || !aligned(final_state, 16))
        return KDA_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < kda_kcp_workspace_size(H, dk, dv, num_segments))
        return KDA_ERR_WORKSPACE_TOO_SMALL;
    size_t pbytes, sbytes;
    kcp_parts(H, dk, dv, num_segments, &pbytes, &sbytes);
    float* pairs = static_cast<float*>(workspace);
    float* starts = reinterpret_cast<float*>(static_cast<char*>(workspace) + pbytes);
    const int64_t seg_len = (T + num_segments - 1) / num_segments;
    // segments hold seg_len tokens each; with T not a multiple, trailing ones may be empty
    kda::PrefillArgs a{};
    a.dtype = (int)dt;
    a.H = H;
    a.dk = dk;
    a.dv = dv;
    a.chunk = chunk;
    a.scale = scale;
    a.num_seqs = num_segments;
    a.T_total = T;
    a.cu_seqlens = nullptr;
    a.seg_len = seg_len;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.z = z;
    a.stream = stream;
    a.vs = 0;
    // phase 1: (M, Sloc) of every segment, as the state that the augmented value
    // block [0 | v] builds from the augmented start [I | 0]
    a.mode = 2;
    a.initial_state = nullptr;
    a.final_state = pairs;
    a.final_seq_lo = 0;
    a.y = nullptr;
    hipError_t e = kda::launch_prefill(a);
    if (e != hipSuccess) return KDA_ERR_HIP;
    // phase 2: entering state of every segment
    e = kda::launch_kcp_scan(H, dk, dv, num_segments, pairs, initial_state, starts, final_state,
                             (hipStream_t)stream);
    if (e != hipSuccess) return KDA_ERR_HIP;
    // phase 3: outputs of every segment from its entering state; the last
    // segment's final state is the sequence's final state
    a.mode = 3;
    a.initial_state = starts;
    a.final_state = final_state;
    a.final_seq_lo = num_segments - 1;
    a.y = y;
    return from_hip(kda::launch_prefill(a));
}

kda_status kda_decode_step(kda_dtype dt, int N, int H, int dk, int dv, float scale,
                           const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const void* z, float* state, void* y,
                           void* stream) {
    if (dt != KDA_BF16 && dt != KDA_F32) return KDA_ERR_INVALID_ARGUMENT;
    if (N < 0 || H <= 0) return KDA_ERR_INVALID_ARGUMENT;
    if ((int64_t)N * H > (int64_t)1 << 30) return KDA_ERR_INVALID_ARGUMENT;
    if (!head_shape_ok(dk, dv)) return KDA_ERR_UNSUPPORTED;
    if (N > 0 && (!q || !k || !v || !g || !beta || !state || !y)) return KDA_ERR_INVALID_ARGUMENT;
    const size_t ea = elt_align(dt);
    if (!aligned(q, ea) || !aligned(k, ea) || !aligned(v, ea) || !aligned(z, ea) ||
        !aligned(y, ea) || !aligned(g, 8) || !aligned(beta, 4) || !aligned(state, 16))
        return KDA_ERR_INVALID_ARGUMENT;
    kda::DecodeArgs a{};
    a.dtype = (int)dt;
    a.N = N;
    a.H = H;
    a.dk = dk;
    a.dv = dv;
    a.scale = scale;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.z = z;
    a.state = state;
    a.y = y;
    a.stream = stream;
    return from_hip(kda::launch_decode(a));
}

}  // extern "C"
