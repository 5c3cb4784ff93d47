// C ABI of libkda: argument validation, workspace sizing and dispatch to the
// HIP kernels.  Every check runs before anything is enqueued.
#include "../../include/kda.h"

#include <hip/hip_runtime.h>

#include <mutex>
#include <set>
#include <utility>

#include "launch.h"

namespace {

constexpr int kVersion = 1 * 10000 + 1 * 100 + 0;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elt_align(kda_dtype dt) { return dt == KDA_BF16 ? 4 : 8; }

// The prefill kernels move q, k, v, z, y in runs of four elements.
size_t vec_align(kda_dtype dt) { return dt == KDA_BF16 ? 8 : 16; }

bool head_shape_ok(int dk, int dv) { return (dk == 64 && dv == 64) || (dk == 128 && dv == 128); }

kda_status from_hip(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace of the two-pass prefill: sequence plan, the carry of the state
// between time slabs (bounded workspaces only), then the per-(chunk, head)
// product arrays of one slab of nchunks chunks, each part 256-byte aligned.
struct Layout {
    size_t chunk_off, order, carry, wn, qt, kht, pm, tt, gam, total;
};

Layout twopass_layout(kda_dtype dt, int H, int dk, int dv, int chunk, int num_seqs, int64_t nchunks,
                      size_t carry_bytes = 0) {
    const kda::TwoPassDims d = kda::twopass_dims((int)dt, dk, dv, chunk);
    const size_t nb = (size_t)nchunks * H;
    Layout l;
    size_t o = 0;
    auto take = [&](size_t bytes) { const size_t at = o; o += round_up(bytes, 256); return at; };
    l.chunk_off = take((size_t)(num_seqs + 1) * 4);
    l.order = take((size_t)num_seqs * 4);
    l.carry = take(carry_bytes);
    l.wn = take(nb * d.wn() * d.esz);
    l.qt = take(nb * d.qt() * d.esz);
    l.kht = take(nb * d.kht() * d.esz);
    l.pm = take(nb * d.pm() * d.esz);
    l.tt = take(nb * d.tt() * d.esz);
    l.gam = take(nb * d.gam() * 4);
    l.total = o;
    return l;
}

// Chunks per slab that fit `bytes` with the given carry, at most `all` (0 when
// not even one chunk fits).
int64_t slab_chunks(kda_dtype dt, int H, int dk, int dv, int chunk, int num_seqs, int64_t all,
                    size_t carry_bytes, size_t bytes) {
    const size_t fixed = twopass_layout(dt, H, dk, dv, chunk, num_seqs, 0, carry_bytes).total;
    if (bytes <= fixed) return 0;
    const size_t per = kda::twopass_dims((int)dt, dk, dv, chunk).block_bytes() * (size_t)H;
    int64_t n = (int64_t)((bytes - fixed) / per);
    if (n > all) n = all;
    while (n > 0 && twopass_layout(dt, H, dk, dv, chunk, num_seqs, n, carry_bytes).total > bytes) --n;
    return n;
}

kda::TwoPassBufs bufs_at(void* ws, const Layout& l) {
    char* b = static_cast<char*>(ws);
    kda::TwoPassBufs x;
    x.wn = b + l.wn;
    x.qt = b + l.qt;
    x.kht = b + l.kht;
    x.pm = b + l.pm;
    x.tt = b + l.tt;
    x.gam = reinterpret_cast<float*>(b + l.gam);
    return x;
}

// Upper bound on the chunks of packed sequences: sum ceil(len_n / C) <= T/C + N.
int64_t varlen_chunks(int64_t T_total, int chunk, int num_seqs) { return T_total / chunk + num_seqs; }

int64_t seg_chunks(int64_t seg_len, int chunk, int num_seqs) {
    return (int64_t)num_seqs * ((seg_len + chunk - 1) / chunk);
}

// Value tiles per scan wave: two (half the operand traffic per column) when
// that still leaves many workgroups; a scan workgroup covers 64 NVT state
// columns (4 waves of 16 NVT).  The scan launcher keeps one tile wherever its
// loader waves apply (all but the KCP pairs), which measured faster there.
int pick_nvt(int64_t chains, int dvt) {
    if (dvt % 128 != 0) return 1;
    return chains * (dvt / 128) >= 1024 ? 2 : 1;
}

// Byte sizes of the KCP workspace parts: segment pairs and entering states,
// then the group pairs and group entering states of the two-level scan.
void kcp_parts(int H, int dk, int dv, int nseg, size_t* pairs, size_t* starts, size_t* gpairs,
               size_t* gstarts) {
    const int L = kda::kcp_group_len(nseg), G = (nseg + L - 1) / L;
    *pairs = round_up((size_t)nseg * H * dk * (size_t)(dk + dv) * sizeof(float), 256);
    *starts = round_up((size_t)nseg * H * dk * (size_t)dv * sizeof(float), 256);
    *gpairs = round_up((size_t)G * H * dk * (size_t)(dk + dv) * sizeof(float), 256);
    *gstarts = round_up((size_t)G * H * dk * (size_t)dv * sizeof(float), 256);
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

size_t kda_chunk_fwd_workspace_size(kda_dtype dt, int H, int dk, int dv, int chunk, int num_seqs,
                                    int64_t T_total) {
    if ((dt != KDA_BF16 && dt != KDA_F32) || H <= 0 || num_seqs <= 0 || T_total < 0) return 0;
    if (!kda::prefill_supported((int)dt, dk, dv, chunk)) return 0;
    return twopass_layout(dt, H, dk, dv, chunk, num_seqs, varlen_chunks(T_total, chunk, num_seqs)).total;
}

size_t kda_chunk_fwd_workspace_min(kda_dtype dt, int H, int dk, int dv, int chunk, int num_seqs,
                                   int64_t T_total) {
    const size_t full = kda_chunk_fwd_workspace_size(dt, H, dk, dv, chunk, num_seqs, T_total);
    if (full == 0) return 0;
    const size_t one = twopass_layout(dt, H, dk, dv, chunk, num_seqs, 1,
                                      (size_t)num_seqs * H * dk * dv * sizeof(float)).total;
    return one < full ? one : full;
}

}  // extern "C"

namespace {

// kda_chunk_fwd, optionally saving the state every ckpt_interval tokens.
// fused: q, k are raw and g, beta are the pre-activations a, b in dtype dt.
kda_status chunk_fwd_impl(kda_dtype dt, bool fused, int H, int dk, int dv, int chunk, float scale, int num_seqs,
                          int64_t T_total, const int32_t* cu_seqlens, const void* q, const void* k,
                          const void* v, const void* g, const void* beta, const void* z,
                          const float* initial_state, float* final_state, void* y, int ckpt_interval,
                          float* checkpoints, int32_t* ckpt_offsets, int64_t ckpt_capacity,
                          void* workspace, size_t workspace_bytes, void* stream) {
    if (dt != KDA_BF16 && dt != KDA_F32) return KDA_ERR_INVALID_ARGUMENT;
    if (H <= 0 || num_seqs <= 0 || T_total < 0) return KDA_ERR_INVALID_ARGUMENT;
    if (!cu_seqlens && num_seqs != 1) return KDA_ERR_INVALID_ARGUMENT;
    if ((int64_t)num_seqs * H > (int64_t)1 << 28) return KDA_ERR_INVALID_ARGUMENT;
    if (T_total / 16 + num_seqs > ((int64_t)1 << 31) / H) return KDA_ERR_INVALID_ARGUMENT;
    if (!head_shape_ok(dk, dv)) return KDA_ERR_UNSUPPORTED;
    if (!kda::prefill_supported((int)dt, dk, dv, chunk)) return KDA_ERR_UNSUPPORTED;
    if (T_total > 0 && (!q || !k || !v || !g || !beta || !y)) return KDA_ERR_INVALID_ARGUMENT;
    if (!workspace) return KDA_ERR_INVALID_ARGUMENT;
    const bool ckpt = ckpt_interval != 0;
    if (ckpt) {
        if (ckpt_interval < 0 || ckpt_interval % chunk != 0) return KDA_ERR_INVALID_ARGUMENT;
        if (!ckpt_offsets || (!checkpoints && T_total >= ckpt_interval)) return KDA_ERR_INVALID_ARGUMENT;
        if (ckpt_capacity < T_total / ckpt_interval) return KDA_ERR_INVALID_ARGUMENT;
        if (!aligned(checkpoints, 16) || !aligned(ckpt_offsets, 4)) return KDA_ERR_INVALID_ARGUMENT;
    }
    const size_t ea = vec_align(dt);
    // g in runs of four fp32 (fused: a in runs of four elements), beta one scalar per (token, head)
    const size_t ga = fused ? ea : 16, ba = fused ? (dt == KDA_BF16 ? 2 : 4) : 4;
    if (!aligned(q, ea) || !aligned(k, ea) || !aligned(v, ea) || !aligned(z, ea) ||
        !aligned(y, ea) || !aligned(g, ga) || !aligned(beta, ba) || !aligned(cu_seqlens, 4) ||
        !aligned(initial_state, 16) || !aligned(final_state, 16) || !aligned(workspace, 256))
        return KDA_ERR_INVALID_ARGUMENT;
    // all chunks of the call (an upper bound with packed sequences), and the
    // slab the workspace holds: all of them, or as many as fit beside a carry
    const int64_t nchunks = cu_seqlens ? varlen_chunks(T_total, chunk, num_seqs)
                                       : seg_chunks(T_total, chunk, num_seqs);
    const size_t carry_bytes = (size_t)num_seqs * H * dk * dv * sizeof(float);
    Layout l = twopass_layout(dt, H, dk, dv, chunk, num_seqs, varlen_chunks(T_total, chunk, num_seqs));
    int64_t slab = nchunks;
    bool bounded = workspace_bytes < l.total;
    if (bounded) {
        slab = slab_chunks(dt, H, dk, dv, chunk, num_seqs, nchunks, carry_bytes, workspace_bytes);
        if (slab <= 0) return KDA_ERR_WORKSPACE_TOO_SMALL;
        l = twopass_layout(dt, H, dk, dv, chunk, num_seqs, slab, carry_bytes);
    }
    kda::TwoPassArgs a{};
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
    a.fused = fused;
    a.z = z;
    a.initial_state = initial_state;
    a.final_state = final_state;
    a.final_seq_lo = 0;
    a.y = y;
    a.mode = cu_seqlens ? kda::kModeVarlen : kda::kModeSeq;
    a.nvt = pick_nvt((int64_t)num_seqs * H, dv);
    a.bufs = bufs_at(workspace, l);
    a.chunk_cap = nchunks;
    a.carry = bounded ? reinterpret_cast<float*>(static_cast<char*>(workspace) + l.carry) : nullptr;
    a.ckpt = ckpt ? checkpoints : nullptr;
    a.ckpt_off = ckpt ? ckpt_offsets : nullptr;
    a.ckpt_every = ckpt ? ckpt_interval / chunk : 1;
    a.ckpt_cap = ckpt ? ckpt_capacity : 0;
    a.stream = stream;
    int32_t* chunk_off = nullptr;
    int32_t* order = nullptr;
    if (cu_seqlens) {
        chunk_off = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + l.chunk_off);
        order = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + l.order);
    }
    if (cu_seqlens || ckpt) {
        if (kda::launch_varlen_plan(num_seqs, cu_seqlens, T_total, chunk, ckpt ? ckpt_interval : 0, chunk_off,
                                    order, ckpt ? ckpt_offsets : nullptr, stream) != hipSuccess)
            return KDA_ERR_HIP;
    }
    // one slab after the other on the stream: its products, then every chain's
    // chunks inside it (with no chunks, one empty slab still runs the chains)
    for (int64_t lo = 0; lo < nchunks || lo == 0; lo += slab) {
        a.slab_lo = lo;
        a.slab_hi = lo + slab < nchunks ? lo + slab : nchunks;
        if (kda::launch_chunk_prep(a, chunk_off, a.slab_hi - lo) != hipSuccess) return KDA_ERR_HIP;
        if (kda::launch_chunk_state(a, chunk_off, order) != hipSuccess) return KDA_ERR_HIP;
        if (slab <= 0) break;
    }
    return KDA_OK;
}

// kda_decode_step; fused: q, k raw and g, beta the pre-activations a, b in dtype dt.
kda_status decode_impl(kda_dtype dt, bool fused, int N, int H, int dk, int dv, float scale, const void* q,
                       const void* k, const void* v, const void* g, const void* beta, const void* z,
                       float* state, void* y, void* stream) {
    if (dt != KDA_BF16 && dt != KDA_F32) return KDA_ERR_INVALID_ARGUMENT;
    if (N < 0 || H <= 0) return KDA_ERR_INVALID_ARGUMENT;
    if ((int64_t)N * H > (int64_t)1 << 30) return KDA_ERR_INVALID_ARGUMENT;
    if (!head_shape_ok(dk, dv)) return KDA_ERR_UNSUPPORTED;
    if (N > 0 && (!q || !k || !v || !g || !beta || !state || !y)) return KDA_ERR_INVALID_ARGUMENT;
    const size_t ea = elt_align(dt);
    const size_t ga = fused ? ea : 8, ba = fused ? (dt == KDA_BF16 ? 2 : 4) : 4;
    if (!aligned(q, ea) || !aligned(k, ea) || !aligned(v, ea) || !aligned(z, ea) ||
        !aligned(y, ea) || !aligned(g, ga) || !aligned(beta, ba) || !aligned(state, 16))
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
    a.fused = fused;
    a.z = z;
    a.state = state;
    a.y = y;
    a.stream = stream;
    return from_hip(kda::launch_decode(a));
}

}  // namespace

extern "C" {

kda_status kda_chunk_fwd(kda_dtype dt, int H, int dk, int dv, int chunk, float scale,
                         int num_seqs, int64_t T_total, const int32_t* cu_seqlens,
                         const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const void* z, const float* initial_state,
                         float* final_state, void* y, void* workspace, size_t workspace_bytes,
                         void* stream) {
    return chunk_fwd_impl(dt, false, H, dk, dv, chunk, scale, num_seqs, T_total, cu_seqlens, q, k, v, g, beta,
                          z, initial_state, final_state, y, 0, nullptr, nullptr, 0, workspace, workspace_bytes,
                          stream);
}

}  // extern "C"

namespace {

// Device scratch of kda_chunk_fwd_noalloc: a file-scope array that every GPU
// holds a copy of from the moment the library is loaded until the process
// ends.  Host code never names it directly (its host-side name is only a
// stand-in for the symbol); the device address of each GPU's copy is looked up
// once, with that GPU current, and kept per device.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

kda_status scratch_on_current_device(void** out) {
    constexpr int kMaxDev = 64;
    static std::mutex mu;
    static void* ptrs[kMaxDev] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KDA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDev) return KDA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return KDA_ERR_HIP;
        ptrs[dev] = ptr;
    }
    *out = ptrs[dev];
    return KDA_OK;
}

}  // namespace

extern "C" {

size_t kda_noalloc_scratch_bytes(void) { return kScratchBytes; }

kda_status kda_chunk_fwd_noalloc(kda_dtype dt, int H, int dk, int dv, int chunk, float scale,
                                 int num_seqs, int64_t T_total, const int32_t* cu_seqlens,
                                 const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const void* z, const float* initial_state,
                                 float* final_state, void* y, void* stream) {
    // a shape whose smallest workspace exceeds the scratch is refused before
    // anything is looked up or launched
    const size_t least = kda_chunk_fwd_workspace_min(dt, H, dk, dv, chunk, num_seqs, T_total);
    if (least == 0) {
        return (dt != KDA_BF16 && dt != KDA_F32) || H <= 0 || num_seqs <= 0 || T_total < 0
                   ? KDA_ERR_INVALID_ARGUMENT : KDA_ERR_UNSUPPORTED;
    }
    if (least > kScratchBytes) return KDA_ERR_WORKSPACE_TOO_SMALL;
    void* ws = nullptr;
    const kda_status st = scratch_on_current_device(&ws);
    if (st != KDA_OK) return st;
    return chunk_fwd_impl(dt, false, H, dk, dv, chunk, scale, num_seqs, T_total, cu_seqlens, q, k, v, g, beta,
                          z, initial_state, final_state, y, 0, nullptr, nullptr, 0, ws, kScratchBytes, stream);
}

kda_status kda_chunk_fwd_fused(kda_dtype dt, int H, int dk, int dv, int chunk, float scale,
                               int num_seqs, int64_t T_total, const int32_t* cu_seqlens,
                               const void* q, const void* k, const void* v, const void* a,
                               const void* b, const void* z, const float* initial_state,
                               float* final_state, void* y, void* workspace, size_t workspace_bytes,
                               void* stream) {
    return chunk_fwd_impl(dt, true, H, dk, dv, chunk, scale, num_seqs, T_total, cu_seqlens, q, k, v, a, b, z,
                          initial_state, final_state, y, 0, nullptr, nullptr, 0, workspace, workspace_bytes,
                          stream);
}

kda_status kda_chunk_fwd_checkpointed(kda_dtype dt, int H, int dk, int dv, int chunk, float scale,
                                      int num_seqs, int64_t T_total, const int32_t* cu_seqlens,
                                      const void* q, const void* k, const void* v, const float* g,
                                      const float* beta, const void* z, const float* initial_state,
                                      float* final_state, void* y, int ckpt_interval, float* checkpoints,
                                      int32_t* ckpt_offsets, int64_t ckpt_capacity, void* workspace,
                                      size_t workspace_bytes, void* stream) {
    if (ckpt_interval <= 0) return KDA_ERR_INVALID_ARGUMENT;
    return chunk_fwd_impl(dt, false, H, dk, dv, chunk, scale, num_seqs, T_total, cu_seqlens, q, k, v, g, beta, z,
                          initial_state, final_state, y, ckpt_interval, checkpoints, ckpt_offsets,
                          ckpt_capacity, workspace, workspace_bytes, stream);
}

size_t kda_kcp_workspace_size(kda_dtype dt, int H, int dk, int dv, int chunk, int64_t T,
                              int num_segments) {
    if ((dt != KDA_BF16 && dt != KDA_F32) || H <= 0 || num_segments <= 0 || T < num_segments) return 0;
    if (!kda::prefill_supported((int)dt, dk, dv, chunk)) return 0;
    size_t pairs, starts, gpairs, gstarts;
    kcp_parts(H, dk, dv, num_segments, &pairs, &starts, &gpairs, &gstarts);
    const int64_t seg_len = (T + num_segments - 1) / num_segments;
    return pairs + starts + gpairs + gstarts +
           twopass_layout(dt, H, dk, dv, chunk, num_segments, seg_chunks(seg_len, chunk, num_segments)).total;
}

size_t kda_kcp_workspace_min(kda_dtype dt, int H, int dk, int dv, int chunk, int64_t T,
                             int num_segments) {
    const size_t full = kda_kcp_workspace_size(dt, H, dk, dv, chunk, T, num_segments);
    if (full == 0) return 0;
    size_t pairs, starts, gpairs, gstarts;
    kcp_parts(H, dk, dv, num_segments, &pairs, &starts, &gpairs, &gstarts);
    const size_t one = pairs + starts + gpairs + gstarts + twopass_layout(dt, H, dk, dv, chunk, num_segments, 1).total;
    return one < full ? one : full;
}

kda_status kda_kcp_scan(kda_dtype dt, int H, int dk, int dv, int chunk, float scale, int64_t T,
                        int num_segments, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, const void* z,
                        const float* initial_state, float* final_state, void* y,
                        void* workspace, size_t workspace_bytes, void* stream) {
    if (dt != KDA_BF16 && dt != KDA_F32) return KDA_ERR_INVALID_ARGUMENT;
    if (H <= 0 || num_segments <= 0 || T < num_segments) return KDA_ERR_INVALID_ARGUMENT;
    if (T / 16 + num_segments > ((int64_t)1 << 31) / H) return KDA_ERR_INVALID_ARGUMENT;
    if (!head_shape_ok(dk, dv)) return KDA_ERR_UNSUPPORTED;
    if (!kda::prefill_supported((int)dt, dk, dv, chunk)) return KDA_ERR_UNSUPPORTED;
    if (!q || !k || !v || !g || !beta || !y || !workspace) return KDA_ERR_INVALID_ARGUMENT;
    const size_t ea = vec_align(dt);
    if (!aligned(q, ea) || !aligned(k, ea) || !aligned(v, ea) || !aligned(z, ea) ||
        !aligned(y, ea) || !aligned(g, 16) || !aligned(beta, 4) || !aligned(workspace, 256) ||
        !aligned(initial_state, 16) || !aligned(final_state, 16))
        return KDA_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < kda_kcp_workspace_min(dt, H, dk, dv, chunk, T, num_segments))
        return KDA_ERR_WORKSPACE_TOO_SMALL;
    size_t pbytes, sbytes, gpbytes, gsbytes;
    kcp_parts(H, dk, dv, num_segments, &pbytes, &sbytes, &gpbytes, &gsbytes);
    float* pairs = static_cast<float*>(workspace);
    float* starts = reinterpret_cast<float*>(static_cast<char*>(workspace) + pbytes);
    float* gpairs = reinterpret_cast<float*>(static_cast<char*>(workspace) + pbytes + sbytes);
    float* gstarts = reinterpret_cast<float*>(static_cast<char*>(workspace) + pbytes + sbytes + gpbytes);
    const size_t fixed = pbytes + sbytes + gpbytes + gsbytes;
    void* tp = static_cast<char*>(workspace) + fixed;
    // segments hold seg_len tokens each; with T not a multiple, trailing ones may be empty
    const int64_t seg_len = (T + num_segments - 1) / num_segments;
    const int64_t nchunks = seg_chunks(seg_len, chunk, num_segments);
    // the chunk products of all segments at once, or, in a bounded workspace,
    // of rectangles of segments x chunks (formed twice then: for the pairs
    // and for the outputs)
    int64_t slab = slab_chunks(dt, H, dk, dv, chunk, num_segments, nchunks, 0, workspace_bytes - fixed);
    if (slab <= 0) return KDA_ERR_WORKSPACE_TOO_SMALL;
    const bool bounded = slab < nchunks;
    const Layout l = twopass_layout(dt, H, dk, dv, chunk, num_segments, slab);
    kda::TwoPassArgs a{};
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
    a.bufs = bufs_at(tp, l);
    a.chunk_cap = nchunks;
    a.stream = stream;
    // phase 1: (M, Sloc) of every segment, as the state that the augmented value
    // block [0 | v] builds from the augmented start [I | 0]; between slabs the
    // augmented state waits in the pairs array itself
    a.mode = kda::kModePairs;
    a.nvt = pick_nvt((int64_t)num_segments * H, dk + dv);
    a.initial_state = nullptr;
    a.final_state = pairs;
    a.final_seq_lo = 0;
    a.carry = pairs;
    a.y = nullptr;
    // a bounded workspace holds a rectangle of segments x chunks at a time:
    // as many segments as make about one round of scan workgroups, and as
    // many of their chunks as then fit (slabs of consecutive global chunks
    // would hold a few whole segments, too few workgroups to fill the GPU)
    int cus = 0;
    if (bounded && kda::device_cu_count(&cus) != hipSuccess) return KDA_ERR_HIP;
    const int64_t cps = (seg_len + chunk - 1) / chunk;
    auto rects = [&](int wg_per_chain, int wg_per_cu, bool prep) -> kda_status {
        int64_t gs = (int64_t)cus * wg_per_cu / ((int64_t)wg_per_chain * H);
        gs = gs < 1 ? 1 : gs > num_segments ? num_segments : gs;
        if (gs > slab) gs = slab;
        int64_t pw = slab / gs;
        if (pw > cps) pw = cps;
        for (int64_t s0 = 0; s0 < num_segments; s0 += gs) {
            for (int64_t c0 = 0; c0 < cps; c0 += pw) {
                a.rect_w = (int)(c0 + pw < cps ? pw : cps - c0);
                a.rect_c0 = (int)c0;
                a.rect_s0 = (int)s0;
                a.rect_s1 = (int)(s0 + gs < num_segments ? s0 + gs : num_segments);
                if (prep && kda::launch_chunk_prep(a, nullptr, (int64_t)(a.rect_s1 - a.rect_s0) * a.rect_w) !=
                                hipSuccess)
                    return KDA_ERR_HIP;
                if (kda::launch_chunk_state(a, nullptr, nullptr) != hipSuccess) return KDA_ERR_HIP;
            }
        }
        a.rect_w = 0;
        return KDA_OK;
    };
    if (bounded) {
        // The pairs read no Qt and no P, which pass 1 then skips; the
        // outputs below prepare their rectangles again in full
        int per_chain = 1, per_cu = 1;
        kda::state_geometry(a, &per_chain, &per_cu);
        a.pairs_only = true;
        const kda_status st = rects(per_chain, per_cu, true);
        a.pairs_only = false;
        if (st != KDA_OK) return st;
    } else {
        a.slab_lo = 0;
        a.slab_hi = nchunks;
        if (kda::launch_chunk_prep(a, nullptr, nchunks) != hipSuccess) return KDA_ERR_HIP;
        if (kda::launch_chunk_state(a, nullptr, nullptr) != hipSuccess) return KDA_ERR_HIP;
    }
    // phase 2: entering state of every segment
    if (kda::launch_kcp_scan(H, dk, dv, num_segments, pairs, initial_state, starts, gpairs, gstarts,
                             (hipStream_t)stream) != hipSuccess)
        return KDA_ERR_HIP;
    // phase 3: outputs of every segment from its entering state; the last
    // segment's final state is the sequence's final state.  Between slabs a
    // segment's state waits in its own entering-state slot.
    a.mode = kda::kModeFinish;
    a.nvt = pick_nvt((int64_t)num_segments * H, dv);
    a.initial_state = starts;
    a.final_state = final_state;
    a.final_seq_lo = num_segments - 1;
    a.carry = starts;
    a.y = y;
    if (bounded) {
        int per_chain = 1, per_cu = 1;
        kda::state_geometry(a, &per_chain, &per_cu);
        return rects(per_chain, per_cu, true);
    }
    // one slab: the products of phase 1 are still in place
    if (kda::launch_chunk_state(a, nullptr, nullptr) != hipSuccess) return KDA_ERR_HIP;
    return KDA_OK;
}

kda_status kda_decode_step(kda_dtype dt, int N, int H, int dk, int dv, float scale,
                           const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const void* z, float* state, void* y,
                           void* stream) {
    return decode_impl(dt, false, N, H, dk, dv, scale, q, k, v, g, beta, z, state, y, stream);
}

kda_status kda_decode_step_fused(kda_dtype dt, int N, int H, int dk, int dv, float scale,
                                 const void* q, const void* k, const void* v, const void* a,
                                 const void* b, const void* z, float* state, void* y,
                                 void* stream) {
    return decode_impl(dt, true, N, H, dk, dv, scale, q, k, v, a, b, z, state, y, stream);
}

kda_status kda_decode_replay(kda_dtype dt, int N, int Td, int H, int dk, int dv, float scale,
                             const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const void* z, const int32_t* accepted,
                             float* state, void* y, void* stream) {
    if (dt != KDA_BF16 && dt != KDA_F32) return KDA_ERR_INVALID_ARGUMENT;
    if (N < 0 || Td <= 0 || H <= 0) return KDA_ERR_INVALID_ARGUMENT;
    if ((int64_t)N * H > (int64_t)1 << 30 || (int64_t)N * Td * H > (int64_t)1 << 31)
        return KDA_ERR_INVALID_ARGUMENT;
    if (!head_shape_ok(dk, dv)) return KDA_ERR_UNSUPPORTED;
    if (!y && !accepted) return KDA_ERR_INVALID_ARGUMENT;   // nothing to produce
    if (N > 0 && (!q || !k || !v || !g || !beta || !state)) return KDA_ERR_INVALID_ARGUMENT;
    const size_t ea = elt_align(dt);
    if (!aligned(q, ea) || !aligned(k, ea) || !aligned(v, ea) || !aligned(z, ea) ||
        !aligned(y, ea) || !aligned(g, 8) || !aligned(beta, 4) || !aligned(state, 16) ||
        !aligned(accepted, 4))
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
    return from_hip(kda::launch_replay(a, Td, accepted));
}

}  // extern "C"

namespace kda {

hipError_t ensure_lds_limit(const void* kern, int bytes) {
    static std::mutex mu;
    static std::set<std::pair<int, const void*>> done;   // (device, kernel) already raised
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    if (done.count({dev, kern})) return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) done.insert({dev, kern});
    return e;
}

hipError_t device_cu_count(int* cus) {
    constexpr int kMaxDev = 64;
    static int cached[kMaxDev] = {};   // 0: not queried yet
    static std::mutex mu;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    if (dev >= 0 && dev < kMaxDev && cached[dev] > 0) {
        *cus = cached[dev];
        return hipSuccess;
    }
    e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess && dev >= 0 && dev < kMaxDev) cached[dev] = *cus;
    return e;
}

bool prefill_supported(int dtype, int dk, int dv, int chunk) {
    if (!((dk == 64 && dv == 64) || (dk == 128 && dv == 128))) return false;
    if (chunk != 16 && chunk != 32 && chunk != 64) return false;
    return dtype == 0 || dtype == 1;
}

}  // namespace kda
