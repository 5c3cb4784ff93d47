/*
 * kda.h -- C ABI of libkda: the Kimi Delta Attention (KDA) recurrence on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (per sequence and head; page "Exercices", Niveau 2 Q7 names
 * its three operations forget / erase / write; page "Ce qui est public et ce
 * qui ne l'est pas", table "Entièrement publié et vérifiable", lists the
 * recurrence, its parametrisation (q, k, v, beta, z), the bounded decay and
 * the output gate):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 *     y_t = o_t * sigmoid(z_t)        (gated; y_t = o_t when z == NULL)
 *
 * S is dk x dv per head.  Every entry point takes caller-owned device memory,
 * enqueues its kernels on `stream` (a hipStream_t; NULL = the null stream)
 * and returns without synchronising.  Problems the host can see (a NULL
 * required pointer, unsupported sizes, misalignment, a short workspace) are
 * reported by the return code BEFORE anything is launched; a failed launch
 * returns KDA_ERR_HIP; faults inside a kernel surface at the caller's next
 * synchronisation.  No call allocates device or host memory, keeps state
 * between calls, or throws across the ABI.  Calls on different streams may
 * run concurrently; results are deterministic (no atomics in reductions).
 * No call issues a memset or a host synchronisation, so a call can be
 * recorded in a HIP graph (stream capture) once an earlier call on the same
 * device has run: the first call of each kernel on a device raises its LDS
 * limit, which is not a stream operation.
 *
 * Layouts (row-major, last index fastest; T_total = packed token count):
 *   q, k        [T_total, H, dk]       dtype dt
 *   v, z, y     [T_total, H, dv]       dtype dt
 *   g           [T_total, H, dk]       fp32, natural log of the decay alpha
 *   beta        [T_total, H]           fp32
 *   states      [N, H, dk, dv]         fp32 (N = sequences or requests)
 * Alignment: kda_chunk_fwd and kda_kcp_scan move q, k, v, z and y in runs of
 * four elements, so those need 8 bytes (bf16) or 16 bytes (fp32), and g 16
 * bytes; kda_decode_step needs 4 bytes (bf16) or 8 bytes (fp32) and g 8.
 * States are 16-byte aligned, workspaces 256-byte aligned.
 *
 * Preconditions (documented, not checked on the hot path; the *_fused entry
 * points establish the first three themselves from raw inputs):
 *   - q and k are L2-normalised per (token, head): page "Exercices",
 *     Niveau 2 Q9 -- with unit keys I - beta k k^T does not expand the state;
 *   - g lies in [g_min, 0] with g_min = -5 (page "Exercices", Niveau 2 Q8:
 *     the cumulative log-decay of a 16-token tile is then >= -80, and e^80
 *     fits the bf16 range); the kernels keep their accuracy down to
 *     g = -5.4 over whole 16-token tiles (e^86.4 still fits bf16), which the
 *     GPU tests check on every entry point that carries a state;
 *   - beta lies in [0, 1];
 *   - cu_seqlens is non-decreasing, cu_seqlens[0] = 0,
 *     cu_seqlens[num_seqs] = T_total.
 *
 * Supported sizes: (dk, dv) in {(64, 64), (128, 128)}; chunk in {16, 32, 64}.
 * Anything else returns KDA_ERR_UNSUPPORTED.
 */
#ifndef LIBKDA_KDA_H
#define LIBKDA_KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1,   /* NULL required pointer, negative size, misalignment */
    KDA_ERR_UNSUPPORTED = 2,        /* dk/dv/chunk/dtype combination not built */
    KDA_ERR_WORKSPACE_TOO_SMALL = 3,
    KDA_ERR_HIP = 4                 /* a HIP runtime call or kernel launch failed */
} kda_status;

typedef enum {
    KDA_BF16 = 0,   /* q, k, v, z, y stored as bfloat16 */
    KDA_F32 = 1     /* q, k, v, z, y stored as float32 */
} kda_dtype;

/* Version of the library as 10000 * major + 100 * minor + patch. */
int kda_version(void);

/* Static description of a status code (never NULL). */
const char* kda_status_string(kda_status status);

/*
 * kda_chunk_fwd -- prefill: run the recurrence over every token of a batch of
 * packed sequences (page "Exercices", Niveau 1 Q4: prefill processes the
 * whole input in parallel and is compute-limited).
 *
 *   dt, H, dk, dv   dtype and head shape.
 *   chunk           tokens per chunk of the blocked algorithm (16, 32 or 64); it
 *                   changes rounding only, never the result's definition.
 *   scale           factor on the output o_t (1.0 for the plain recurrence).
 *   num_seqs        number of packed sequences (>= 1).
 *   T_total         total tokens (>= 0; 0 is a no-op apart from copying the
 *                   initial state to the final state).
 *   cu_seqlens      device int32 [num_seqs + 1] offsets, or NULL when
 *                   num_seqs == 1 (one sequence of T_total tokens).
 *   q, k, v, g, beta  inputs (layouts above); all required.
 *   z               gate input [T_total, H, dv], or NULL for no gate.
 *   initial_state   fp32 [num_seqs, H, dk, dv] or NULL (zeros).
 *   final_state     fp32 [num_seqs, H, dk, dv] or NULL (not written).  May
 *                   alias initial_state (each state is read before written).
 *   y               output [T_total, H, dv] in dtype dt; must not alias inputs.
 *   workspace       device buffer, 256-byte aligned, overwritten; of
 *   workspace_bytes at least kda_chunk_fwd_workspace_min bytes for the same
 *                   (dt, H, dk, dv, chunk, num_seqs, T_total), else
 *                   KDA_ERR_WORKSPACE_TOO_SMALL; kda_chunk_fwd_workspace_size
 *                   bytes or more run in one pass.
 *
 * Two passes on `stream`: every (chunk, head) first forms the products of its
 * chunk that do not involve the entering state (the gated Gram products, the
 * inverse of the unit lower-triangular I + diag(beta) A, and the operands
 * derived from them) into the workspace, all chunks at once; then one pass
 * per (sequence, head) carries the state through its chunks.
 */
kda_status kda_chunk_fwd(kda_dtype dt, int H, int dk, int dv, int chunk, float scale,
                         int num_seqs, int64_t T_total, const int32_t* cu_seqlens,
                         const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const void* z, const float* initial_state,
                         float* final_state, void* y, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * kda_chunk_fwd_fused -- kda_chunk_fwd fed by the layer's raw projections, with
 * the input-side step fused into the chunk-preparation kernel (page "Ce qui
 * est public et ce qui ne l'est pas", table "Entièrement publié": the KDA
 * parametrisation (q, k, v, beta, z) and the bounded decay with g_min = -5;
 * page "Retrouver les 2,8 T de paramètres", Bloc 4: beta and alpha come from
 * the low-rank projections W_beta, W_alpha; page "Exercices", Niveau 2 Q9:
 * unit keys).  Per (token, head) the kernel forms
 *     k^ = k / sqrt(sum_c k_c^2 + 1e-6)      q^ likewise
 *     g  = -5 sigmoid(a)  (per key channel, in (-5, 0))
 *     beta = sigmoid(b)
 * in fp32 and runs kda_chunk_fwd's recurrence on (q^, k^, v, g, beta, z).
 *
 *   q, k             [T_total, H, dk] in dtype dt, any length (a zero vector
 *                    stays zero).
 *   a                [T_total, H, dk] in dtype dt: decay pre-activation
 *                    (aligned like q).  Half the bytes of an fp32 g at bf16.
 *   b                [T_total, H] in dtype dt: beta pre-activation (aligned to
 *                    one element).
 *   all other arguments, the workspace and its size: as kda_chunk_fwd.
 */
kda_status kda_chunk_fwd_fused(kda_dtype dt, int H, int dk, int dv, int chunk, float scale,
                               int num_seqs, int64_t T_total, const int32_t* cu_seqlens,
                               const void* q, const void* k, const void* v, const void* a,
                               const void* b, const void* z, const float* initial_state,
                               float* final_state, void* y, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * kda_chunk_fwd_workspace_size -- bytes of device workspace with which
 * kda_chunk_fwd (and its _fused and _checkpointed forms) runs every chunk in
 * one pass of each kernel, the fastest way: per (chunk, head) about
 * 3 dk C elements of dtype dt, the lower triangles of two C x C products in
 * dtype dt, and dk fp32 (60.5 KiB at bf16, dk = dv = 128, C = 64), for up to
 * T_total / chunk + num_seqs chunks.
 * Returns 0 for invalid or unsupported sizes.
 *
 * kda_chunk_fwd_workspace_min -- the smallest workspace those calls accept:
 * one chunk per head plus a carry of num_seqs * H * dk * dv fp32 states.  Any
 * size from the minimum up works, so the memory of a prefill need not grow
 * with T_total (the state itself has a fixed size whatever the length: page
 * "Exercices", Niveau 1 Q6).  With less than the full size the chunks are
 * taken in time slabs of as many chunks as fit, one slab after the other on
 * the stream, each chain's state carried between slabs through the carry
 * (the same arithmetic, so the same results bit for bit); each slab costs two
 * more kernel launches and one read and write of the carried states.
 */
size_t kda_chunk_fwd_workspace_size(kda_dtype dt, int H, int dk, int dv, int chunk, int num_seqs,
                                    int64_t T_total);
size_t kda_chunk_fwd_workspace_min(kda_dtype dt, int H, int dk, int dv, int chunk, int num_seqs,
                                   int64_t T_total);

/*
 * kda_chunk_fwd_checkpointed -- kda_chunk_fwd that also saves the state every
 * ckpt_interval tokens of each sequence, for a prefix cache (page
 * "Exercices", Niveau 3 Q26: on a hybrid model a cached prefix is reusable
 * only at a boundary where the KDA state was saved, and the pages decouple the
 * 512-token hash granularity from allocation; the boundaries here are every
 * ckpt_interval tokens).
 *
 *   ckpt_interval    tokens between checkpoints: a positive multiple of chunk.
 *   checkpoints      fp32 [capacity, H, dk, dv]: checkpoint j of sequence n,
 *                    the state after its first (j + 1) ckpt_interval tokens,
 *                    lands in row ckpt_offsets[n] + j, for
 *                    j < floor(len_n / ckpt_interval).  Other rows untouched.
 *   ckpt_offsets     device int32 [num_seqs + 1], written by the call: the
 *                    prefix sum of floor(len_n / ckpt_interval).
 *   ckpt_capacity    rows of checkpoints; at least T_total / ckpt_interval
 *                    (which bounds the total), else KDA_ERR_INVALID_ARGUMENT.
 *   all other arguments and the workspace: as kda_chunk_fwd.
 * The checkpoints are states of the same computation as final_state (same
 * rounding); each costs one extra write of the fp32 state.
 */
kda_status kda_chunk_fwd_checkpointed(kda_dtype dt, int H, int dk, int dv, int chunk, float scale,
                                      int num_seqs, int64_t T_total, const int32_t* cu_seqlens,
                                      const void* q, const void* k, const void* v, const float* g,
                                      const float* beta, const void* z, const float* initial_state,
                                      float* final_state, void* y, int ckpt_interval,
                                      float* checkpoints, int32_t* ckpt_offsets,
                                      int64_t ckpt_capacity, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * kda_chunk_fwd_noalloc -- kda_chunk_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts that
 * forbid allocation): the same arguments minus the workspace.  The chunk
 * products go to a scratch array of kda_noalloc_scratch_bytes() (64 MiB) that
 * the library holds on every GPU it is loaded on until the process ends; the
 * call runs in time slabs of as many chunks as fit there (as kda_chunk_fwd
 * with that workspace: the same results bit for bit).  It allocates nothing,
 * calls no allocating routine and needs nothing zeroed.
 *
 *   Returns KDA_ERR_WORKSPACE_TOO_SMALL when even one chunk per head plus the
 *   carried states (num_seqs * H * dk * dv fp32) exceed the scratch
 *   (kda_chunk_fwd_workspace_min above kda_noalloc_scratch_bytes()).
 *   Every call on one GPU uses that GPU's one scratch: calls that overlap in
 *   time on one GPU (different streams, or different host threads) race and
 *   corrupt each other's results; callers must order them.
 */
kda_status kda_chunk_fwd_noalloc(kda_dtype dt, int H, int dk, int dv, int chunk, float scale,
                                 int num_seqs, int64_t T_total, const int32_t* cu_seqlens,
                                 const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const void* z, const float* initial_state,
                                 float* final_state, void* y, void* stream);
size_t kda_noalloc_scratch_bytes(void);

/*
 * kda_kcp_workspace_size -- bytes of device workspace with which kda_kcp_scan
 * runs fastest for H heads of a T-token sequence split into num_segments
 * segments: the segment pairs (M [dk x dk], Sloc [dk x dv]) and the entering
 * states [dk x dv], all fp32, plus the chunk products of kda_chunk_fwd over
 * all segments, formed once for the pairs and the outputs.  Returns 0 for
 * invalid or unsupported sizes.
 *
 * kda_kcp_workspace_min -- the smallest workspace kda_kcp_scan accepts: the
 * pairs and entering states (which do not depend on T) plus one chunk per
 * head.  Between the two sizes the chunk products are formed in slabs of
 * consecutive chunks, twice (once for the pairs, once for the outputs), and a
 * segment cut by a slab boundary waits in its own pair or entering-state slot.
 */
size_t kda_kcp_workspace_size(kda_dtype dt, int H, int dk, int dv, int chunk, int64_t T,
                              int num_segments);
size_t kda_kcp_workspace_min(kda_dtype dt, int H, int dk, int dv, int chunk, int64_t T,
                             int num_segments);

/*
 * kda_kcp_scan -- one long sequence of T tokens split into num_segments equal
 * contiguous segments (the last one may be shorter) processed side by side.
 * Each segment's effect on the state entering it is the pair (cumulative
 * transition M, local state Sloc): S_end = M S_start + Sloc; pairs compose as
 * (M2, S2) o (M1, S1) = (M2 M1, M2 S1 + S2) (page "Exercices", Niveau 3
 * Q21-Q22; page "Reproduire Kimi K3", "Le script de vérification").  Three
 * phases on `stream`: pairs of all segments in parallel, a scan of the pairs
 * giving every segment its entering state, then every segment's outputs (the
 * chunk products are formed once and serve the first and third phases).  The
 * result equals kda_chunk_fwd on the same sequence up to rounding.
 *
 *   T, num_segments  T >= num_segments >= 1.
 *   q..z, initial_state, final_state, y: as kda_chunk_fwd with one sequence.
 *   workspace        device buffer, 256-byte aligned, overwritten, of at least
 *                    kda_kcp_workspace_min bytes (else
 *                    KDA_ERR_WORKSPACE_TOO_SMALL); kda_kcp_workspace_size
 *                    bytes or more form the chunk products only once.
 */
kda_status kda_kcp_scan(kda_dtype dt, int H, int dk, int dv, int chunk, float scale, int64_t T,
                        int num_segments, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, const void* z,
                        const float* initial_state, float* final_state, void* y,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_decode_step -- decode: one token for each of N requests against states
 * resident in device memory (page "Exercices", Niveau 1 Q4: decode is limited
 * by memory bandwidth; Q6: the KDA state has a fixed size whatever the
 * length).  One pass over each state: decay, the two reductions S^T k and
 * S^T q, the in-place rank-1 update and the gated output.
 *
 *   N                requests (>= 0).
 *   q, k, v, z       [N, H, d] in dtype dt (z may be NULL).
 *   g, beta          [N, H, dk] and [N, H] fp32.
 *   state            fp32 [N, H, dk, dv], read and updated in place.
 *   y                [N, H, dv] output in dtype dt.
 */
kda_status kda_decode_step(kda_dtype dt, int N, int H, int dk, int dv, float scale,
                           const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const void* z, float* state, void* y,
                           void* stream);

/*
 * kda_decode_step_fused -- kda_decode_step on raw inputs: the fused input step
 * of kda_chunk_fwd_fused (unit q, k; g = g_min sigmoid(a); beta = sigmoid(b))
 * inside the decode kernel.
 *
 *   q, k             [N, H, dk] in dtype dt, any length (zero gives zero).
 *   a                [N, H, dk] in dtype dt: decay pre-activation.
 *   b                [N, H] in dtype dt: beta pre-activation.
 *   all other arguments: as kda_decode_step (a aligned like q; b to one element).
 */
kda_status kda_decode_step_fused(kda_dtype dt, int N, int H, int dk, int dv, float scale,
                                 const void* q, const void* k, const void* v, const void* a,
                                 const void* b, const void* z, float* state, void* y,
                                 void* stream);

/*
 * kda_decode_replay -- speculative decoding: Td draft tokens per request
 * replayed against the resident states (page "Exercices", Niveau 3 Q27: the
 * state after any accepted prefix is fully determined by the draft tokens'
 * projected inputs, which are much smaller than the state, so only those are
 * kept; the recurrence is replayed on chip and the verified state written
 * back).  One pass reads each state once.
 *
 *   N, Td            requests (>= 0) and draft tokens per request (>= 1).
 *   q, k, v, z       [N, Td, H, d] in dtype dt (z may be NULL): draft token t
 *                    of request n at [n, t].
 *   g, beta          [N, Td, H, dk] and [N, Td, H] fp32.
 *   accepted         device int32 [N] or NULL.  Given: the state of request n
 *                    is overwritten with the state after its first accepted[n]
 *                    draft tokens (clamped to [0, Td]; 0 leaves it as is).
 *                    NULL: the states are only read.
 *   state            fp32 [N, H, dk, dv], resident.
 *   y                [N, Td, H, dv] or NULL: the output of every draft token,
 *                    each computed from the state before the call (the
 *                    verification pass).
 * At least one of y and accepted must be given.  A verify call (y, no
 * accepted) followed by a commit call (accepted, no y) leaves the states as
 * if the accepted tokens had gone through kda_decode_step one by one.
 */
kda_status kda_decode_replay(kda_dtype dt, int N, int Td, int H, int dk, int dv, float scale,
                             const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const void* z, const int32_t* accepted,
                             float* state, void* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBKDA_KDA_H */
