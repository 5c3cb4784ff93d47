/*
 * kda_oracle.c -- plain fp64 CPU oracle of the Kimi Delta Attention (KDA)
 * recurrence.  TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and
 * the benchmark's CPU-baseline leg load this library.  It shares no source,
 * header, table or helper with the HIP library.
 *
 * What it computes (per sequence n and head h, everything in double):
 *
 *   S <- S0[n,h]                       (dk x dv; zeros when none is given)
 *   for each token t of the sequence:
 *       S     <- Diag(exp(g_t)) S                 (1) forget, channel by channel
 *       delta <- beta_t (v_t - S^T k_t)           (2) erase what the key held ...
 *       S     <- S + k_t delta^T                  (3) ... and write the new value
 *       o_t   <- scale * S^T q_t                  output read from S_t
 *       y_t   <- o_t * sigmoid(z_t)  (gated)  or  o_t
 *
 * Steps (1)-(3) are S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1}
 * + beta_t k_t v_t^T with alpha_t = exp(g_t): the three operations (forget,
 * erase, write) of page "Exercices", Niveau 2 Q7; the log-decay g is per key
 * channel and bounded below by g_min = -5 (same page, Q8; page "Ce qui est
 * public et ce qui ne l'est pas", table "Entièrement publié", decay row); the
 * output gate o * sigmoid(z) is the KDA output gate of that table.
 *
 * KCP (page "Exercices", Niveau 3 Q21-Q22; page "Reproduire Kimi K3", "Le
 * script de vérification"): a segment acts on the state entering it as
 * S_end = M S_start + Sloc, with M the product of the segment's transitions
 * (I - beta k k^T) Diag(alpha) and Sloc the state the segment builds from
 * zero.  Pairs compose as (M2, S2) o (M1, S1) = (M2 M1, M2 S1 + S2), so a
 * prefix over segments gives every segment its entering state.
 *
 * Inputs are read in place: bf16 values are given as their raw 16-bit
 * patterns and widened exactly; fp32 values are widened exactly.  With dtype
 * KDAO_F64 every input (q, k, v, z and also g, beta) is double, which is how
 * the fused-input path (gates and norms formed from raw inputs in double)
 * reaches the same loop.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KDAO_BF16 0
#define KDAO_F32 1
#define KDAO_F64 2

static double load_elt(int dtype, const void* base, int64_t i) {
    if (dtype == KDAO_BF16) {
        uint32_t u = ((uint32_t)((const uint16_t*)base)[i]) << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    if (dtype == KDAO_F64) return ((const double*)base)[i];
    return (double)((const float*)base)[i];
}

/* g and beta are fp32 unless the whole input set is double */
static int gate_dtype(int dtype) { return dtype == KDAO_F64 ? KDAO_F64 : KDAO_F32; }

static int dtype_ok(int dtype) { return dtype == KDAO_BF16 || dtype == KDAO_F32 || dtype == KDAO_F64; }

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int kdao_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * One token of the recurrence applied to the dk x ncol matrix X (row-major,
 * row = key channel).  With vt == NULL the value term is zero, i.e. X <-
 * (I - beta k k^T) Diag(alpha) X: the token's transition alone.  Work buffer
 * u has ncol entries.
 */
static void token_step(int dtype, int dk, int ncol, double* X, const void* k, int64_t koff,
                       const void* vt, int64_t voff, const void* g, int64_t goff, double beta,
                       double* u) {
    /* (1) forget: row c scaled by alpha_c = exp(g_c) */
    for (int c = 0; c < dk; ++c) {
        double a = exp(load_elt(gate_dtype(dtype), g, goff + c));
        double* row = X + (int64_t)c * ncol;
        for (int j = 0; j < ncol; ++j) row[j] *= a;
    }
    /* (2) erase: u = X^T k, delta = beta (v - u) */
    for (int j = 0; j < ncol; ++j) u[j] = 0.0;
    for (int c = 0; c < dk; ++c) {
        double kc = load_elt(dtype, k, koff + c);
        const double* row = X + (int64_t)c * ncol;
        for (int j = 0; j < ncol; ++j) u[j] += kc * row[j];
    }
    for (int j = 0; j < ncol; ++j) {
        double vj = vt ? load_elt(dtype, vt, voff + j) : 0.0;
        u[j] = beta * (vj - u[j]);
    }
    /* (3) write: X += k delta^T */
    for (int c = 0; c < dk; ++c) {
        double kc = load_elt(dtype, k, koff + c);
        double* row = X + (int64_t)c * ncol;
        for (int j = 0; j < ncol; ++j) row[j] += kc * u[j];
    }
}

/* y_t = scale * S^T q_t (gated by sigmoid(z_t) when z is given). */
static void token_output(int dtype, int dk, int dv, const double* S, const void* q, int64_t qoff,
                         const void* z, int64_t zoff, double scale, double* yrow) {
    for (int j = 0; j < dv; ++j) yrow[j] = 0.0;
    for (int c = 0; c < dk; ++c) {
        double qc = load_elt(dtype, q, qoff + c);
        const double* row = S + (int64_t)c * dv;
        for (int j = 0; j < dv; ++j) yrow[j] += qc * row[j];
    }
    for (int j = 0; j < dv; ++j) {
        double o = scale * yrow[j];
        if (z) o *= sigmoid(load_elt(dtype, z, zoff + j));
        yrow[j] = o;
    }
}

/*
 * Run the recurrence over tokens [t0, t1) of head h starting from the state
 * in S (dk x dv, overwritten with the final state).  y (layout [T, H, dv])
 * receives the outputs of those tokens when non-NULL.
 */
static void run_tokens(int dtype, int H, int dk, int dv, double scale, int64_t t0, int64_t t1,
                       int h, const void* q, const void* k, const void* v, const void* g,
                       const void* beta, const void* z, double* S, double* y, double* u) {
    for (int64_t t = t0; t < t1; ++t) {
        int64_t th = t * H + h;
        token_step(dtype, dk, dv, S, k, th * dk, v, th * dv, g, th * dk,
                   load_elt(gate_dtype(dtype), beta, th), u);
        if (y) token_output(dtype, dk, dv, S, q, th * dk, z, th * dv, scale, y + th * dv);
    }
}

/*
 * Sequential recurrence for a list of (sequence, head) chains.
 *   cu_seqlens [num_seqs+1]: token offsets of the packed sequences.
 *   chains [nchains][2] = (seq, head); NULL means every (seq, head) in order
 *     seq-major (nchains must then be num_seqs * H).
 *   state [nchains][dk][dv]: the initial state on entry, the final state on
 *     return (caller fills it, e.g. with zeros or a widened fp32 S0).
 *   y [T_total][H][dv] or NULL: the outputs of the chains' tokens.
 * Returns 0, or -1 on an invalid argument.
 */
int kdao_recurrence(int dtype, int num_seqs, const int32_t* cu_seqlens, int H, int dk, int dv,
                    double scale, const void* q, const void* k, const void* v, const void* g,
                    const void* beta, const void* z, int nchains, const int32_t* chains,
                    double* state, double* y, int nthreads) {
    if (!dtype_ok(dtype)) return -1;
    if (num_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0 || !cu_seqlens || !state) return -1;
    if (!chains && nchains != num_seqs * H) return -1;
    set_threads(nthreads);
    int bad = 0;
#pragma omp parallel
    {
        double* u = (double*)malloc(sizeof(double) * (size_t)(dv > dk ? dv : dk));
#pragma omp for schedule(dynamic, 1)
        for (int c = 0; c < nchains; ++c) {
            int n = chains ? chains[2 * c] : c / H;
            int h = chains ? chains[2 * c + 1] : c % H;
            if (n < 0 || n >= num_seqs || h < 0 || h >= H || !u) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            run_tokens(dtype, H, dk, dv, scale, cu_seqlens[n], cu_seqlens[n + 1], h, q, k, v, g,
                       beta, z, state + (int64_t)c * dk * dv, y, u);
        }
        free(u);
    }
    return bad ? -1 : 0;
}

/*
 * KCP segment pair of tokens [t0, t1) of head h: M (dk x dk) is the product
 * of the segment's transitions applied to the identity, Sloc (dk x dv) the
 * state the segment builds from zero.
 */
static void segment_pair(int dtype, int H, int dk, int dv, int64_t t0, int64_t t1, int h,
                         const void* k, const void* v, const void* g, const void* beta,
                         double* M, double* Sloc, double* u) {
    memset(M, 0, sizeof(double) * (size_t)dk * dk);
    for (int c = 0; c < dk; ++c) M[(int64_t)c * dk + c] = 1.0;
    memset(Sloc, 0, sizeof(double) * (size_t)dk * dv);
    for (int64_t t = t0; t < t1; ++t) {
        int64_t th = t * H + h;
        double b = load_elt(gate_dtype(dtype), beta, th);
        token_step(dtype, dk, dk, M, k, th * dk, NULL, 0, g, th * dk, b, u);
        token_step(dtype, dk, dv, Sloc, k, th * dk, v, th * dv, g, th * dk, b, u);
    }
}

/* (M2, S2) o (M1, S1) = (M2 M1, M2 S1 + S2); outputs may not alias inputs. */
void kdao_compose(int dk, int dv, const double* M2, const double* S2, const double* M1,
                  const double* S1, double* Mout, double* Sout) {
    for (int i = 0; i < dk; ++i) {
        for (int j = 0; j < dk; ++j) {
            double acc = 0.0;
            for (int c = 0; c < dk; ++c) acc += M2[(int64_t)i * dk + c] * M1[(int64_t)c * dk + j];
            Mout[(int64_t)i * dk + j] = acc;
        }
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int c = 0; c < dk; ++c) acc += M2[(int64_t)i * dk + c] * S1[(int64_t)c * dv + j];
            Sout[(int64_t)i * dv + j] = acc + S2[(int64_t)i * dv + j];
        }
    }
}

/*
 * KCP over one packed sequence of T tokens split at seg_bounds[0..nseg]
 * (seg_bounds[0] = 0, seg_bounds[nseg] = T, non-decreasing).
 *   S0 [H][dk][dv] or NULL (zeros): state before the first segment.
 *   pairs_M [nseg][H][dk][dk], pairs_S [nseg][H][dk][dv]: optional outputs.
 *   starts [nseg][H][dk][dv]: optional, the state entering each segment.
 *   final [H][dk][dv]: the state after the last segment (required).
 *   y [T][H][dv] or NULL: outputs, recomputed per segment from its start.
 * Phase 1 (pairs) and phase 3 (outputs) run in parallel over (segment, head);
 * phase 2 folds the pairs in segment order, S <- M_i S + Sloc_i.
 */
int kdao_kcp(int dtype, int64_t T, int H, int dk, int dv, double scale, const void* q,
             const void* k, const void* v, const void* g, const void* beta, const void* z,
             int nseg, const int64_t* seg_bounds, const double* S0, double* pairs_M,
             double* pairs_S, double* starts, double* final_state, double* y, int nthreads) {
    if (!dtype_ok(dtype)) return -1;
    if (nseg <= 0 || H <= 0 || dk <= 0 || dv <= 0 || !seg_bounds || !final_state) return -1;
    if (seg_bounds[0] != 0 || seg_bounds[nseg] != T) return -1;
    for (int i = 0; i < nseg; ++i)
        if (seg_bounds[i + 1] < seg_bounds[i]) return -1;
    set_threads(nthreads);
    const int64_t mk = (int64_t)dk * dk, sk = (int64_t)dk * dv;
    double* M = pairs_M ? pairs_M : (double*)malloc(sizeof(double) * (size_t)(nseg * H * mk));
    double* L = pairs_S ? pairs_S : (double*)malloc(sizeof(double) * (size_t)(nseg * H * sk));
    double* St = starts ? starts : (double*)malloc(sizeof(double) * (size_t)(nseg * H * sk));
    int bad = (!M || !L || !St);
    if (!bad) {
        /* phase 1: pairs */
#pragma omp parallel
        {
            double* u = (double*)malloc(sizeof(double) * (size_t)(dv > dk ? dv : dk));
#pragma omp for schedule(dynamic, 1)
            for (int i = 0; i < nseg * H; ++i) {
                int s = i / H, h = i % H;
                segment_pair(dtype, H, dk, dv, seg_bounds[s], seg_bounds[s + 1], h, k, v, g, beta,
                             M + (int64_t)i * mk, L + (int64_t)i * sk, u);
            }
            free(u);
        }
        /* phase 2: fold pairs in order, per head */
#pragma omp parallel for schedule(static, 1)
        for (int h = 0; h < H; ++h) {
            double* cur = (double*)malloc(sizeof(double) * (size_t)sk);
            double* nxt = (double*)malloc(sizeof(double) * (size_t)sk);
            if (S0) memcpy(cur, S0 + (int64_t)h * sk, sizeof(double) * (size_t)sk);
            else memset(cur, 0, sizeof(double) * (size_t)sk);
            for (int s = 0; s < nseg; ++s) {
                int64_t i = (int64_t)s * H + h;
                memcpy(St + i * sk, cur, sizeof(double) * (size_t)sk);
                const double* Mi = M + i * mk;
                const double* Li = L + i * sk;
                for (int r = 0; r < dk; ++r)
                    for (int j = 0; j < dv; ++j) {
                        double acc = 0.0;
                        for (int c = 0; c < dk; ++c) acc += Mi[(int64_t)r * dk + c] * cur[(int64_t)c * dv + j];
                        nxt[(int64_t)r * dv + j] = acc + Li[(int64_t)r * dv + j];
                    }
                double* tmp = cur; cur = nxt; nxt = tmp;
            }
            memcpy(final_state + (int64_t)h * sk, cur, sizeof(double) * (size_t)sk);
            free(cur);
            free(nxt);
        }
        /* phase 3: outputs of each segment from its entering state */
        if (y) {
#pragma omp parallel
            {
                double* u = (double*)malloc(sizeof(double) * (size_t)(dv > dk ? dv : dk));
                double* S = (double*)malloc(sizeof(double) * (size_t)sk);
#pragma omp for schedule(dynamic, 1)
                for (int i = 0; i < nseg * H; ++i) {
                    int s = i / H, h = i % H;
                    memcpy(S, St + (int64_t)i * sk, sizeof(double) * (size_t)sk);
                    run_tokens(dtype, H, dk, dv, scale, seg_bounds[s], seg_bounds[s + 1], h, q, k, v,
                               g, beta, z, S, y, u);
                }
                free(S);
                free(u);
            }
        }
    }
    if (!pairs_M) free(M);
    if (!pairs_S) free(L);
    if (!starts) free(St);
    return bad ? -1 : 0;
}
