/*
 * The oracle: a plain, slow, single-threaded CPU definition of MoE token
 * dispatch and combine, written from the problem statement. It is TEST
 * INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load it; the GPU library shares no code, header, table or
 * helper with it.
 *
 * Sources (page title, section):
 *   [P1] NeMo AutoModel API page "nemo_automodel.components.moe.uccl_ep.buffer":
 *        Buffer.get_dispatch_layout, Buffer.dispatch (topk_idx, expert_alignment,
 *        num_tokens_per_rank, is_token_in_rank, num_tokens_per_expert),
 *        Buffer.combine, Buffer.low_latency_dispatch (receive layout
 *        [num_local_experts, num_ranks * num_max_dispatch_tokens_per_rank, hidden]),
 *        Buffer.low_latency_combine (reduce with weights, -1 ids allowed).
 *   [P3] "dots-infra/ultraep architecture": Overview (plan replicas, expand the
 *        routing before the experts), GPU operations (Load computation,
 *        Placement planning, Routing expansion).
 *
 * Readings of points the pages leave open (each is listed with its reason in
 * the design notes of this repository):
 *   - a (token, k) pair with id -1 is not counted and gets slot -1;
 *   - ids >= E or < -1 are skipped and set status bit 1;
 *   - rows inside an expert are ordered by pair index t*K+k (stable);
 *   - per-expert row counts are rounded up to the expert alignment A;
 *   - combine is weighted (weights NULL = all ones), summed in ascending k;
 *   - bf16 rounding is round-to-nearest-even, NaN -> 0x7FC0;
 *   - low-latency row of the j-th pair of expert e sent by rank s is
 *     (e*R + s)*M + j; pairs with j >= M are dropped and set status bit 2;
 *   - replica plan: the C most loaded experts (ties -> lower id) get one extra
 *     physical replica; a pair of token t uses replica (t mod count);
 *   - normal mode sends one row per (token, rank), tokens ascending within a
 *     rank; received expert ids are rank-local (-1 for other ranks' experts);
 *   - FP8: one scale per 128 channels, max(amax, 1e-4) / 448; codes are the
 *     nearest E4M3 of x / scale (ties to even, saturating at 448, sign kept);
 *     round_scale rounds the scale up to a power of two; UE8M0 packs group
 *     4w+b into byte b of word w; low-latency scales are stored [E][G][R*M].
 *
 * Arithmetic: combine is provided twice -- in double (the exact definition up
 * to rounding of a K-term sum), and in float with every product and every sum
 * rounded to float, in ascending k, no fused multiply-add (build with
 * -ffp-contract=off).
 *
 * Mutants: building with -DORACLE_MUTANT=n plants one known mistake; the test
 * suite uses those builds to show that its pins catch each of them. A normal
 * build has ORACLE_MUTANT undefined.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* A second build with -fopenmp (used only to time the CPU baseline on all of
 * the host's cores) splits the token loops of dispatch and combine over
 * threads. Each token is still handled by one thread in the same order, so
 * every result is the same bit for bit; the normal build ignores this. */
#ifdef _OPENMP
#include <omp.h>
#define FOR_TOKENS _Pragma("omp parallel for schedule(static) reduction(|:st)")
#define TOKEN_REGION _Pragma("omp parallel")
#define TOKEN_SPLIT _Pragma("omp for schedule(static) reduction(|:st)")
#else
#define FOR_TOKENS
#define TOKEN_REGION
#define TOKEN_SPLIT
#endif

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

#define ST_BAD_EXPERT 1
#define ST_LL_OVERFLOW 2
#define ST_BAD_SLOT 4
#define ST_BAD_REPLICA 8

int oracle_mutant(void) { return ORACLE_MUTANT; }

/* Threads the token loops may use: sets the count when n > 0, returns the
 * count in force (1 in the normal build). */
int oracle_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* bf16 <-> f32                                                        */
/* ------------------------------------------------------------------ */

static float bf16_to_f32(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round a float to the nearest bf16, ties to even; any NaN becomes 0x7FC0. */
static uint16_t f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    uint32_t lsb = (u >> 16) & 1u;
#if ORACLE_MUTANT == 9
    lsb = 0; /* mutant: round half up instead of half to even */
#endif
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

void oracle_bf16_from_f32(const float *in, uint16_t *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16(in[i]);
}

/* ------------------------------------------------------------------ */
/* Layout: counts, per-rank token sets, aligned offsets, stable slots  */
/* ------------------------------------------------------------------ */

static int valid_id(int64_t e, int32_t E) { return e >= 0 && e < E; }

/* Count (token, expert) pairs per expert and mark which ranks each token
 * reaches. [P1] Buffer.get_dispatch_layout / Buffer.dispatch:
 * num_tokens_per_expert, is_token_in_rank, num_tokens_per_rank. */
static void count_pairs(int64_t T, int32_t K, int32_t E, int32_t R, const int64_t *idx,
                        int32_t *count, int32_t *rank_token_count, uint8_t *in_rank,
                        int32_t *status) {
    int32_t L = E / R;
    for (int32_t e = 0; e < E; ++e) count[e] = 0;
    uint8_t *mark = (uint8_t *)calloc((size_t)(T > 0 ? T : 1) * (size_t)R, 1);
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int64_t e = idx[t * K + k];
            if (e == -1) continue;
            if (!valid_id(e, E)) {
                if (status) *status |= ST_BAD_EXPERT;
                continue;
            }
            count[e] += 1;
            mark[t * R + e / L] = 1;
        }
    }
    if (rank_token_count) {
        for (int32_t r = 0; r < R; ++r) {
            int32_t n = 0;
            for (int64_t t = 0; t < T; ++t) n += mark[t * R + r];
#if ORACLE_MUTANT == 5
            /* mutant: count pairs per rank instead of distinct tokens */
            n = 0;
            for (int32_t e = r * L; e < (r + 1) * L; ++e) n += count[e];
#endif
            rank_token_count[r] = n;
        }
    }
    if (in_rank) memcpy(in_rank, mark, (size_t)T * (size_t)R);
    free(mark);
}

/* Contiguous layout. offset[0] = 0, offset[e+1] = offset[e] + ceil(count[e]/A)*A
 * ([P1] Buffer.dispatch, expert_alignment). The j-th pair of expert e in
 * row-major (t, k) order takes row offset[e] + j. row_src[row] = t*K + k, and
 * -1 on alignment padding rows in [0, offset[E]). */
int oracle_layout(int64_t T, int32_t K, int32_t E, int32_t R, int32_t A, const int64_t *idx,
                  int32_t *count, int32_t *offset, int32_t *rank_token_count, uint8_t *in_rank,
                  int32_t *slot, int32_t *row_src, int64_t row_src_len, int32_t *status) {
    if (T < 0 || K < 1 || E < 1 || R < 1 || E % R != 0 || A < 1) return -2;
    count_pairs(T, K, E, R, idx, count, rank_token_count, in_rank, status);

    offset[0] = 0;
    for (int32_t e = 0; e < E; ++e) {
        int32_t c = count[e];
        int32_t padded = (c + A - 1) / A * A;
#if ORACLE_MUTANT == 1
        padded = c; /* mutant: alignment dropped */
#endif
        offset[e + 1] = offset[e] + padded;
    }
    if (row_src) {
        if (row_src_len < offset[E]) return -3;
        for (int32_t r = 0; r < offset[E]; ++r) row_src[r] = -1;
    }

    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    for (int32_t e = 0; e < E; ++e) cursor[e] = offset[e];
#if ORACLE_MUTANT == 2
    /* mutant: pairs visited in column-major (k, t) order */
    for (int32_t k = 0; k < K; ++k) {
        for (int64_t t = 0; t < T; ++t) {
#else
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k) {
#endif
            int64_t p = t * K + k;
            int64_t e = idx[p];
            if (!valid_id(e, E)) {
                slot[p] = -1;
                continue;
            }
            int32_t row = cursor[e]++;
            slot[p] = row;
            if (row_src) row_src[row] = (int32_t)p;
        }
    }
    free(cursor);
    return 0;
}

/* Low-latency padded layout ([P1] Buffer.low_latency_dispatch: each rank
 * receives [num_local_experts, num_ranks * M, hidden]; taken together the R
 * receive buffers are [E, R*M, hidden]). This rank is source s; its j-th pair
 * for expert e lands in row (e*R + s)*M + j. recv_count[e] = pairs that fit
 * (min(count, M)); pairs with j >= M are dropped with status bit 2.
 * row_src (optional) is [E*M]: the pair held in stripe row j of expert e, or -1. */
int oracle_ll_layout(int64_t T, int32_t K, int32_t E, int32_t R, int32_t M, int32_t s,
                     const int64_t *idx, int32_t *recv_count, int32_t *rank_token_count,
                     uint8_t *in_rank, int32_t *slot, int32_t *row_src, int32_t *status) {
    if (T < 0 || K < 1 || E < 1 || R < 1 || E % R != 0 || M < 1) return -2;
    if (T > M || s < 0 || s >= R) return -4;
    int32_t *count = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    count_pairs(T, K, E, R, idx, count, rank_token_count, in_rank, status);
    if (row_src)
        for (int64_t r = 0; r < (int64_t)E * M; ++r) row_src[r] = -1;
    int32_t *j = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int64_t p = t * K + k;
            int64_t e = idx[p];
            if (!valid_id(e, E)) {
                slot[p] = -1;
                continue;
            }
            int32_t jj = j[e]++;
            if (jj >= M) {
                slot[p] = -1;
                if (status) *status |= ST_LL_OVERFLOW;
                continue;
            }
            int64_t row = ((int64_t)e * R + s) * M + jj;
#if ORACLE_MUTANT == 6
            row = (int64_t)e * R * M + jj; /* mutant: source stripe dropped */
#endif
            slot[p] = (int32_t)row;
            if (row_src) row_src[(int64_t)e * M + jj] = (int32_t)p;
        }
    }
    for (int32_t e = 0; e < E; ++e) recv_count[e] = count[e] < M ? count[e] : M;
    free(j);
    free(count);
    return 0;
}

/* Per-expert load over the batch ([P3] GPU operations: Load computation). */
int oracle_expert_load(int64_t T, int32_t K, int32_t E, const int64_t *idx, int32_t *load,
                       int32_t *status) {
    if (T < 0 || K < 1 || E < 1) return -2;
    for (int32_t e = 0; e < E; ++e) load[e] = 0;
    for (int64_t p = 0; p < T * K; ++p) {
        int64_t e = idx[p];
        if (e == -1) continue;
        if (!valid_id(e, E)) {
            if (status) *status |= ST_BAD_EXPERT;
            continue;
        }
        load[e] += 1;
    }
    return 0;
}

/* Normal-mode layout, one row per (token, rank) ([P1] Buffer.dispatch:
 * num_tokens_per_rank, is_token_in_rank, topk_idx, topk_weights,
 * expert_alignment; its returns recv_topk_idx, recv_topk_weights and the
 * per-expert receive counts; Buffer.combine adds the rows back without
 * weights). Each token is sent once to every rank that hosts one of its
 * experts. The R ranks' receive buffers are one buffer: rank r owns rows
 * [rank_offset[r], rank_offset[r+1]), its tokens in ascending t. For the row of
 * (t, r): rank_slot[t*R + r] = row (-1 if t does not reach r),
 * recv_src[row] = t, recv_idx[row*K + k] = the rank-local id e - r*L of the
 * k-th expert if it lives on r, else -1, and recv_w[row*K + k] = w[t,k] there,
 * else 0 (w may be NULL: then recv_w is not written). recv_expert_count[e] =
 * ceil(count[e] / A) * A, the receive count of expert e aligned to A. */
int oracle_rank_layout(int64_t T, int32_t K, int32_t E, int32_t R, int32_t A, const int64_t *idx,
                       const float *w, int32_t *rank_slot, int32_t *rank_offset,
                       int32_t *recv_src, int64_t *recv_idx, float *recv_w,
                       int32_t *recv_expert_count, int32_t *status) {
    if (T < 0 || K < 1 || E < 1 || R < 1 || E % R != 0 || A < 1) return -2;
    const int32_t L = E / R;
    int32_t *count = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    int32_t *rtc = (int32_t *)calloc((size_t)R, sizeof(int32_t));
    uint8_t *in_rank = (uint8_t *)calloc((size_t)(T * R > 0 ? T * R : 1), 1);
    count_pairs(T, K, E, R, idx, count, NULL, in_rank, status);
    for (int32_t r = 0; r < R; ++r)
        for (int64_t t = 0; t < T; ++t) rtc[r] += in_rank[t * R + r];
    rank_offset[0] = 0;
    for (int32_t r = 0; r < R; ++r) rank_offset[r + 1] = rank_offset[r] + rtc[r];
    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)R);
    for (int32_t r = 0; r < R; ++r) cursor[r] = rank_offset[r];
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t r = 0; r < R; ++r) {
            if (!in_rank[t * R + r]) {
                rank_slot[t * R + r] = -1;
                continue;
            }
#if ORACLE_MUTANT == 18
            int32_t row = rank_offset[r + 1] - 1 - (cursor[r]++ - rank_offset[r]); /* mutant: tokens descending */
#else
            int32_t row = cursor[r]++;
#endif
            rank_slot[t * R + r] = row;
            recv_src[row] = (int32_t)t;
            for (int32_t k = 0; k < K; ++k) {
                int64_t e = idx[t * K + k];
                int local = valid_id(e, E) && e / L == r;
#if ORACLE_MUTANT == 19
                recv_idx[(int64_t)row * K + k] = local ? e : -1; /* mutant: global id */
#else
                recv_idx[(int64_t)row * K + k] = local ? e - (int64_t)r * L : -1;
#endif
                if (w) recv_w[(int64_t)row * K + k] = local ? w[t * K + k] : 0.0f;
            }
        }
    }
    for (int32_t e = 0; e < E; ++e) recv_expert_count[e] = (count[e] + A - 1) / A * A;
    free(cursor);
    free(in_rank);
    free(rtc);
    free(count);
    return 0;
}

/* Buffer.combine's weight output: the received top-k weights summed back per
 * token over the ranks it reached, ascending r, in float:
 * out_w[t,k] = sum_r recv_w[rank_slot[t,r]*K + k]. */
int oracle_combine_rank_weights(int64_t T, int32_t K, int32_t R, const int32_t *rank_slot,
                                const float *recv_w, int64_t rows, float *out_w,
                                int32_t *status) {
    for (int64_t t = 0; t < T; ++t)
        for (int32_t k = 0; k < K; ++k) {
            float acc = 0.0f;
            for (int32_t r = 0; r < R; ++r) {
                int32_t row = rank_slot[t * R + r];
                if (row == -1) continue;
                if (row < -1 || row >= rows) {
                    if (status) *status |= ST_BAD_SLOT;
                    continue;
                }
                acc = acc + recv_w[(int64_t)row * K + k];
            }
            out_w[t * K + k] = acc;
        }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Dispatch: recv[slot[t,k]] = x[t]                                    */
/* ------------------------------------------------------------------ */

/* [P1] Buffer.dispatch / Buffer.low_latency_dispatch: each selected (token,
 * expert) pair sends the token's hidden row; here the row is copied bit for
 * bit into its slot of the receive buffer. */
int oracle_dispatch(int64_t T, int32_t H, int32_t K, const uint16_t *x, const int32_t *slot,
                    uint16_t *recv, int64_t rows, int32_t *status) {
    int32_t st = 0;
    FOR_TOKENS
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int32_t r = slot[t * K + k];
            if (r == -1) continue;
            if (r < -1 || r >= rows) {
                st |= ST_BAD_SLOT;
                continue;
            }
            memcpy(recv + (int64_t)r * H, x + t * (int64_t)H, sizeof(uint16_t) * (size_t)H);
        }
    }
    if (status) *status |= st;
    return 0;
}

/* ------------------------------------------------------------------ */
/* Combine: out[t] = sum_k w[t,k] * y[slot[t,k]]                       */
/* ------------------------------------------------------------------ */

static int32_t k_of(int32_t k, int32_t K) {
#if ORACLE_MUTANT == 4
    return K - 1 - k; /* mutant: weight index reversed */
#else
    (void)K;
    return k;
#endif
}

static int32_t k_end(int32_t K) {
#if ORACLE_MUTANT == 3
    return K - 1; /* mutant: last top-k term dropped */
#else
    return K;
#endif
}

/* [P1] Buffer.low_latency_combine (reduce with weights) and Buffer.combine:
 * the expert outputs of a token's selected pairs are summed, each times its
 * top-k weight, back into the token's row. Exact definition in double. */
int oracle_combine_f64(int64_t T, int32_t H, int32_t K, const uint16_t *y, int64_t rows,
                       const int32_t *slot, const float *w, double *out, int32_t *status) {
    int32_t st = 0;
    FOR_TOKENS
    for (int64_t t = 0; t < T; ++t) {
        double *o = out + t * (int64_t)H;
        for (int32_t h = 0; h < H; ++h) o[h] = 0.0;
        for (int32_t k = 0; k < k_end(K); ++k) {
            int32_t r = slot[t * K + k];
            if (r == -1) continue;
            if (r < -1 || r >= rows) {
                st |= ST_BAD_SLOT;
                continue;
            }
            double wk = w ? (double)w[t * K + k_of(k, K)] : 1.0;
            const uint16_t *yr = y + (int64_t)r * H;
            for (int32_t h = 0; h < H; ++h) o[h] += wk * (double)bf16_to_f32(yr[h]);
        }
    }
    if (status) *status |= st;
    return 0;
}

/* Same sum in float: ascending k, each product and each sum rounded to float,
 * starting from +0. Also returns the bf16 rounding of the float sum. */
int oracle_combine_f32(int64_t T, int32_t H, int32_t K, const uint16_t *y, int64_t rows,
                       const int32_t *slot, const float *w, float *out_f32, uint16_t *out_bf16,
                       int32_t *status) {
    int32_t st = 0;
    TOKEN_REGION
    {
        float *acc = (float *)malloc(sizeof(float) * (size_t)(H > 0 ? H : 1));
        TOKEN_SPLIT
        for (int64_t t = 0; t < T; ++t) {
            for (int32_t h = 0; h < H; ++h) acc[h] = 0.0f;
            for (int32_t k = 0; k < k_end(K); ++k) {
                int32_t r = slot[t * K + k];
                if (r == -1) continue;
                if (r < -1 || r >= rows) {
                    st |= ST_BAD_SLOT;
                    continue;
                }
                float wk = w ? w[t * K + k_of(k, K)] : 1.0f;
                const uint16_t *yr = y + (int64_t)r * H;
                for (int32_t h = 0; h < H; ++h) {
                    float prod = wk * bf16_to_f32(yr[h]);
                    acc[h] = acc[h] + prod;
                }
            }
            for (int32_t h = 0; h < H; ++h) {
                if (out_f32) out_f32[t * (int64_t)H + h] = acc[h];
                if (out_bf16) out_bf16[t * (int64_t)H + h] = f32_to_bf16(acc[h]);
            }
        }
        free(acc);
    }
    if (status) *status |= st;
    return 0;
}

/* Combine with an active-rank mask ([P1] Buffer.low_latency_combine on a
 * buffer whose ranks can be masked; the combine checks each destination
 * rank's mask entry, as the NIXL EP notes describe for the combine loops).
 * A pair whose expert lives on a masked rank (mask[e / L] != 0, L = E / R)
 * contributes nothing, as if its expert output never arrived; otherwise the
 * sum is oracle_combine_f32's (ascending k, float, no fused multiply-add). */
int oracle_combine_masked_f32(int64_t T, int32_t H, int32_t K, const uint16_t *y, int64_t rows,
                              const int32_t *slot, const int64_t *idx, int32_t E, int32_t R,
                              const int32_t *mask, const float *w, float *out_f32,
                              uint16_t *out_bf16, int32_t *status) {
    if (E < 1 || R < 1 || E % R != 0) return -2;
    const int32_t L = E / R;
    int32_t *s2 = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T * K > 0 ? T * K : 1));
    for (int64_t p = 0; p < T * K; ++p) {
        int64_t e = idx[p];
        int masked = valid_id(e, E) && mask[e / L] != 0;
#if ORACLE_MUTANT == 17
        masked = valid_id(e, E) && mask[e % R] != 0; /* mutant: rank taken as e mod R */
#endif
        s2[p] = masked ? -1 : slot[p];
    }
    int rc = oracle_combine_f32(T, H, K, y, rows, s2, w, out_f32, out_bf16, status);
    free(s2);
    return rc;
}

/* [P1] Buffer.low_latency_dispatch, cumulative_local_expert_recv_stats: a
 * running per-expert count of received tokens, stats[e] += recv_count[e]
 * for every dispatch (the union of the ranks' [L] tensors: rank r's local
 * expert l is entry r*L + l). */
void oracle_accumulate_recv_stats(int32_t E, const int32_t *recv_count, int32_t *stats) {
    for (int32_t e = 0; e < E; ++e) stats[e] += recv_count[e];
}

/* ------------------------------------------------------------------ */
/* Replica plan and routing expansion ([P3] Overview; GPU operations:  */
/* Placement planning, Routing expansion)                              */
/* ------------------------------------------------------------------ */

static const int32_t *g_load;
static int cmp_hot(const void *a, const void *b) {
    int32_t ea = *(const int32_t *)a, eb = *(const int32_t *)b;
    if (g_load[ea] != g_load[eb]) {
#if ORACLE_MUTANT == 7
        return g_load[ea] < g_load[eb] ? -1 : 1; /* mutant: coldest first */
#else
        return g_load[ea] > g_load[eb] ? -1 : 1;
#endif
    }
    return ea < eb ? -1 : (ea > eb ? 1 : 0);
}

/* The C most loaded logical experts (load descending, ties -> lower id) get a
 * second physical replica. Physical numbering: every rank r holds
 * L' = L + C/R physical slots; slot r*L' + l (l < L) is the primary of logical
 * expert r*L + l, and the i-th hottest expert's replica is slot
 * (i mod R)*L' + L + i/R. replica_phys is [E][2] (-1 where there is no second
 * replica); phys_to_logical is [E + C]. */
int oracle_plan_replicas(int32_t E, int32_t R, int32_t C, const int32_t *load,
                         int32_t *replica_count, int32_t *replica_phys,
                         int32_t *phys_to_logical) {
    if (E < 1 || R < 1 || E % R != 0 || C < 0 || C > E || C % R != 0) return -2;
    int32_t L = E / R, Lp = L + C / R;
    int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    for (int32_t e = 0; e < E; ++e) order[e] = e;
    g_load = load;
    qsort(order, (size_t)E, sizeof(int32_t), cmp_hot);
    for (int32_t e = 0; e < E; ++e) {
        int32_t prim = (e / L) * Lp + e % L;
        replica_count[e] = 1;
        replica_phys[2 * e] = prim;
        replica_phys[2 * e + 1] = -1;
        phys_to_logical[prim] = e;
    }
    for (int32_t i = 0; i < C; ++i) {
        int32_t e = order[i];
        int32_t rep = (i % R) * Lp + L + i / R;
        replica_count[e] = 2;
        replica_phys[2 * e + 1] = rep;
        phys_to_logical[rep] = e;
    }
    free(order);
    return 0;
}

/* Replica weight sync ([P3] Overview: replicas get synchronized weights
 * before expert execution; GPU operations: Replica weight sync). The physical
 * expert buffer w [E_phys][S] holds every logical expert's master weights in
 * its primary slot; each expert with a second replica gets a bit copy of them
 * in the replica slot: w[replica_phys[2e+1]] = w[replica_phys[2e]]. */
int oracle_replica_weight_sync(int32_t E, int64_t S, const int32_t *replica_count,
                               const int32_t *replica_phys, int32_t E_phys, uint16_t *w) {
    for (int32_t e = 0; e < E; ++e) {
        if (replica_count[e] != 2) continue;
        int32_t prim = replica_phys[2 * e], rep = replica_phys[2 * e + 1];
        if (prim < 0 || prim >= E_phys || rep < 0 || rep >= E_phys) return -3;
        memcpy(w + (int64_t)rep * S, w + (int64_t)prim * S, sizeof(uint16_t) * (size_t)S);
    }
    return 0;
}

/* Replica gradient reduction ([P3] Overview: replica gradients are reduced
 * during backward; GPU operations: Replica gradient reduction). g [E_phys][S]
 * f32 holds one gradient per physical expert; each replicated expert's master
 * gradient, kept in its primary slot, becomes primary + replica, one float add
 * per element: g[prim] = g[prim] + g[rep]. */
int oracle_replica_grad_reduce(int32_t E, int64_t S, const int32_t *replica_count,
                               const int32_t *replica_phys, int32_t E_phys, float *g) {
    for (int32_t e = 0; e < E; ++e) {
        if (replica_count[e] != 2) continue;
        int32_t prim = replica_phys[2 * e], rep = replica_phys[2 * e + 1];
        if (prim < 0 || prim >= E_phys || rep < 0 || rep >= E_phys) return -3;
        float *gp = g + (int64_t)prim * S;
        const float *gr = g + (int64_t)rep * S;
        for (int64_t i = 0; i < S; ++i) {
#if ORACLE_MUTANT == 20
            gp[i] = gr[i]; /* mutant: the replica gradient replaces the master */
#else
            gp[i] = gp[i] + gr[i];
#endif
        }
    }
    return 0;
}

/* Expand logical routing to physical routing: the pair (t, k) on logical
 * expert e goes to replica (t mod replica_count[e]) of e; -1 stays -1. */
int oracle_reroute(int64_t T, int32_t K, int32_t E, const int64_t *idx,
                   const int32_t *replica_count, const int32_t *replica_phys, int32_t E_phys,
                   int64_t *phys_idx, int32_t *status) {
    if (T < 0 || K < 1 || E < 1) return -2;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int64_t p = t * K + k;
            int64_t e = idx[p];
            if (e == -1) {
                phys_idx[p] = -1;
                continue;
            }
            if (!valid_id(e, E)) {
                if (status) *status |= ST_BAD_EXPERT;
                phys_idx[p] = -1;
                continue;
            }
            int32_t c = replica_count[e];
            if (c < 1 || c > 2) {
                if (status) *status |= ST_BAD_REPLICA;
                phys_idx[p] = -1;
                continue;
            }
            int32_t which = (int32_t)(t % c);
#if ORACLE_MUTANT == 8
            which = (int32_t)(k % c); /* mutant: replica chosen by k instead of t */
#endif
            int32_t ph = replica_phys[2 * e + which];
            if (ph < 0 || ph >= E_phys) {
                if (status) *status |= ST_BAD_REPLICA;
                phys_idx[p] = -1;
                continue;
            }
            phys_idx[p] = ph;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* FP8 rows with per-128-channel scales ([P1] Buffer.low_latency_dispatch: */
/* use_fp8, round_scale, use_ue8m0, and the returned scale tensors;     */
/* Buffer.dispatch: x given as an (e4m3 rows, float scales) tuple)     */
/* ------------------------------------------------------------------ */

#define FP8_GROUP 128       /* channels per scale ([P1]: hidden // 128 scales) */
#define FP8_ROUND_SCALE 1   /* scales rounded up to a power of two */
#define FP8_UE8M0 2         /* scales also emitted as packed exponent bytes */
#define FP8_SCALE_ROWS 4    /* receive-side scales row-major instead of column-major */
#define FP8_AMAX_FLOOR 1e-4f /* reading: a group's amax is taken as at least this */

/* Value of an E4M3 ("fn" variant) code, from the format's definition (OCP 8-bit
 * floating point specification, E4M3): 1 sign bit, 4 exponent bits with bias
 * 7, 3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2^-6; the two
 * codes S.1111.111 are NaN and there is no infinity, so 448 is the largest
 * finite magnitude. */
double oracle_e4m3_value(uint8_t c) {
    int s = c >> 7, ef = (c >> 3) & 15, m = c & 7;
    double v;
    if (ef == 15 && m == 7) return NAN;
    if (ef == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, ef - 7);
    return s ? -v : v;
}

/* Magnitudes of codes 0x00 .. 0x7E; the codes are ordered by magnitude. */
static double g_e4m3_mag[127];
static int g_e4m3_ready;
static void e4m3_table(void) {
    if (g_e4m3_ready) return;
    for (int c = 0; c < 127; ++c) g_e4m3_mag[c] = oracle_e4m3_value((uint8_t)c);
    g_e4m3_ready = 1;
}

/* Nearest E4M3 code to a finite float, ties to the even code (even mantissa),
 * magnitudes of 448 and above saturate to 448 (reading: the format has no
 * infinity). The sign is kept, also for results that round to zero. */
static uint8_t e4m3_from_f32(float v) {
    e4m3_table();
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= 448.0) return sign | 0x7E;
    /* lo = largest code whose magnitude is <= a (binary search) */
    int lo = 0, hi = 126;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (g_e4m3_mag[mid] <= a) lo = mid; else hi = mid - 1;
    }
    if (g_e4m3_mag[lo] == a) return sign | (uint8_t)lo;
    double dlo = a - g_e4m3_mag[lo], dhi = g_e4m3_mag[lo + 1] - a;
    int c;
    if (dlo < dhi)
        c = lo;
    else if (dhi < dlo)
        c = lo + 1;
    else
#if ORACLE_MUTANT == 10
        c = lo + 1; /* mutant: ties away from zero */
#else
        c = (lo & 1) ? lo + 1 : lo;
#endif
    return sign | (uint8_t)c;
}

void oracle_e4m3_from_f32(const float *in, uint8_t *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_from_f32(in[i]);
}

/* Smallest power of two >= s, for a positive normal float s (round_scale). */
static float pow2_ceil(float s) {
    int e;
    float m = frexpf(s, &e); /* s = m * 2^e, m in [0.5, 1) */
#if ORACLE_MUTANT == 12
    (void)m;
    return ldexpf(1.0f, e - 1); /* mutant: rounds the scale down */
#else
    return m == 0.5f ? s : ldexpf(1.0f, e);
#endif
}

/* Per-token cast of bf16 rows to E4M3 with one float scale per 128 channels:
 *   amax  = max |x| over the group (at least FP8_AMAX_FLOOR),
 *   scale = amax / 448 in float (FP8_ROUND_SCALE: then rounded up to a power
 *           of two),
 *   code  = nearest E4M3 (ties to even) of x / scale, divided in float,
 * so the group's largest magnitude maps to the largest finite code and
 * x ~= value(code) * scale. q is [T, H], scale [T, H/128] row-major. With
 * FP8_UE8M0 (needs FP8_ROUND_SCALE and H % 512 == 0) ue8m0 [T, H/512] also
 * receives the scales' biased exponents (scale = 2^(byte - 127)), four groups
 * per int32, group 4w + b in byte b (bits 8b .. 8b+7) of word w. */
int oracle_quantize_fp8(int64_t T, int32_t H, const uint16_t *x, int32_t flags, uint8_t *q,
                        float *scale, int32_t *ue8m0) {
    if (T < 0 || H < FP8_GROUP || H % FP8_GROUP != 0) return -2;
    if ((flags & FP8_UE8M0) && (!(flags & FP8_ROUND_SCALE) || H % (4 * FP8_GROUP) != 0 || !ue8m0))
        return -2;
    const int32_t G = H / FP8_GROUP;
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t *xr = x + t * (int64_t)H;
#if ORACLE_MUTANT == 15
        float row_amax = 0.0f; /* mutant: one amax for the whole row */
        for (int32_t h = 0; h < H; ++h) {
            float a = fabsf(bf16_to_f32(xr[h]));
            if (a > row_amax) row_amax = a;
        }
#endif
        for (int32_t g = 0; g < G; ++g) {
            float amax = 0.0f;
            for (int32_t c = 0; c < FP8_GROUP; ++c) {
                float a = fabsf(bf16_to_f32(xr[g * FP8_GROUP + c]));
                if (a > amax) amax = a;
            }
#if ORACLE_MUTANT == 15
            amax = row_amax;
#endif
            if (amax < FP8_AMAX_FLOOR) amax = FP8_AMAX_FLOOR;
#if ORACLE_MUTANT == 11
            float s = amax / 240.0f; /* mutant: the other FP8 variant's maximum */
#else
            float s = amax / 448.0f;
#endif
            if (flags & FP8_ROUND_SCALE) s = pow2_ceil(s);
            scale[t * G + g] = s;
            for (int32_t c = 0; c < FP8_GROUP; ++c) {
                float v = bf16_to_f32(xr[g * FP8_GROUP + c]) / s;
                q[t * (int64_t)H + g * FP8_GROUP + c] = e4m3_from_f32(v);
            }
            if (flags & FP8_UE8M0) {
                int e;
                (void)frexpf(s, &e); /* s = 0.5 * 2^e exactly */
                uint32_t byte = (uint32_t)(e - 1 + 127);
                int32_t w = g / 4;
#if ORACLE_MUTANT == 14
                int32_t b = 3 - g % 4; /* mutant: bytes packed high to low */
#else
                int32_t b = g % 4;
#endif
                uint32_t *word = (uint32_t *)&ue8m0[t * (G / 4) + w];
                if (g % 4 == 0) *word = 0;
                *word |= byte << (8 * b);
            }
        }
    }
    return 0;
}

/* Low-latency dispatch with the FP8 cast ([P1] Buffer.low_latency_dispatch,
 * use_fp8): every valid pair's row of codes goes to its padded row
 * slot = (e*R + s)*M + j of recv_q [E*R*M, H], and the token's scales go to
 * the same row of the scale tensor, whose last two dimensions are
 * column-major ([P1] returns): recv_scale is stored as [E][H/128][R*M], so
 * the scale of group g for row i of expert e's R*M rows sits at
 * (e*(H/128) + g)*(R*M) + i; with FP8_UE8M0 the packed words go to
 * recv_ue8m0 stored as [E][H/512][R*M] the same way. With FP8_SCALE_ROWS
 * (an option of this implementation, not of the page) both are row-major
 * instead: the scales of receive row r at r*(H/128) + g (UE8M0 words at
 * r*(H/512) + w). Rows no pair maps to are left untouched. */
int oracle_ll_dispatch_fp8(int64_t T, int32_t H, int32_t K, int32_t E, int32_t R, int32_t M,
                           int32_t flags, const int32_t *slot, const uint8_t *q,
                           const float *scale, const int32_t *ue8m0, uint8_t *recv_q,
                           float *recv_scale, int32_t *recv_ue8m0, int32_t *status) {
    if (T < 0 || H % FP8_GROUP != 0 || E < 1 || R < 1 || M < 1) return -2;
    const int32_t G = H / FP8_GROUP, W = G / 4;
    const int64_t RM = (int64_t)R * M, rows = (int64_t)E * RM;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int32_t r = slot[t * K + k];
            if (r == -1) continue;
            if (r < -1 || r >= rows) {
                if (status) *status |= ST_BAD_SLOT;
                continue;
            }
            int64_t e = r / RM, i = r % RM;
            memcpy(recv_q + (int64_t)r * H, q + t * (int64_t)H, (size_t)H);
            for (int32_t g = 0; g < G; ++g) {
                int64_t at = (flags & FP8_SCALE_ROWS) ? (int64_t)r * G + g : (e * G + g) * RM + i;
#if ORACLE_MUTANT == 13
                at = (int64_t)r * G + g; /* mutant: always row-major */
#endif
                recv_scale[at] = scale[t * G + g];
            }
            if ((flags & FP8_UE8M0) && recv_ue8m0)
                for (int32_t w = 0; w < W; ++w) {
                    int64_t at = (flags & FP8_SCALE_ROWS) ? (int64_t)r * W + w : (e * W + w) * RM + i;
#if ORACLE_MUTANT == 16
                    at = (flags & FP8_SCALE_ROWS) ? (int64_t)w * rows + r : at; /* mutant: rows transposed */
#endif
                    recv_ue8m0[at] = ue8m0[t * W + w];
                }
        }
    }
    return 0;
}
