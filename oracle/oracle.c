/*
 * CPU oracle for the gradient-bucket reduction: TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library. It shares no code, header or helper with the GPU path,
 * and it is deliberately plain and slow: one element at a time, in the order
 * the pages describe.
 *
 * Sources (page title, then the part of the page):
 *  [RING]  "图解 Ring All-Reduce：分布式训练梯度同步的核心算法",
 *          Phase 1 (Scatter-Reduce, rounds 1.1-1.3) and Phase 2 (All-Gather,
 *          rounds 2.1-2.3), and the summary table.
 *  [L14]   CMU 11-868 lecture 14 notes, "Distributed Training I:
 *          Communication and Data Parallelism": section 2.2 (the five
 *          primitives and their identities), section 3.2 (ring all-reduce:
 *          round formulas, placement, the 2(K-1)/K*N send volume), section
 *          3.3 (ring summation order differs from a plain sum), section 4.1
 *          (average = all-reduce SUM, then divide by the world size),
 *          exercise 3 and its answer (K = 3 rounds).
 *  [ZERO3] "DeepSpeed ZeRO-3 源码解析：前向与反向", section 5.1 (grads
 *          written into the IPG flat buffer at running offsets), section 5.2
 *          (contiguous path: all-reduce, then rank r keeps slice r), section
 *          5.3 (copy into the partitioned flat grad), section 1 (the single
 *          bf16 -> fp32 cast).
 *
 * Precision. Accumulation is fp32 with IEEE round-to-nearest-even; each bf16
 * input is widened exactly; a bf16 output is rounded once, to nearest even.
 * Built with -O2 -ffp-contract=off and without fast-math, so every add and
 * divide below is one IEEE operation.
 *
 * Readings where the pages leave a step open:
 *  - chunk size C = ceil(N / K); chunk j covers global indices [jC, jC + C);
 *    indices >= N are zero padding and their outputs are +0.0;
 *  - after reduce-scatter, chunk j is held by rank (j - shift) mod K; the
 *    ring gives shift = 1 [RING Phase 1 result; L14 3.2], the ZeRO-3
 *    contiguous path's local slice gives shift = 0 [ZERO3 5.2];
 *  - summation order of chunk j: start with rank j's value, then add ranks
 *    j+1, j+2, ..., j-1 (mod K), one fp32 add each (the path a chunk takes
 *    around the ring [RING Phase 1 rule]);
 *  - average: the fp32 sum divided by K with one IEEE divide [L14 4.1];
 *  - the fp32 partition output is not rounded to bf16 first.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_BF16 = 0, ORC_FP32 = 1 };

/* ------------------------------------------------------------------ bf16
 * bf16 is the upper half of an IEEE binary32 word: 1 sign bit, 8 exponent
 * bits, 7 fraction bits. Widening appends sixteen zero bits, which is exact.
 * Narrowing rounds the dropped sixteen bits to nearest, ties to even; a NaN
 * stays a NaN (its quiet bit is set so that truncation cannot make it Inf).
 */
float orc_bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

uint16_t orc_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t exp_bits = u & 0x7F800000u, frac = u & 0x007FFFFFu;
    if (exp_bits == 0x7F800000u && frac != 0) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t upper = u >> 16, lower = u & 0xFFFFu;
    /* lower > half: round up; lower == half: round up only if upper is odd */
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
    return (uint16_t)upper;
}

void orc_bf16_to_f32_array(const uint16_t* in, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_to_f32(in[i]);
}

void orc_f32_to_bf16_array(const float* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16(in[i]);
}

static float load_elem(const void* base, int dt, int64_t i) {
    if (dt == ORC_BF16) return orc_bf16_to_f32(((const uint16_t*)base)[i]);
    return ((const float*)base)[i];
}

static void store_elem(void* base, int dt, int64_t i, float v) {
    if (dt == ORC_BF16)
        ((uint16_t*)base)[i] = orc_f32_to_bf16(v);
    else
        ((float*)base)[i] = v;
}

static int64_t chunk_of(int64_t N, int K) { return (N + K - 1) / K; }

static int mod(int64_t a, int K) {
    int64_t m = a % K;
    return (int)(m < 0 ? m + K : m);
}

/* ------------------------------------------------------- ring simulator
 * A literal message-passing ring [RING; L14 3.2]. `state` is K ranks x K
 * chunks x C elements (rank-major), fp32. Rank r sends to rank (r+1) mod K.
 *
 *  scatter-reduce round i (i = 0 .. K-2): rank r sends its chunk
 *      (r - i) mod K; the receiver adds it to its own copy of that chunk.
 *  all-gather round i (i = 0 .. K-2): rank r sends its chunk
 *      (r + 1 - i) mod K; the receiver overwrites its copy.
 *
 * All sends of a round are collected before any receive is applied, as in a
 * real synchronous round. `sent[r]` accumulates the elements rank r sent.
 * Runs the first n_rs scatter-reduce rounds, then (only if n_rs == K-1) the
 * first n_ag all-gather rounds. With wire != 0 the ring carries bf16: the
 * receiver's new partial sum is rounded to bf16 before it is kept (and sent
 * on in the next round). Returns 0, or -1 on bad arguments.
 */
int orc_ring_run(int K, int64_t C, float* state, int n_rs, int n_ag, int64_t* sent, int wire) {
    if (K < 1 || C < 0 || n_rs < 0 || n_rs > K - 1 || n_ag < 0 || n_ag > K - 1) return -1;
    if (n_ag > 0 && n_rs != K - 1) return -1;
    float* msg = (float*)malloc(sizeof(float) * (size_t)(K * (C > 0 ? C : 1)));
    int* msg_chunk = (int*)malloc(sizeof(int) * (size_t)K);
    if (!msg || !msg_chunk) { free(msg); free(msg_chunk); return -1; }
    for (int phase = 0; phase < 2; ++phase) {
        int rounds = phase == 0 ? n_rs : n_ag;
        for (int i = 0; i < rounds; ++i) {
            /* every rank puts one chunk on the wire */
            for (int r = 0; r < K; ++r) {
                int c = phase == 0 ? mod((int64_t)r - i, K) : mod((int64_t)r + 1 - i, K);
                msg_chunk[r] = c;
                const float* src = state + ((int64_t)r * K + c) * C;
                memcpy(msg + (int64_t)r * C, src, sizeof(float) * (size_t)C);
                if (sent) sent[r] += C;
            }
            /* every rank receives from its left neighbour */
            for (int r = 0; r < K; ++r) {
                int from = mod((int64_t)r - 1, K);
                int c = msg_chunk[from];
                float* dst = state + ((int64_t)r * K + c) * C;
                const float* m = msg + (int64_t)from * C;
                for (int64_t o = 0; o < C; ++o) {
                    if (phase == 0) {
                        dst[o] = dst[o] + m[o];
                        if (wire) dst[o] = orc_bf16_to_f32(orc_f32_to_bf16(dst[o]));
                    } else {
                        dst[o] = m[o];
                    }
                }
            }
        }
    }
    free(msg);
    free(msg_chunk);
    return 0;
}

/* ------------------------------------------------------------ direct fold
 * Ring-order fold at explicit points. xs holds K rows of n values (row r =
 * rank r); point p starts with rank start[p] and adds the others in ring
 * order: acc = x[s], acc = acc + x[s+1], ..., acc = acc + x[s-1]. With
 * wire != 0 every partial sum is rounded to bf16 (a ring that carries bf16).
 */
static float hop(float acc, float x, int wire) {
    acc = acc + x;
    return wire ? orc_bf16_to_f32(orc_f32_to_bf16(acc)) : acc;
}

void orc_fold_points(int K, int64_t n, const float* xs, const int32_t* start, float* out, int wire) {
    for (int64_t p = 0; p < n; ++p) {
        int s = start[p];
        float acc = xs[(int64_t)s * n + p];
        for (int h = 1; h < K; ++h) acc = hop(acc, xs[(int64_t)((s + h) % K) * n + p], wire);
        out[p] = acc;
    }
}

/* The exact sum, for the free-order variant: accumulated in fp64 (its error,
 * at most about K * 2^-53 of the sum of magnitudes, is far below the
 * tolerance applied to a free-order result). abs_sum gets sum |x|. */
void orc_exact_sum_points(int K, int64_t n, const float* xs, double* out, double* abs_sum) {
    for (int64_t p = 0; p < n; ++p) {
        double s = 0.0, a = 0.0;
        for (int r = 0; r < K; ++r) {
            double v = (double)xs[(int64_t)r * n + p];
            s += v;
            a += fabs(v);
        }
        out[p] = s;
        if (abs_sum) abs_sum[p] = a;
    }
}

/* ------------------------------------------------ reduce-scatter (+avg+cast)
 * For every holder rank q and every offset o in [o_lo, o_hi) of its chunk:
 *   j = (q + shift) mod K, g = j*C + o,
 *   S = ring-order fold of x_{j}, x_{j+1}, ..., x_{j-1} at g (0 if g >= N),
 *   A = S / K if (flags & 1) else S,
 *   out_q[o] = A, or, if (flags & 2), the value already in out_q[o] plus A
 *   in one fp32 add (gradient accumulation: the first micro-step copies,
 *   later ones add in place [ZERO3 5.3, 6]),
 * stored as fp32 or rounded to bf16. With (flags & 4) the fold rounds every
 * partial sum to bf16 (a ring carrying bf16 partial sums); for fp32 input
 * this has no effect on the meaning of "the ring", so it is applied only to
 * bf16 input.
 */
int orc_reduce_scatter_part(int K, int64_t N, int in_dt, const void* const* in, int out_dt,
                            void* const* out, int shift, int flags, int64_t o_lo,
                            int64_t o_hi) {
    if (K < 1 || N < 0 || shift < 0 || shift >= K || (flags & ~7)) return -1;
    int average = flags & 1, accumulate = flags & 2, wire = (flags & 4) && in_dt == ORC_BF16;
    int64_t C = chunk_of(N, K);
    if (o_lo < 0 || o_hi > C || o_lo > o_hi) return -1;
    for (int q = 0; q < K; ++q) {
        int j = (q + shift) % K;
        for (int64_t o = o_lo; o < o_hi; ++o) {
            int64_t g = (int64_t)j * C + o;
            float acc = 0.0f;
            if (g < N) {
                acc = load_elem(in[j], in_dt, g);
                for (int h = 1; h < K; ++h) acc = hop(acc, load_elem(in[(j + h) % K], in_dt, g), wire);
                if (average) acc = acc / (float)K;
            }
            if (accumulate) acc = load_elem(out[q], out_dt, o) + acc;
            store_elem(out[q], out_dt, o, acc);
        }
    }
    return 0;
}

int orc_reduce_scatter(int K, int64_t N, int in_dt, const void* const* in, int out_dt,
                       void* const* out, int shift, int flags) {
    return orc_reduce_scatter_part(K, N, in_dt, in, out_dt, out, shift, flags, 0, chunk_of(N, K));
}

/* --------------------------------------------------------------- all-gather
 * segs: n_segs rows of (shard_off, full_off, numel). For each segment, with
 * C = ceil(numel / K), chunk j of the full tensor is shard (j - shift) mod K:
 *   full_r[full_off + j*C + o] = shard_{(j - shift) mod K}[shard_off + o]
 * for every destination rank r and every j*C + o < numel [RING Phase 2;
 * L14 3.2 all-gather; ZERO3 section 1, shards of 1/N rebuilt by all-gather].
 */
int orc_all_gather(int K, int dt, const void* const* shards, void* const* fulls,
                   const int64_t* segs, int n_segs, int shift) {
    if (K < 1 || shift < 0 || shift >= K || n_segs < 0) return -1;
    size_t es = dt == ORC_BF16 ? 2 : 4;
    for (int s = 0; s < n_segs; ++s) {
        int64_t shard_off = segs[3 * s], full_off = segs[3 * s + 1], numel = segs[3 * s + 2];
        int64_t C = chunk_of(numel, K);
        for (int r = 0; r < K; ++r)
            for (int j = 0; j < K; ++j) {
                int holder = mod((int64_t)j - shift, K);
                for (int64_t o = 0; o < C && (int64_t)j * C + o < numel; ++o) {
                    const char* src = (const char*)shards[holder] + (shard_off + o) * es;
                    char* dst = (char*)fulls[r] + (full_off + (int64_t)j * C + o) * es;
                    memcpy(dst, src, es);
                }
            }
    }
    return 0;
}

/* ---------------------------------------------------------------- all-reduce
 * All-reduce = reduce-scatter followed by all-gather [L14 2.2]: each chunk
 * is folded in ring order, divided by K when averaging (flags & 1), stored in
 * the output dtype once, and every rank receives the same stored value.
 * (flags & 4) selects the bf16-wire fold. in and out may be the same buffers.
 */
int orc_allreduce(int K, int64_t N, int dt, const void* const* in, void* const* out, int flags) {
    if (K < 1 || N < 0) return -1;
    int64_t C = chunk_of(N, K);
    size_t es = dt == ORC_BF16 ? 2 : 4;
    char* shard_mem = (char*)malloc(es * (size_t)(K * (C > 0 ? C : 1)));
    void** shards = (void**)malloc(sizeof(void*) * (size_t)K);
    if (!shard_mem || !shards) { free(shard_mem); free(shards); return -1; }
    for (int q = 0; q < K; ++q) shards[q] = shard_mem + (size_t)q * es * (size_t)C;
    /* ring placement: rank q holds chunk (q + 1) mod K, a shift of 1 mod K */
    int shift = 1 % K;
    int rc = orc_reduce_scatter(K, N, dt, in, dt, shards, shift, flags & 5);
    if (rc == 0) {
        int64_t seg[3] = {0, 0, N};
        rc = orc_all_gather(K, dt, (const void* const*)shards, out, seg, 1, shift);
    }
    free(shard_mem);
    free(shards);
    return rc;
}

/* ------------------------------------------------------------------ flatten
 * IPG bucket flatten [ZERO3 5.1]: fragment p of rank r lands at offset
 * n_0 + ... + n_{p-1} of bucket r; the bucket is then zero-filled from
 * n_0 + ... + n_{F-1} up to `padded`. frags is rank-major: frags[r*F + p].
 */
int orc_flatten(int K, int n_frag, int dt, const void* const* frags, const int64_t* numels,
                void* const* buckets, int64_t padded) {
    if (K < 1 || n_frag < 0) return -1;
    size_t es = dt == ORC_BF16 ? 2 : 4;
    int64_t total = 0;
    for (int p = 0; p < n_frag; ++p) {
        if (numels[p] < 0) return -1;
        total += numels[p];
    }
    if (padded < total) return -1;
    for (int r = 0; r < K; ++r) {
        int64_t off = 0;
        for (int p = 0; p < n_frag; ++p) {
            const char* src = (const char*)frags[(int64_t)r * n_frag + p];
            char* dst = (char*)buckets[r] + off * es;
            for (int64_t i = 0; i < numels[p]; ++i) memcpy(dst + i * es, src + i * es, es);
            off += numels[p];
        }
        memset((char*)buckets[r] + off * es, 0, (size_t)(padded - off) * es);
    }
    return 0;
}
