/*
 * pc_oracle.c -- plain, slow, fp64 CPU oracle for the paged KV-cache write and
 * paged decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Tests, the smoke check and the benchmark's CPU
 * baseline call it; the product library never links, loads or calls it, and it
 * shares no code, header, table or helper with the GPU path.
 *
 * What it computes, and where the pages define it:
 *
 *  oracle_write   -- "Inside vLLM CUDA Kernels: KV-Cache Writes and Paged
 *                    Attention", Part 2, sections "Decomposing a Slot into Block
 *                    and Offset" (negative slot = no destination; block = slot / B,
 *                    offset = slot % B) and "Why Layout and Quantization Scale
 *                    Produce Two Copy Paths" (block/page/head strides form the
 *                    address); "How vLLM CUDA Kernels Write and Read the Paged KV
 *                    Cache", section "Writing K and V into the cache".  Values are
 *                    copied as raw bits (the conversion is an identity when the
 *                    input and cache formats match).
 *
 *  oracle_decode  -- per (sequence s, query head h): the dense decode attention of
 *                    "vLLM 源码完全拆解（七）", section 先明确问题 (one query per (s,h),
 *                    softmax over the L_s visible tokens, max subtracted for
 *                    stability), with the head mapping of section 线程组织
 *                    (kv_head = h / (Hq/Hkv)), and the logical-to-physical walk of
 *                    "How vLLM CUDA Kernels Write and Read the Paged KV Cache",
 *                    section "Reading logical blocks during attention"
 *                    (physical block = block_table[t / B], offset = t % B).  The
 *                    logical K/V rows are materialised first, then scores
 *                    x_t = scale * q.k_t, m = max x, p_t = exp(x_t - m),
 *                    out = sum p_t v_t / sum p_t, all in double.  No epsilon in the
 *                    denominator; scale is the caller's float widened to double.
 *                    With ALiBi (alibi_slopes non-NULL, one slope a_h per query
 *                    head; same page, section 第一步): x_t = scale * q.k_t +
 *                    a_h * (t - (L_s - 1)) -- zero at the newest position, the
 *                    negative distance times the slope before it, added before
 *                    the softmax.
 *
 *  oracle_partials, oracle_merge -- the split-context form of "vLLM 源码完全拆解
 *                    （七）", section V1与V2 (512-token partitions; a partition past
 *                    seq_len does nothing) and the stable merge of "Inside vLLM CUDA
 *                    Kernels", Part 3, section "How Each K/V Tile Contributes to the
 *                    Output" (local states rescaled to a common maximum).  A
 *                    partition stores its own max m_p, exp-sum l_p and normalised
 *                    output o_p; the merge forms M = max m_p, w_p = l_p e^(m_p - M),
 *                    out = sum w_p o_p / sum w_p.
 *
 *  oracle_varlen  -- several query tokens per request over the paged history
 *                    ("Inside vLLM CUDA Kernels", Part 3, "How Metadata Connects a
 *                    Q Tile to Paged K/V": query_start_loc delimits each request's
 *                    rows of the packed query, seq_lens its visible KV length,
 *                    block_table its pages).  Request r owns packed rows
 *                    [qs[r], qs[r+1]), n = qs[r+1] - qs[r] <= L_r of them; these are
 *                    the request's newest tokens, so token i sits at position
 *                    p = L_r - n + i.  Causal: it attends positions t <= p; else all
 *                    of [0, L_r).  Scores, softmax and ALiBi as for the decode, the
 *                    bias measured from p.  With n = 1 this is the decode.
 *
 *  oracle_write_kv8, oracle_decode_kv8, oracle_partials_kv8 -- the same with an
 *                    8-bit floating-point cache ("Inside vLLM CUDA Kernels", Part 2,
 *                    "Why Layout and Quantization Scale Produce Two Copy Paths":
 *                    k_scale / v_scale, one shared scale when kv_scale_stride is 0,
 *                    else head h uses scale[h * kv_scale_stride]; "vLLM 源码完全拆解
 *                    （七）", 参数与内存布局: the kernel converts the quantised cache
 *                    with k_scale / v_scale when it loads it).  The pages name no
 *                    format; this oracle takes OCP E4M3 (see e4m3_to_double).  The
 *                    write stores code(x / scale), x / scale computed in binary32;
 *                    the decode reads code value * scale, in double.
 *
 * Storage formats: 0 = fp32, 1 = fp16, 2 = bf16 (raw bits in memory); caches may
 * also be 3 = OCP FP8 E4M3 (one byte per element).
 * Return codes: 0 ok, -1 invalid argument, -2 a data value points outside the
 * pool (slot, block id or sequence length) -- the oracle refuses to read or write
 * out of range, so a test that passes proves no such access was needed.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_EINVAL (-1)
#define OR_ERANGE (-2)

static int esize_of(int fmt) {
    return fmt == 0 ? 4 : (fmt == 1 || fmt == 2) ? 2 : 0;
}

/* IEEE binary16 -> double, from the format's definition. */
static double half_to_double(uint16_t h) {
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 is the upper half of a binary32. */
static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* OCP 8-bit floating point, E4M3 variant: sign bit, 4 exponent bits (bias 7), 3
 * mantissa bits.  Exponent field 0 holds subnormals m/8 * 2^-6; there are no
 * infinities; exponent 1111 with mantissa 111 is NaN, so the largest finite
 * magnitude is 1.75 * 2^8 = 448. */
static double e4m3_to_double(uint8_t c) {
    int sign = c >> 7;
    int e = (c >> 3) & 0xf;
    int m = c & 7;
    if (e == 0xf && m == 7)
        return NAN;
    double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return sign ? -v : v;
}

/* The E4M3 code nearest to y, found by comparing against every finite positive
 * code (codes 0..0x7E increase with their value); a tie goes to the code with the
 * even mantissa.  Magnitudes of 448 and above (infinities included) give +-448;
 * NaN gives 0xFF. */
static uint8_t e4m3_from_float(float y) {
    if (isnan(y))
        return 0xff;
    uint8_t sign = signbit(y) ? 0x80 : 0;
    double a = fabs((double)y);
    if (a >= 448.0)
        return sign | 0x7e;
    int lo = 0; /* largest code whose value is <= a */
    for (int c = 1; c <= 0x7e; ++c)
        if (e4m3_to_double((uint8_t)c) <= a)
            lo = c;
    double below = a - e4m3_to_double((uint8_t)lo);
    double above = e4m3_to_double((uint8_t)(lo + 1)) - a;
    int c = below < above ? lo : above < below ? lo + 1 : ((lo & 1) ? lo + 1 : lo);
    return sign | (uint8_t)c;
}

static double load_elem(const void *base, int64_t idx, int fmt) {
    if (fmt == 3)
        return e4m3_to_double(((const uint8_t *)base)[idx]);
    if (fmt == 0) {
        float f;
        memcpy(&f, (const char *)base + idx * 4, 4);
        return (double)f;
    }
    uint16_t b;
    memcpy(&b, (const char *)base + idx * 2, 2);
    return fmt == 1 ? half_to_double(b) : bf16_to_double(b);
}

/* ------------------------------------------------------------------------- */
/* write                                                                      */
/* ------------------------------------------------------------------------- */

int oracle_write(void *k_pool, void *v_pool, int64_t pool_elems, int64_t num_blocks,
                 int64_t block_stride, int64_t token_stride, int64_t head_stride,
                 const void *key, const void *value, int64_t key_row_stride, int64_t value_row_stride,
                 const int64_t *slot_mapping, int64_t num_tokens,
                 int num_kv_heads, int head_size, int block_size, int fmt) {
    int es = esize_of(fmt);
    if (!es || !k_pool || !v_pool || num_tokens < 0 || num_kv_heads <= 0 || head_size <= 0 || block_size <= 0)
        return OR_EINVAL;
    if (num_tokens > 0 && (!key || !value || !slot_mapping))
        return OR_EINVAL;
    for (int64_t t = 0; t < num_tokens; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot < 0)
            continue; /* padding: no destination */
        int64_t blk = slot / block_size;
        int64_t off = slot % block_size;
        if (blk >= num_blocks)
            return OR_ERANGE;
        for (int h = 0; h < num_kv_heads; ++h) {
            /* the head_size elements of one head are contiguous on both sides */
            int64_t dst = blk * block_stride + off * token_stride + (int64_t)h * head_stride;
            if (dst < 0 || dst + head_size > pool_elems)
                return OR_ERANGE;
            int64_t ks = t * key_row_stride + (int64_t)h * head_size;
            int64_t vs = t * value_row_stride + (int64_t)h * head_size;
            memcpy((char *)k_pool + dst * es, (const char *)key + ks * es, (size_t)head_size * es);
            memcpy((char *)v_pool + dst * es, (const char *)value + vs * es, (size_t)head_size * es);
        }
    }
    return OR_OK;
}

/* The write into an E4M3 cache: element x of head h becomes the code of
 * x / scale[h * scale_stride], the division done in binary32 (x is exact in it). */
int oracle_write_kv8(uint8_t *k_pool, uint8_t *v_pool, int64_t pool_elems, int64_t num_blocks,
                     int64_t block_stride, int64_t token_stride, int64_t head_stride,
                     const void *key, const void *value, int64_t key_row_stride, int64_t value_row_stride,
                     const int64_t *slot_mapping, int64_t num_tokens, int num_kv_heads, int head_size,
                     int block_size, int src_fmt, const float *k_scale, const float *v_scale,
                     int64_t scale_stride) {
    if (!esize_of(src_fmt) || !k_pool || !v_pool || num_tokens < 0 || num_kv_heads <= 0 || head_size <= 0 ||
        block_size <= 0 || scale_stride < 0 || !k_scale || !v_scale)
        return OR_EINVAL;
    if (num_tokens > 0 && (!key || !value || !slot_mapping))
        return OR_EINVAL;
    for (int64_t t = 0; t < num_tokens; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot < 0)
            continue; /* padding: no destination */
        int64_t blk = slot / block_size;
        int64_t off = slot % block_size;
        if (blk >= num_blocks)
            return OR_ERANGE;
        for (int h = 0; h < num_kv_heads; ++h) {
            int64_t dst = blk * block_stride + off * token_stride + (int64_t)h * head_stride;
            if (dst < 0 || dst + head_size > pool_elems)
                return OR_ERANGE;
            float ks = k_scale[(int64_t)h * scale_stride];
            float vs = v_scale[(int64_t)h * scale_stride];
            for (int d = 0; d < head_size; ++d) {
                float kx = (float)load_elem(key, t * key_row_stride + (int64_t)h * head_size + d, src_fmt);
                float vx = (float)load_elem(value, t * value_row_stride + (int64_t)h * head_size + d, src_fmt);
                k_pool[dst + d] = e4m3_from_float(kx / ks);
                v_pool[dst + d] = e4m3_from_float(vx / vs);
            }
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------- */
/* decode                                                                     */
/* ------------------------------------------------------------------------- */

typedef struct {
    const void *q, *k_pool, *v_pool;
    int64_t pool_elems, num_blocks, block_stride, token_stride, head_stride;
    const int32_t *block_tables;
    int max_blocks_per_seq;
    const int32_t *seq_lens;
    int num_seqs, num_q_heads, num_kv_heads, head_size, block_size;
    double scale;
    const float *alibi_slopes;       /* NULL, or one slope per query head */
    int fmt;                         /* q (and out) */
    int kv_fmt;                      /* the pool */
    const float *k_scale, *v_scale;  /* E4M3 pool: head kv uses scale[kv * scale_stride] */
    int64_t scale_stride;
    int partition_size; /* 0: whole sequence (decode); > 0: partials */
    const int32_t *query_start_loc;  /* varlen: [num_seqs + 1] row ranges of the packed q */
    int varlen, causal;
    int max_partitions;
    /* outputs */
    double *out;                                  /* decode: [S, Hq, D] */
    double *tmp_out, *max_logits, *exp_sums;      /* partials: [S, Hq, P, D], [S, Hq, P] */
    /* work split */
    int64_t n_items;
    int nthreads;
    int status;
    pthread_mutex_t lock;
} job_t;

typedef struct {
    job_t *job;
    int tid;
} worker_arg_t;

/* Materialise the logical rows [t0, t1) of sequence s, kv head kv, as doubles:
 * block_table[s, t / B] gives the physical block, t % B the row inside it. */
static int gather_rows(const job_t *j, int s, int kv, int t0, int t1, double *K, double *V) {
    const int32_t *row = j->block_tables + (int64_t)s * j->max_blocks_per_seq;
    for (int t = t0; t < t1; ++t) {
        int lb = t / j->block_size;
        int off = t % j->block_size;
        if (lb >= j->max_blocks_per_seq)
            return OR_ERANGE;
        int64_t phys = row[lb];
        if (phys < 0 || phys >= j->num_blocks)
            return OR_ERANGE;
        int64_t base = phys * j->block_stride + (int64_t)off * j->token_stride + (int64_t)kv * j->head_stride;
        if (base < 0 || base + j->head_size > j->pool_elems)
            return OR_ERANGE;
        double ks = 1.0, vs = 1.0;
        if (j->kv_fmt == 3) {
            ks = (double)j->k_scale[(int64_t)kv * j->scale_stride];
            vs = (double)j->v_scale[(int64_t)kv * j->scale_stride];
        }
        for (int d = 0; d < j->head_size; ++d) {
            K[(int64_t)(t - t0) * j->head_size + d] = load_elem(j->k_pool, base + d, j->kv_fmt) * ks;
            V[(int64_t)(t - t0) * j->head_size + d] = load_elem(j->v_pool, base + d, j->kv_fmt) * vs;
        }
    }
    return OR_OK;
}

/* Dense softmax attention of one query over n materialised rows; row t sits at
 * position pos0 + t relative to the newest token (so pos0 + t <= 0), which the ALiBi
 * term slope * (pos0 + t) uses (slope 0 without ALiBi).
 * Writes o[D] = sum p_t v_t / sum p_t, *m = max x_t, *l = sum p_t. */
static void dense_attention(const double *qv, const double *K, const double *V, int n, int D, double scale,
                            double slope, int64_t pos0, double *x, double *o, double *m_out, double *l_out) {
    double m = -INFINITY;
    for (int t = 0; t < n; ++t) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += qv[d] * K[(int64_t)t * D + d];
        x[t] = scale * dot + slope * (double)(pos0 + t);
        if (x[t] > m)
            m = x[t];
    }
    double l = 0.0;
    for (int t = 0; t < n; ++t) {
        x[t] = exp(x[t] - m);
        l += x[t];
    }
    for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int t = 0; t < n; ++t)
            acc += x[t] * V[(int64_t)t * D + d];
        o[d] = acc / l;
    }
    *m_out = m;
    *l_out = l;
}

/* Varlen work item = one (packed query row, head). */
static int run_varlen_item(job_t *j, int64_t item, double *K, double *V, double *x, double *qv) {
    int D = j->head_size;
    int G = j->num_q_heads / j->num_kv_heads;
    int h = (int)(item % j->num_q_heads);
    int64_t row = item / j->num_q_heads;
    const int32_t *qs = j->query_start_loc;
    int lo = 0, hi = j->num_seqs - 1; /* the request r with qs[r] <= row < qs[r + 1] */
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (qs[mid] <= row)
            lo = mid;
        else
            hi = mid - 1;
    }
    int r = lo;
    int n = qs[r + 1] - qs[r];
    int i = (int)(row - qs[r]);
    int L = j->seq_lens[r];
    if (L < n || (int64_t)L > (int64_t)j->max_blocks_per_seq * j->block_size)
        return OR_ERANGE;
    int p = L - n + i; /* position of this query token */
    int visible = j->causal ? p + 1 : L;
    for (int d = 0; d < D; ++d)
        qv[d] = load_elem(j->q, (row * j->num_q_heads + h) * D + d, j->fmt);
    int rc = gather_rows(j, r, h / G, 0, visible, K, V);
    if (rc)
        return rc;
    double slope = j->alibi_slopes ? (double)j->alibi_slopes[h] : 0.0;
    double m, l;
    dense_attention(qv, K, V, visible, D, j->scale, slope, -(int64_t)p, x, j->out + (row * j->num_q_heads + h) * D,
                    &m, &l);
    return OR_OK;
}

/* One work item = one (s, h) for decode, one (s, h, p) for partials. */
static int run_item(job_t *j, int64_t item, double *K, double *V, double *x, double *qv) {
    if (j->varlen)
        return run_varlen_item(j, item, K, V, x, qv);
    int D = j->head_size;
    int G = j->num_q_heads / j->num_kv_heads;
    int s, h, p = 0;
    if (j->partition_size > 0) {
        p = (int)(item % j->max_partitions);
        h = (int)((item / j->max_partitions) % j->num_q_heads);
        s = (int)(item / ((int64_t)j->max_partitions * j->num_q_heads));
    } else {
        h = (int)(item % j->num_q_heads);
        s = (int)(item / j->num_q_heads);
    }
    int kv = h / G;
    double slope = j->alibi_slopes ? (double)j->alibi_slopes[h] : 0.0;
    int L = j->seq_lens[s];
    if (L < 0 || (int64_t)L > (int64_t)j->max_blocks_per_seq * j->block_size)
        return OR_ERANGE;
    for (int d = 0; d < D; ++d)
        qv[d] = load_elem(j->q, ((int64_t)s * j->num_q_heads + h) * D + d, j->fmt);

    if (j->partition_size == 0) {
        double *o = j->out + ((int64_t)s * j->num_q_heads + h) * D;
        if (L == 0) { /* no visible token: defined as zeros */
            for (int d = 0; d < D; ++d)
                o[d] = 0.0;
            return OR_OK;
        }
        int rc = gather_rows(j, s, kv, 0, L, K, V);
        if (rc)
            return rc;
        double m, l;
        dense_attention(qv, K, V, L, D, j->scale, slope, -(int64_t)(L - 1), x, o, &m, &l);
        return OR_OK;
    }

    int t0 = p * j->partition_size;
    if (t0 >= L)
        return OR_OK; /* empty partition: writes nothing */
    if ((int64_t)L > (int64_t)j->max_partitions * j->partition_size)
        return OR_ERANGE;
    int t1 = t0 + j->partition_size < L ? t0 + j->partition_size : L;
    int rc = gather_rows(j, s, kv, t0, t1, K, V);
    if (rc)
        return rc;
    int64_t sp = ((int64_t)s * j->num_q_heads + h) * j->max_partitions + p;
    dense_attention(qv, K, V, t1 - t0, D, j->scale, slope, (int64_t)t0 - (L - 1), x, j->tmp_out + sp * D,
                    &j->max_logits[sp], &j->exp_sums[sp]);
    return OR_OK;
}

static void *worker(void *argp) {
    worker_arg_t *a = (worker_arg_t *)argp;
    job_t *j = a->job;
    /* rows of one materialised range: a partition, or the longest valid sequence */
    int64_t rows = j->partition_size;
    if (j->partition_size == 0) {
        int64_t cap = (int64_t)j->max_blocks_per_seq * j->block_size;
        rows = 1;
        for (int s = 0; s < j->num_seqs; ++s)
            if (j->seq_lens[s] > rows)
                rows = j->seq_lens[s] < cap ? j->seq_lens[s] : cap;
    }
    double *K = (double *)malloc(sizeof(double) * (size_t)rows * (size_t)j->head_size + 8);
    double *V = (double *)malloc(sizeof(double) * (size_t)rows * (size_t)j->head_size + 8);
    double *x = (double *)malloc(sizeof(double) * (size_t)rows + 8);
    double *qv = (double *)malloc(sizeof(double) * (size_t)j->head_size);
    int rc = OR_OK;
    if (!K || !V || !x || !qv)
        rc = OR_EINVAL;
    for (int64_t it = a->tid; rc == OR_OK && it < j->n_items; it += j->nthreads)
        rc = run_item(j, it, K, V, x, qv);
    if (rc) {
        pthread_mutex_lock(&j->lock);
        if (!j->status)
            j->status = rc;
        pthread_mutex_unlock(&j->lock);
    }
    free(K);
    free(V);
    free(x);
    free(qv);
    return NULL;
}

static int run_job(job_t *j, int nthreads) {
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    j->nthreads = nthreads;
    j->status = OR_OK;
    pthread_mutex_init(&j->lock, NULL);
    pthread_t th[256];
    worker_arg_t args[256];
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        args[i].job = j;
        args[i].tid = i;
        if (i == 0)
            continue;
        if (pthread_create(&th[i], NULL, worker, &args[i]) == 0)
            started = i;
        else
            break;
    }
    if (started + 1 < nthreads) {
        /* could not start every thread: let the caller's thread take every item */
        for (int i = 1; i <= started; ++i)
            pthread_join(th[i], NULL);
        j->nthreads = 1;
        args[0].tid = 0;
        worker(&args[0]);
    } else {
        worker(&args[0]);
        for (int i = 1; i < nthreads; ++i)
            pthread_join(th[i], NULL);
    }
    pthread_mutex_destroy(&j->lock);
    return j->status;
}

static int check_common(const void *q, const void *k_pool, const void *v_pool, const int32_t *block_tables,
                        const int32_t *seq_lens, int num_seqs, int num_q_heads, int num_kv_heads, int head_size,
                        int block_size, int max_blocks_per_seq, int fmt) {
    if (!esize_of(fmt) || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 ||
        block_size <= 0 || max_blocks_per_seq < 0 || num_q_heads % num_kv_heads)
        return OR_EINVAL;
    if (num_seqs > 0 && (!q || !k_pool || !v_pool || !block_tables || !seq_lens))
        return OR_EINVAL;
    return OR_OK;
}

int oracle_decode(double *out, const void *q, const void *k_pool, const void *v_pool, int64_t pool_elems,
                  int64_t num_blocks, int64_t block_stride, int64_t token_stride, int64_t head_stride,
                  const int32_t *block_tables, int max_blocks_per_seq, const int32_t *seq_lens, int num_seqs,
                  int num_q_heads, int num_kv_heads, int head_size, int block_size, float scale,
                  const float *alibi_slopes, int fmt, int nthreads) {
    int rc = check_common(q, k_pool, v_pool, block_tables, seq_lens, num_seqs, num_q_heads, num_kv_heads,
                          head_size, block_size, max_blocks_per_seq, fmt);
    if (rc)
        return rc;
    if (num_seqs > 0 && !out)
        return OR_EINVAL;
    job_t j;
    memset(&j, 0, sizeof j);
    j.q = q;
    j.k_pool = k_pool;
    j.v_pool = v_pool;
    j.pool_elems = pool_elems;
    j.num_blocks = num_blocks;
    j.block_stride = block_stride;
    j.token_stride = token_stride;
    j.head_stride = head_stride;
    j.block_tables = block_tables;
    j.max_blocks_per_seq = max_blocks_per_seq;
    j.seq_lens = seq_lens;
    j.num_seqs = num_seqs;
    j.num_q_heads = num_q_heads;
    j.num_kv_heads = num_kv_heads;
    j.head_size = head_size;
    j.block_size = block_size;
    j.scale = (double)scale;
    j.alibi_slopes = alibi_slopes;
    j.fmt = fmt;
    j.kv_fmt = fmt;
    j.out = out;
    j.n_items = (int64_t)num_seqs * num_q_heads;
    return run_job(&j, nthreads);
}

int oracle_partials(double *tmp_out, double *max_logits, double *exp_sums, const void *q, const void *k_pool,
                    const void *v_pool, int64_t pool_elems, int64_t num_blocks, int64_t block_stride,
                    int64_t token_stride, int64_t head_stride, const int32_t *block_tables, int max_blocks_per_seq,
                    const int32_t *seq_lens, int num_seqs, int num_q_heads, int num_kv_heads, int head_size,
                    int block_size, float scale, const float *alibi_slopes, int partition_size, int max_partitions,
                    int fmt, int nthreads) {
    int rc = check_common(q, k_pool, v_pool, block_tables, seq_lens, num_seqs, num_q_heads, num_kv_heads,
                          head_size, block_size, max_blocks_per_seq, fmt);
    if (rc)
        return rc;
    if (partition_size <= 0 || max_partitions < 0 || (num_seqs > 0 && (!tmp_out || !max_logits || !exp_sums)))
        return OR_EINVAL;
    job_t j;
    memset(&j, 0, sizeof j);
    j.q = q;
    j.k_pool = k_pool;
    j.v_pool = v_pool;
    j.pool_elems = pool_elems;
    j.num_blocks = num_blocks;
    j.block_stride = block_stride;
    j.token_stride = token_stride;
    j.head_stride = head_stride;
    j.block_tables = block_tables;
    j.max_blocks_per_seq = max_blocks_per_seq;
    j.seq_lens = seq_lens;
    j.num_seqs = num_seqs;
    j.num_q_heads = num_q_heads;
    j.num_kv_heads = num_kv_heads;
    j.head_size = head_size;
    j.block_size = block_size;
    j.scale = (double)scale;
    j.alibi_slopes = alibi_slopes;
    j.fmt = fmt;
    j.kv_fmt = fmt;
    j.partition_size = partition_size;
    j.max_partitions = max_partitions;
    j.tmp_out = tmp_out;
    j.max_logits = max_logits;
    j.exp_sums = exp_sums;
    j.n_items = (int64_t)num_seqs * num_q_heads * max_partitions;
    return run_job(&j, nthreads);
}

/* Merge the partials of the ceil(L_s / partition_size) partitions that hold tokens.
 * A sequence with no token gets zeros. */
int oracle_merge(double *out, const double *tmp_out, const double *max_logits, const double *exp_sums,
                 const int32_t *seq_lens, int num_seqs, int num_q_heads, int head_size, int max_partitions,
                 int partition_size) {
    if (num_seqs < 0 || num_q_heads <= 0 || head_size <= 0 || max_partitions < 0 || partition_size <= 0)
        return OR_EINVAL;
    if (num_seqs > 0 && (!out || !tmp_out || !max_logits || !exp_sums || !seq_lens))
        return OR_EINVAL;
    for (int s = 0; s < num_seqs; ++s) {
        int L = seq_lens[s];
        if (L < 0)
            return OR_ERANGE;
        int np_ = (int)(((int64_t)L + partition_size - 1) / partition_size);
        if (np_ > max_partitions)
            return OR_ERANGE;
        for (int h = 0; h < num_q_heads; ++h) {
            int64_t sh = (int64_t)s * num_q_heads + h;
            double *o = out + sh * head_size;
            double M = -INFINITY;
            for (int p = 0; p < np_; ++p)
                if (max_logits[sh * max_partitions + p] > M)
                    M = max_logits[sh * max_partitions + p];
            double wsum = 0.0;
            for (int d = 0; d < head_size; ++d)
                o[d] = 0.0;
            for (int p = 0; p < np_; ++p) {
                double w = exp_sums[sh * max_partitions + p] * exp(max_logits[sh * max_partitions + p] - M);
                wsum += w;
                const double *op = tmp_out + (sh * max_partitions + p) * head_size;
                for (int d = 0; d < head_size; ++d)
                    o[d] += w * op[d];
            }
            if (np_ > 0)
                for (int d = 0; d < head_size; ++d)
                    o[d] /= wsum;
        }
    }
    return OR_OK;
}

/* Multi-token queries: each packed query row of request r (rows query_start_loc[r] ..
   query_start_loc[r+1], its newest tokens) attends the positions it may see (causal: up to
   its own position seq_len - n + i; otherwise all of [0, seq_len)). */
int oracle_varlen(double *out, const void *q, const void *k_pool, const void *v_pool, int64_t pool_elems,
                  int64_t num_blocks, int64_t block_stride, int64_t token_stride, int64_t head_stride,
                  const int32_t *block_tables, int max_blocks_per_seq, const int32_t *query_start_loc,
                  const int32_t *seq_lens, int num_reqs, int64_t total_q, int num_q_heads, int num_kv_heads,
                  int head_size, int block_size, float scale, int causal, const float *alibi_slopes, int fmt,
                  int nthreads) {
    int rc = check_common(q, k_pool, v_pool, block_tables, seq_lens, num_reqs, num_q_heads, num_kv_heads,
                          head_size, block_size, max_blocks_per_seq, fmt);
    if (rc)
        return rc;
    if (!query_start_loc || total_q < 0 || (total_q > 0 && !out))
        return OR_EINVAL;
    if (query_start_loc[0] != 0 || (num_reqs >= 0 && query_start_loc[num_reqs] != total_q))
        return OR_EINVAL;
    for (int r = 0; r < num_reqs; ++r)
        if (query_start_loc[r + 1] < query_start_loc[r])
            return OR_EINVAL;
    job_t j;
    memset(&j, 0, sizeof j);
    j.q = q;
    j.k_pool = k_pool;
    j.v_pool = v_pool;
    j.pool_elems = pool_elems;
    j.num_blocks = num_blocks;
    j.block_stride = block_stride;
    j.token_stride = token_stride;
    j.head_stride = head_stride;
    j.block_tables = block_tables;
    j.max_blocks_per_seq = max_blocks_per_seq;
    j.seq_lens = seq_lens;
    j.num_seqs = num_reqs;
    j.num_q_heads = num_q_heads;
    j.num_kv_heads = num_kv_heads;
    j.head_size = head_size;
    j.block_size = block_size;
    j.scale = (double)scale;
    j.alibi_slopes = alibi_slopes;
    j.fmt = fmt;
    j.kv_fmt = fmt;
    j.out = out;
    j.query_start_loc = query_start_loc;
    j.varlen = 1;
    j.causal = causal != 0;
    j.n_items = total_q * num_q_heads;
    return run_job(&j, nthreads);
}

/* The decode and the partials over an E4M3 pool (q, out in fmt). */
int oracle_decode_kv8(double *out, const void *q, const uint8_t *k_pool, const uint8_t *v_pool, int64_t pool_elems,
                      int64_t num_blocks, int64_t block_stride, int64_t token_stride, int64_t head_stride,
                      const int32_t *block_tables, int max_blocks_per_seq, const int32_t *seq_lens, int num_seqs,
                      int num_q_heads, int num_kv_heads, int head_size, int block_size, float scale,
                      const float *alibi_slopes, int fmt, const float *k_scale, const float *v_scale,
                      int64_t scale_stride, int nthreads) {
    int rc = check_common(q, k_pool, v_pool, block_tables, seq_lens, num_seqs, num_q_heads, num_kv_heads,
                          head_size, block_size, max_blocks_per_seq, fmt);
    if (rc)
        return rc;
    if ((num_seqs > 0 && !out) || !k_scale || !v_scale || scale_stride < 0)
        return OR_EINVAL;
    job_t j;
    memset(&j, 0, sizeof j);
    j.q = q;
    j.k_pool = k_pool;
    j.v_pool = v_pool;
    j.pool_elems = pool_elems;
    j.num_blocks = num_blocks;
    j.block_stride = block_stride;
    j.token_stride = token_stride;
    j.head_stride = head_stride;
    j.block_tables = block_tables;
    j.max_blocks_per_seq = max_blocks_per_seq;
    j.seq_lens = seq_lens;
    j.num_seqs = num_seqs;
    j.num_q_heads = num_q_heads;
    j.num_kv_heads = num_kv_heads;
    j.head_size = head_size;
    j.block_size = block_size;
    j.scale = (double)scale;
    j.alibi_slopes = alibi_slopes;
    j.fmt = fmt;
    j.kv_fmt = 3;
    j.k_scale = k_scale;
    j.v_scale = v_scale;
    j.scale_stride = scale_stride;
    j.out = out;
    j.n_items = (int64_t)num_seqs * num_q_heads;
    return run_job(&j, nthreads);
}

int oracle_partials_kv8(double *tmp_out, double *max_logits, double *exp_sums, const void *q, const uint8_t *k_pool,
                        const uint8_t *v_pool, int64_t pool_elems, int64_t num_blocks, int64_t block_stride,
                        int64_t token_stride, int64_t head_stride, const int32_t *block_tables,
                        int max_blocks_per_seq, const int32_t *seq_lens, int num_seqs, int num_q_heads,
                        int num_kv_heads, int head_size, int block_size, float scale, const float *alibi_slopes,
                        int partition_size, int max_partitions, int fmt, const float *k_scale,
                        const float *v_scale, int64_t scale_stride, int nthreads) {
    int rc = check_common(q, k_pool, v_pool, block_tables, seq_lens, num_seqs, num_q_heads, num_kv_heads,
                          head_size, block_size, max_blocks_per_seq, fmt);
    if (rc)
        return rc;
    if (partition_size <= 0 || max_partitions < 0 || (num_seqs > 0 && (!tmp_out || !max_logits || !exp_sums)) ||
        !k_scale || !v_scale || scale_stride < 0)
        return OR_EINVAL;
    job_t j;
    memset(&j, 0, sizeof j);
    j.q = q;
    j.k_pool = k_pool;
    j.v_pool = v_pool;
    j.pool_elems = pool_elems;
    j.num_blocks = num_blocks;
    j.block_stride = block_stride;
    j.token_stride = token_stride;
    j.head_stride = head_stride;
    j.block_tables = block_tables;
    j.max_blocks_per_seq = max_blocks_per_seq;
    j.seq_lens = seq_lens;
    j.num_seqs = num_seqs;
    j.num_q_heads = num_q_heads;
    j.num_kv_heads = num_kv_heads;
    j.head_size = head_size;
    j.block_size = block_size;
    j.scale = (double)scale;
    j.alibi_slopes = alibi_slopes;
    j.fmt = fmt;
    j.kv_fmt = 3;
    j.k_scale = k_scale;
    j.v_scale = v_scale;
    j.scale_stride = scale_stride;
    j.partition_size = partition_size;
    j.max_partitions = max_partitions;
    j.tmp_out = tmp_out;
    j.max_logits = max_logits;
    j.exp_sums = exp_sums;
    j.n_items = (int64_t)num_seqs * num_q_heads * max_partitions;
    return run_job(&j, nthreads);
}

/* Element-wise access for tests: the value of E4M3 codes, and the codes of floats. */
void oracle_e4m3_decode(double *out, const uint8_t *codes, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = e4m3_to_double(codes[i]);
}

void oracle_e4m3_encode(uint8_t *out, const float *x, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = e4m3_from_float(x[i]);
}
