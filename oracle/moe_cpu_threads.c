/*
 * moe_cpu_threads.c -- the all-cores CPU baseline of the benchmark.
 *
 * NOT the oracle, and not the product: the benchmark's cpu_baseline leg times
 * it beside the single-threaded oracle (moe_oracle.c) to report what the
 * host's own cores do on the same step, and tests/test_cpu_threads.py checks
 * that its outputs equal the oracle's bit for bit. It shares no code with the
 * HIP library. Build: gcc -O2 -ffp-contract=off -pthread (no fast-math), like
 * the oracle, so the arithmetic is the same.
 *
 * Same method and readings as the oracle (see its header): dispatch is a
 * stable counting sort of the (token, k) pairs by expert ("aclnnMoeDistribute
 * DispatchV4", 计算公式: the all-to-all with every rank's window in one
 * memory), optionally with per-token dynamic int8 quantisation (quantMode 2:
 * scale = max|x| / 127 in fp32, q = rint(x / scale) clamped to +-127); combine
 * is the weighted sum of the combine_doubleplane README's check formula, fp32
 * with one fused multiply-add per k in ascending k and one rounding.
 *
 * Parallel split: the counting sort (counts, ep_recv_count, the row of every
 * pair) runs on one thread; the payload (row copies or codes) and the combine's
 * per-token sums are split over `threads` threads by token ranges. Only the
 * plain shapes of the benchmark are covered: no masks, no special experts, no
 * static or per-group quantisation.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { CT_INT32 = 0, CT_FP16 = 1, CT_BF16 = 2 };

/* binary16 / bfloat16 <-> binary32, from the IEEE definitions */
static float f16_to_f32(uint16_t v)
{
    int sign = v >> 15, expo = (v >> 10) & 0x1f, frac = v & 0x3ff;
    float mag = expo == 0 ? ldexpf((float)frac, -24)
                          : (expo == 31 ? (frac ? NAN : INFINITY) : ldexpf((float)(1024 + frac), expo - 25));
    return sign ? -mag : mag;
}

static uint32_t bits_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float bf16_to_f32(uint16_t v) { uint32_t u = (uint32_t)v << 16; float f; memcpy(&f, &u, 4); return f; }

static uint16_t f32_to_bf16(float f)
{
    uint32_t u = bits_of(f);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040);
    uint32_t hi = u >> 16, lo = u & 0xffff;
    if (lo > 0x8000 || (lo == 0x8000 && (hi & 1))) hi += 1;
    return (uint16_t)hi;
}

static uint16_t f32_to_f16(float f)
{
    uint16_t sign = (bits_of(f) >> 31) ? 0x8000 : 0;
    float a = fabsf(f);
    if (isnan(f)) return sign | 0x7e00;
    if (a == 0.0f) return sign;
    if (a < ldexpf(1.0f, -14)) return sign | (uint16_t)rintf(a / ldexpf(1.0f, -24));
    int e2;
    frexpf(a, &e2);
    int E = e2 - 1;
    float n = rintf(ldexpf(a, 10 - E));
    if (n == 2048.0f) { n = 1024.0f; E += 1; }
    if (E + 15 >= 31) return sign | 0x7c00;
    return sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)n - 1024);
}

static float load_elem(const void *base, size_t i, int dtype)
{
    const uint16_t *p = (const uint16_t *)base;
    return dtype == CT_FP16 ? f16_to_f32(p[i]) : bf16_to_f32(p[i]);
}

/* ---------------------------------------------------------------------- */

struct dispatch_job {
    const void *x;
    const int32_t *ids;
    const int64_t *row;          /* row of every pair */
    void *expand_x;
    float *dyn;
    long long t0, t1;
    int h, K, dtype, quant;
};

static void *dispatch_payload(void *arg)
{
    const struct dispatch_job *j = (const struct dispatch_job *)arg;
    const size_t xs = j->dtype == CT_INT32 ? 4 : 2;
    for (long long t = j->t0; t < j->t1; ++t) {
        float scale = 0.0f;
        if (j->quant == 2) {
            float amax = 0.0f;
            for (int c = 0; c < j->h; ++c) {
                float v = fabsf(load_elem(j->x, (size_t)(t * j->h + c), j->dtype));
                if (v > amax) amax = v;
            }
            scale = amax / 127.0f;
        }
        for (int k = 0; k < j->K; ++k) {
            long long row = j->row[t * j->K + k];
            if (j->quant == 0) {
                memcpy((char *)j->expand_x + (size_t)row * j->h * xs, (const char *)j->x + (size_t)t * j->h * xs,
                       (size_t)j->h * xs);
                continue;
            }
            int8_t *q = (int8_t *)j->expand_x + (size_t)row * j->h;
            for (int c = 0; c < j->h; ++c) {
                float v = load_elem(j->x, (size_t)(t * j->h + c), j->dtype);
                float n = scale == 0.0f ? 0.0f : rintf(v / scale);
                if (n > 127.0f) n = 127.0f;
                if (n < -127.0f) n = -127.0f;
                q[c] = (int8_t)n;
            }
            j->dyn[row] = scale;
        }
    }
    return NULL;
}

/* Dispatch with quant 0 or 2; outputs as the oracle's. Returns 0, or -1 on a bad argument. */
int cpu_dispatch_threads(const void *x, const int32_t *ids, int W, int bs, int epr, int h, int K, int dtype,
                         int quant, void *expand_x, float *dyn, int32_t *assist, int32_t *ep_recv_count,
                         int threads)
{
    if (W < 1 || bs < 0 || epr < 1 || h < 1 || K < 1 || threads < 1) return -1;
    if ((quant != 0 && quant != 2) || (quant == 2 && dtype == CT_INT32)) return -1;
    const long long E = (long long)W * epr, N = (long long)W * bs, S = E;
    long long *cnt = calloc((size_t)(W * S + 1), sizeof(long long));
    long long *fill = calloc((size_t)(W * S + 1), sizeof(long long));
    long long *base = malloc(((size_t)W + 1) * sizeof(long long));
    int64_t *row = malloc((size_t)(N * K + 1) * sizeof(int64_t));
    if (!cnt || !fill || !base || !row) { free(cnt); free(fill); free(base); free(row); return -1; }
    for (long long t = 0; t < N; ++t)
        for (int k = 0; k < K; ++k) {
            int32_t e = ids[t * K + k];
            if (e < 0 || e >= E) { free(cnt); free(fill); free(base); free(row); return -1; }
            cnt[(e / epr) * S + (e % epr) * W + t / bs] += 1;
        }
    long long running = 0;
    for (long long r = 0; r < W; ++r) {
        base[r] = running;
        long long c = 0;
        for (long long i = 0; i < S; ++i) {
            c += cnt[r * S + i];
            ep_recv_count[r * S + i] = (int32_t)c;
        }
        running += c;
    }
    for (long long t = 0; t < N; ++t)
        for (int k = 0; k < K; ++k) {
            int32_t e = ids[t * K + k];
            long long r = e / epr, i = (e % epr) * W + t / bs;
            long long rw = base[r] + (i ? ep_recv_count[r * S + i - 1] : 0) + fill[r * S + i]++;
            row[t * K + k] = rw;
            assist[rw * 3 + 0] = (int32_t)(t / bs);
            assist[rw * 3 + 1] = (int32_t)(t % bs);
            assist[rw * 3 + 2] = k;
        }
    pthread_t *tid = malloc(sizeof(pthread_t) * (size_t)threads);
    struct dispatch_job *jobs = malloc(sizeof(struct dispatch_job) * (size_t)threads);
    int *ok = calloc((size_t)threads, sizeof(int));
    for (int i = 0; i < threads; ++i) {
        struct dispatch_job j = {x, ids, row, expand_x, dyn, N * i / threads, N * (i + 1) / threads, h, K, dtype,
                                 quant};
        jobs[i] = j;
    }
    for (int i = 1; i < threads; ++i) ok[i] = pthread_create(&tid[i], NULL, dispatch_payload, &jobs[i]) == 0;
    dispatch_payload(&jobs[0]);
    for (int i = 1; i < threads; ++i) {
        if (ok[i]) pthread_join(tid[i], NULL);
        else dispatch_payload(&jobs[i]);          /* no thread: run its share here */
    }
    free(ok);
    free(jobs);
    free(tid);
    free(row);
    free(base);
    free(fill);
    free(cnt);
    return 0;
}

/* ---------------------------------------------------------------------- */

struct combine_job {
    const void *expand_x;
    const int64_t *slot;
    const void *scales;
    void *x_out;
    long long t0, t1;
    int h, K, dtype;
};

static void *combine_sums(void *arg)
{
    const struct combine_job *j = (const struct combine_job *)arg;
    for (long long t = j->t0; t < j->t1; ++t)
        for (int c = 0; c < j->h; ++c) {
            if (j->dtype == CT_INT32) {
                uint32_t acc = 0;
                for (int k = 0; k < j->K; ++k) {
                    const int32_t *y = (const int32_t *)j->expand_x + (size_t)j->slot[t * j->K + k] * j->h;
                    acc += (uint32_t)y[c] * (uint32_t)((const int32_t *)j->scales)[t * j->K + k];
                }
                ((int32_t *)j->x_out)[t * j->h + c] = (int32_t)acc;
            } else {
                float acc = 0.0f;
                for (int k = 0; k < j->K; ++k)
                    acc = fmaf(load_elem(j->expand_x, (size_t)j->slot[t * j->K + k] * j->h + c, j->dtype),
                               ((const float *)j->scales)[t * j->K + k], acc);
                ((uint16_t *)j->x_out)[t * j->h + c] = j->dtype == CT_FP16 ? f32_to_f16(acc) : f32_to_bf16(acc);
            }
        }
    return NULL;
}

/* Combine of a full dispatch (every pair has a row); the return path rebuilds each
 * pair's row from assist_info. Returns 0, or -1 on a bad argument or assist_info. */
int cpu_combine_threads(const void *expand_x, const int32_t *assist, const void *scales, int W, int bs, int h,
                        int K, int dtype, void *x_out, int threads)
{
    if (W < 1 || bs < 0 || h < 1 || K < 1 || threads < 1) return -1;
    const long long N = (long long)W * bs;
    int64_t *slot = malloc((size_t)(N * K + 1) * sizeof(int64_t));
    if (!slot) return -1;
    for (long long i = 0; i < N * K; ++i) {
        long long s = assist[i * 3 + 0], tok = assist[i * 3 + 1], k = assist[i * 3 + 2];
        if (s < 0 || s >= W || tok < 0 || tok >= bs || k < 0 || k >= K) { free(slot); return -1; }
        slot[(s * bs + tok) * K + k] = i;
    }
    pthread_t *tid = malloc(sizeof(pthread_t) * (size_t)threads);
    struct combine_job *jobs = malloc(sizeof(struct combine_job) * (size_t)threads);
    for (int i = 0; i < threads; ++i) {
        struct combine_job j = {expand_x, slot, scales, x_out, N * i / threads, N * (i + 1) / threads, h, K, dtype};
        jobs[i] = j;
    }
    int *ok = calloc((size_t)threads, sizeof(int));
    for (int i = 1; i < threads; ++i) ok[i] = pthread_create(&tid[i], NULL, combine_sums, &jobs[i]) == 0;
    combine_sums(&jobs[0]);
    for (int i = 1; i < threads; ++i) {
        if (ok[i]) pthread_join(tid[i], NULL);
        else combine_sums(&jobs[i]);
    }
    free(ok);
    free(jobs);
    free(tid);
    free(slot);
    return 0;
}
