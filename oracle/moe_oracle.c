/*
 * moe_oracle.c -- plain, slow CPU reference for MoE token dispatch and combine.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call
 * this file: only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark use it. It shares no source, header, table or helper with the HIP
 * library; the two only ever see the same seeded inputs.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no fast-math). Every fused
 * multiply-add is written out as fmaf(); nothing else may be contracted.
 *
 * What it follows (the pages):
 *  [P1] CANN SHMEM examples, "双平面 MoE Combine 示例" (combine_doubleplane
 *       README): section 功能说明 defines the dispatch outputs expand_x,
 *       assist_info_for_combine ([src_rank_id, src_token_id, src_topk_id] per
 *       expert-output row), ep_recv_count (cumulative count per
 *       (local_expert_id, src_rank_id) segment), and the check formula
 *       x_out[token] = sum_k topk_output[token,k] * expert_scales[token,k];
 *       section 方案设计 defines the large-segment predicate; section 实现逻辑
 *       describes the push-style return and the weighted sum on the source.
 *  [P3] CANN 9.1.0-beta.3 API reference, "aclnnMoeDistributeDispatchV4":
 *       接口功能 / 计算公式 (optional quantisation, then expandXOut =
 *       AllToAllV(X)), the quantMode list (2 = per-token dynamic
 *       quantisation, dynamicScalesOut only in that mode), and 约束说明
 *       (deterministic by default).
 *
 * Readings taken where the pages leave a step open (each one is also listed in
 * the design notes):
 *  - expert e lives on rank r = e / epr as local expert el = e % epr;
 *  - src_token_id is the token index inside its source rank, tok in [0, bs);
 *  - a rank's segments are ordered local-expert-major, source-rank-minor
 *    (index el*W + s), which matches the (epWorldSize*localExpertNum,) shape
 *    of epRecvCountsOut in [P3];
 *  - "cumulative" means an inclusive prefix sum over that index;
 *  - rows inside one segment are in ascending src_token order;
 *  - the emulated per-rank windows are packed back to back, rank 0 first,
 *    so expand_x holds exactly N*K rows;
 *  - quantMode 1 (static; [P3] 参数说明 gives the coefficient input three
 *    shapes: one value (1,), a smoothing vector shared by all experts (H,),
 *    or per-expert coefficients fused with smoothing (E, H); the formula
 *    itself is garbled): the coefficient multiplies the token and the exact
 *    product is rounded to the nearest integer, ties to even, then saturated
 *    to int8's range [-128, 127] (computed in double, where the product of a
 *    16-bit float and a binary32 value is exact); c is qscale[0], qscale[j]
 *    or qscale[e*h + j] for a row of expert e; a NaN product gives -128 (the
 *    C fmax/fmin rule: the number wins over NaN); no dynamic scales;
 *  - quantMode 2: scale = max|x| / 127 in fp32, q = rint(x / scale) with
 *    ties to even, clamped to [-127, 127]; an all-zero token gets scale 0 and
 *    q = 0; one scale per expand_x row;
 *  - quantMode 3 (per-group dynamic; [P3] lists it with garbled output types
 *    and a garbled group size): groups of 128 consecutive elements of a token
 *    (the last one shorter when 128 does not divide h); per group
 *    scale = max|x| / 448 in fp32 (448 = largest finite E4M3); code = the
 *    OCP FP8 E4M3 ("fn") value nearest to the correctly rounded quotient
 *    x / scale, ties to even, after clamping the quotient to [-448, 448]; the
 *    code keeps the sign of x (so -0 gives 0x80); an all-zero group gets
 *    scale 0 and codes 0x00; G = ceil(h / 128) scales per expand_x row;
 *  - quantMode 4 ("mx" dynamic quantisation; [P3] lists it with four output
 *    types, a garbled scale shape and no scale input; the two types that need
 *    an even H are the 4-bit ones): the OCP Microscaling (MX) format v1.0
 *    with E4M3 elements (MXFP8), the 8-bit member that quantMode 3 already
 *    fixes the element encoding for. Blocks of 32 consecutive elements of a
 *    token (the last one shorter when 32 does not divide h); per block the
 *    shared exponent is floor(log2(max|x|)) - 8 (8 = the exponent of E4M3's
 *    largest normal, 448 = 1.75 * 2^8), clamped to E8M0's range [-127, 127]
 *    (-127 for an all-zero block); the scale byte is that exponent + 127
 *    (E8M0: the value 2^(byte - 127)); code = the E4M3 value nearest to
 *    x * 2^-shared (exact in binary64), ties to even, after clamping to
 *    [-448, 448], with the sign of x (-0 gives 0x80 in every block);
 *    B = ceil(h / 32) scale bytes per expand_x row. Inputs are finite; the
 *    other three element types are not built;
 *  - combine accumulates in fp32 with one fused multiply-add per k, k
 *    ascending from 0.0f, and rounds once (to nearest even) to the output
 *    type; int32 data combine in wrapping 32-bit integer arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_INT32 = 0, OR_FP16 = 1, OR_BF16 = 2 };
enum { MX_BLOCK = 32 };                    /* elements per quantMode 4 scale block */
enum { OR_OK = 0, OR_BAD_ARG = -1, OR_BAD_ID = -2, OR_DUP_ID = -3, OR_BAD_ASSIST = -4 };

/* ------------------------------------------------------------------------ */
/* Scalar type conversions, written from the IEEE 754 binary16 and bfloat16  */
/* definitions (sign, biased exponent, fraction).                            */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
float oracle_f16_to_f32(uint16_t v)
{
    int sign = (v >> 15) & 1;
    int expo = (v >> 10) & 0x1f;
    int frac = v & 0x3ff;
    float mag;
    if (expo == 0)
        mag = ldexpf((float)frac, -24);                 /* subnormal: frac * 2^-24 */
    else if (expo == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexpf((float)(1024 + frac), expo - 25);  /* (1 + frac/1024) * 2^(expo-15) */
    return sign ? -mag : mag;
}

/* Round a float to the nearest binary16 value, ties to even. The quantum
 * (spacing of representable values) is 2^-24 below 2^-14 and 2^(E-10) for a
 * value in [2^E, 2^(E+1)); the value divided by its quantum is rounded to an
 * integer with rint (ties to even), which is exact because both are powers of
 * two apart. Anything that rounds to 2^16 or above is infinite. */
uint16_t oracle_f32_to_f16(float f)
{
    uint16_t sign = (f32_bits(f) >> 31) ? 0x8000 : 0;
    float a = fabsf(f);
    if (isnan(f))
        return sign | 0x7e00;
    if (a == 0.0f)
        return sign;
    if (a < ldexpf(1.0f, -14)) {                       /* subnormal range */
        float n = rintf(a / ldexpf(1.0f, -24));        /* 0..1024 */
        return sign | (uint16_t)n;                     /* 1024 encodes 2^-14 exactly */
    }
    int e2;
    frexpf(a, &e2);                                    /* a = m * 2^e2, m in [0.5,1) */
    int E = e2 - 1;                                    /* a in [2^E, 2^(E+1)) */
    float n = rintf(ldexpf(a, 10 - E));                /* in [1024, 2048] */
    if (n == 2048.0f) { n = 1024.0f; E += 1; }
    if (E + 15 >= 31)
        return sign | 0x7c00;
    return sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)n - 1024);
}

/* bfloat16 is the top half of a binary32. */
float oracle_bf16_to_f32(uint16_t v) { return bits_f32((uint32_t)v << 16); }

/* Keep the upper 16 bits of the binary32 encoding and round on the lower 16:
 * above half rounds up, below half down, exactly half to the even neighbour.
 * A carry out of the fraction moves into the exponent, which is the correct
 * next value (and reaches infinity past the largest finite bfloat16). */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u = f32_bits(f);
    if (isnan(f))
        return (uint16_t)((u >> 16) | 0x0040);
    uint32_t hi = u >> 16, lo = u & 0xffff;
    if (lo > 0x8000 || (lo == 0x8000 && (hi & 1)))
        hi += 1;
    return (uint16_t)hi;
}

/* OCP 8-bit floating point E4M3, "fn" variant: 1 sign bit, 4 exponent bits
 * (bias 7), 3 fraction bits, no infinities; exponent 15 with fraction 7 is
 * NaN, so the largest finite value is 1.75 * 2^8 = 448. Normal values are
 * (1 + f/8) * 2^(e-7), subnormals (e = 0) f * 2^-9. */
float oracle_e4m3_to_f32(uint8_t v)
{
    int sign = v >> 7, expo = (v >> 3) & 15, frac = v & 7;
    float mag;
    if (expo == 15 && frac == 7)
        mag = NAN;
    else if (expo == 0)
        mag = ldexpf((float)frac, -9);
    else
        mag = ldexpf((float)(8 + frac), expo - 10);
    return sign ? -mag : mag;
}

/* Nearest E4M3 value, ties to even, for |f| <= 448 (callers clamp first).
 * Same quantum argument as for binary16: the spacing is 2^-9 below 2^-6 and
 * 2^(E-3) in [2^E, 2^(E+1)), so value / quantum is rounded with rint. */
uint8_t oracle_f32_to_e4m3(float f)
{
    uint8_t sign = (f32_bits(f) >> 31) ? 0x80 : 0;
    float a = fabsf(f);
    if (a == 0.0f)
        return sign;
    if (a < ldexpf(1.0f, -6)) {
        float n = rintf(a / ldexpf(1.0f, -9));         /* 0..8; 8 encodes 2^-6 */
        return sign | (uint8_t)n;
    }
    int e2;
    frexpf(a, &e2);
    int E = e2 - 1;                                    /* a in [2^E, 2^(E+1)) */
    float n = rintf(ldexpf(a, 3 - E));                 /* in [8, 16] */
    if (n == 16.0f) { n = 8.0f; E += 1; }
    return sign | (uint8_t)((E + 7) << 3) | (uint8_t)((int)n - 8);
}

static float load_f32(const void *base, size_t i, int dtype)
{
    const uint16_t *p = (const uint16_t *)base;
    return dtype == OR_FP16 ? oracle_f16_to_f32(p[i]) : oracle_bf16_to_f32(p[i]);
}

static uint16_t store_16(float v, int dtype)
{
    return dtype == OR_FP16 ? oracle_f32_to_f16(v) : oracle_f32_to_bf16(v);
}

static size_t elem_size(int dtype) { return dtype == OR_INT32 ? 4 : 2; }

/* ------------------------------------------------------------------------ */
/* Dispatch                                                                  */
/* ------------------------------------------------------------------------ */

/*
 * Pair (t, k) takes part unless a token mask says otherwise ([P3] 参数说明,
 * xActiveMaskOptional: a 1D mask (BS,) per rank, or a 2D mask (BS, K); a token
 * whose K entries are all false is not exchanged). mask_kind 0: no mask;
 * 1: mask[t], one byte per token of all W*bs tokens; 2: mask[t*K + k]; a
 * nonzero byte is true. Reading taken: an inactive pair is not sent at all. It
 * gets no row and is not counted, and its expert id is never read, so it is
 * not checked either. Rows stay packed, so expand_x holds A rows, A = number
 * of active pairs, and the buffers may be sized for N*K. The 1D rule that true
 * entries come first is not needed by this definition, so any pattern is
 * accepted.
 */
/*
 * Special experts ([P3] 参数说明, zeroExpertNum / copyExpertNum /
 * constExpertNum): ids in [E, E + zero) are zero experts, ids in
 * [E + zero, E + zero + copy) copy experts, ids in
 * [E + zero + copy, E + zero + copy + const) const experts. The pages give only
 * the id ranges; reading taken: a special pair is not exchanged (no row, no
 * count); in the combine, at the pair's place in the k order, a zero expert
 * contributes nothing, a copy expert the token itself, ori_x[t] * weight, and
 * const expert j a fixed vector, const_x[j] * weight (the same for every
 * token: the plainest meaning of an expert whose output is constant).
 */
static int pair_active(const uint8_t *mask, int mask_kind, long long t, int k, int K)
{
    if (mask_kind == 1) return mask[t] != 0;
    if (mask_kind == 2) return mask[t * K + k] != 0;
    return 1;
}

/*
 * x            [W*bs, h] dtype           tokens, source rank s owns rows s*bs..s*bs+bs-1
 * ids          [W*bs, K] int32           global expert ids, distinct per token
 * qscale       fp32 [qscale_n]           quant == 1 only: qscale_n is 1, h or E*h
 * expand_x     [W*bs*K, h]               dtype; int8 when quant is 1 or 2; E4M3 bytes when 3 or 4
 * dyn_scales   [W*bs*K] fp32             quant == 2: one scale per row;
 *              [W*bs*K, G] fp32          quant == 3: G = ceil(h / 128) group scales per row
 *              [W*bs*K, B] uint8         quant == 4: B = ceil(h / 32) E8M0 block scales per row
 * assist       [W*bs*K, 3] int32         (src_rank, src_token, topk_id) per row
 * ep_recv_count[W, epr*W] int32          inclusive per-rank segment counts
 * expand_scales[W*bs*K] fp32|int32|NULL  expert_scales[t,k] moved to row(t,k)
 *
 * The steps are the plain counting sort by expert that the all-to-all of
 * [P3] 计算公式 amounts to when every rank's window sits in one memory.
 */
int oracle_dispatch(const void *x, const int32_t *ids, const void *expert_scales,
                    int W, int bs, int epr, int h, int K, int dtype, int quant,
                    const float *qscale, long long qscale_n, const uint8_t *mask, int mask_kind, int zero_num,
                    int copy_num, int const_num,
                    void *expand_x, void *dyn_scales, int32_t *assist,
                    int32_t *ep_recv_count, void *expand_scales)
{
    if (W < 1 || bs < 0 || epr < 1 || h < 1 || K < 1) return OR_BAD_ARG;
    if (mask_kind < 0 || mask_kind > 2 || (mask_kind != 0) != (mask != NULL)) return OR_BAD_ARG;
    if (zero_num < 0 || copy_num < 0 || const_num < 0) return OR_BAD_ARG;
    if (quant < 0 || quant > 4) return OR_BAD_ARG;
    if (quant != 0 && dtype == OR_INT32) return OR_BAD_ARG;
    const int G = (h + 127) / 128;                     /* quantMode 3 groups per row */
    const int B = (h + MX_BLOCK - 1) / MX_BLOCK;       /* quantMode 4 blocks per row */
    const long long E = (long long)W * epr, N = (long long)W * bs, S = (long long)epr * W;
    if (K > E) return OR_BAD_ARG;
    if (quant == 1 && (!qscale || (qscale_n != 1 && qscale_n != h && qscale_n != E * h))) return OR_BAD_ARG;

    /* Step 1: count the (token, k) pairs of every segment (r, el*W + s). */
    long long *cnt = calloc((size_t)(W * S), sizeof(long long));
    if (!cnt) return OR_BAD_ARG;
    for (long long t = 0; t < N; ++t) {
        for (int k = 0; k < K; ++k) {
            if (!pair_active(mask, mask_kind, t, k, K)) continue;
            int32_t e = ids[t * K + k];
            if (e < 0 || (long long)e >= E + zero_num + copy_num + const_num) { free(cnt); return OR_BAD_ID; }
            for (int j = 0; j < k; ++j)
                if (pair_active(mask, mask_kind, t, j, K) && ids[t * K + j] == e) { free(cnt); return OR_DUP_ID; }
            if (e >= E) continue;                      /* special expert: not exchanged */
            long long r = e / epr, el = e % epr, s = t / bs;
            cnt[r * S + el * W + s] += 1;
        }
    }

    /* Step 2: inclusive prefix per rank -> ep_recv_count; window base B_r. */
    long long *base = malloc((size_t)W * sizeof(long long));
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

    /* Steps 3-6: walk tokens in order; each pair takes the next free row of
     * its segment, so rows inside a segment come out in ascending src_token. */
    long long *fill = calloc((size_t)(W * S), sizeof(long long));
    const size_t xs = elem_size(dtype);
    for (long long t = 0; t < N; ++t) {
        long long s = t / bs, tok = t % bs;
        int any = 0;
        for (int k = 0; k < K; ++k) any |= pair_active(mask, mask_kind, t, k, K) && ids[t * K + k] < E;
        if (!any) continue;
        float scale = 0.0f;
        if (quant == 2) {
            float amax = 0.0f;
            for (int j = 0; j < h; ++j) {
                float v = fabsf(load_f32(x, (size_t)(t * h + j), dtype));
                if (v > amax) amax = v;
            }
            scale = amax / 127.0f;
        }
        for (int k = 0; k < K; ++k) {
            if (!pair_active(mask, mask_kind, t, k, K)) continue;
            int32_t e = ids[t * K + k];
            if (e >= E) continue;
            long long r = e / epr, el = e % epr, i = el * W + s;
            long long start = i == 0 ? 0 : ep_recv_count[r * S + i - 1];
            long long row = base[r] + start + fill[r * S + i];
            fill[r * S + i] += 1;

            assist[row * 3 + 0] = (int32_t)s;
            assist[row * 3 + 1] = (int32_t)tok;
            assist[row * 3 + 2] = k;

            if (expand_scales)   /* fp32 and int32 scales are both 4-byte words */
                memcpy((char *)expand_scales + row * 4, (const char *)expert_scales + (t * K + k) * 4, 4);

            if (quant == 0) {
                memcpy((char *)expand_x + (size_t)row * h * xs, (const char *)x + (size_t)t * h * xs,
                       (size_t)h * xs);
            } else if (quant == 1) {
                int8_t *q = (int8_t *)expand_x + (size_t)row * h;
                for (int j = 0; j < h; ++j) {
                    float c = qscale_n == 1 ? qscale[0] : qscale_n == h ? qscale[j] : qscale[(long long)e * h + j];
                    double p = (double)load_f32(x, (size_t)(t * h + j), dtype) * (double)c;   /* exact */
                    double n = rint(p);
                    n = fmax(n, -128.0);
                    n = fmin(n, 127.0);
                    q[j] = (int8_t)n;
                }
            } else if (quant == 3) {
                uint8_t *q = (uint8_t *)expand_x + (size_t)row * h;
                for (int g = 0; g < G; ++g) {
                    int j0 = g * 128, j1 = j0 + 128 < h ? j0 + 128 : h;
                    float amax = 0.0f;
                    for (int j = j0; j < j1; ++j) {
                        float v = fabsf(load_f32(x, (size_t)(t * h + j), dtype));
                        if (v > amax) amax = v;
                    }
                    float gs = amax / 448.0f;
                    for (int j = j0; j < j1; ++j) {
                        float v = load_f32(x, (size_t)(t * h + j), dtype);
                        if (gs == 0.0f) { q[j] = 0; continue; }
                        float n = v / gs;
                        if (n > 448.0f) n = 448.0f;
                        if (n < -448.0f) n = -448.0f;
                        q[j] = oracle_f32_to_e4m3(n);
                    }
                    ((float *)dyn_scales)[row * G + g] = gs;
                }
            } else if (quant == 4) {
                uint8_t *q = (uint8_t *)expand_x + (size_t)row * h;
                uint8_t *sb = (uint8_t *)dyn_scales + (size_t)row * B;
                for (int b = 0; b < B; ++b) {
                    int j0 = b * MX_BLOCK, j1 = j0 + MX_BLOCK < h ? j0 + MX_BLOCK : h;
                    double amax = 0.0;
                    for (int j = j0; j < j1; ++j) {
                        double v = fabs((double)load_f32(x, (size_t)(t * h + j), dtype));
                        if (v > amax) amax = v;
                    }
                    int shared = -127;                 /* all-zero block */
                    if (amax > 0.0) {
                        int e2;
                        frexp(amax, &e2);              /* amax in [2^(e2-1), 2^e2) */
                        shared = (e2 - 1) - 8;
                        if (shared < -127) shared = -127;
                        if (shared > 127) shared = 127;
                    }
                    sb[b] = (uint8_t)(shared + 127);
                    for (int j = j0; j < j1; ++j) {
                        double n = ldexp((double)load_f32(x, (size_t)(t * h + j), dtype), -shared);
                        if (n > 448.0) n = 448.0;
                        if (n < -448.0) n = -448.0;
                        q[j] = oracle_f32_to_e4m3((float)n);
                    }
                }
            } else {
                int8_t *q = (int8_t *)expand_x + (size_t)row * h;
                for (int j = 0; j < h; ++j) {
                    float v = load_f32(x, (size_t)(t * h + j), dtype);
                    float n = scale == 0.0f ? 0.0f : rintf(v / scale);
                    if (n > 127.0f) n = 127.0f;
                    if (n < -127.0f) n = -127.0f;
                    q[j] = (int8_t)n;
                }
                ((float *)dyn_scales)[row] = scale;
            }
        }
    }
    free(fill);
    free(base);
    free(cnt);
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Combine                                                                   */
/* ------------------------------------------------------------------------ */

static int is_copy(const int32_t *ids, const uint8_t *mask, int mask_kind, long long t, int k, int K,
                   long long E, int zero_num, int copy_num)
{
    long long e = ids[t * K + k];
    return pair_active(mask, mask_kind, t, k, K) && e >= E + zero_num && e < E + zero_num + copy_num;
}

/* Index j of the const expert of pair (t, k), or -1 when it is not an active
 * const-expert pair. */
static long long const_index(const int32_t *ids, const uint8_t *mask, int mask_kind, long long t, int k, int K,
                             long long E, int zero_num, int copy_num, int const_num)
{
    long long e = ids[t * K + k], c0 = E + zero_num + copy_num;
    return pair_active(mask, mask_kind, t, k, K) && e >= c0 && e < c0 + const_num ? e - c0 : -1;
}

/*
 * Push-style, as [P1] 实现逻辑 describes it: every expert-output row is
 * returned to slot (src_token, topk_id) of its source rank's window; the
 * source then forms, per token, the weighted sum of its K returned rows
 * ([P1] 功能说明, check formula).
 *
 * expand_x [rows, h] dtype (fp16/bf16/int32), scales [W*bs, K] fp32 (int32 for
 * int32 data), x_out [W*bs, h] dtype. The row's segment (hence its expert) is
 * recovered from ep_recv_count and must equal ids[t,k]; every active (t,k)
 * slot must be filled exactly once and no inactive one (same mask as the
 * dispatch). The sum runs over the active pairs in ascending k; a token with
 * none gets 0 (reading: the pages say nothing about the output of a token
 * that was not exchanged). Special experts contribute as described above
 * (ori_x [N, h] and const_x [const_num, h], in the dtype of expand_x).
 */
int oracle_combine(const void *expand_x, const int32_t *assist, const int32_t *ep_recv_count,
                   const int32_t *ids, const void *scales, int W, int bs, int epr, int h, int K,
                   int dtype, const uint8_t *mask, int mask_kind, int zero_num, int copy_num, int const_num,
                   const void *ori_x, const void *const_x, void *x_out)
{
    if (W < 1 || bs < 0 || epr < 1 || h < 1 || K < 1) return OR_BAD_ARG;
    if (mask_kind < 0 || mask_kind > 2 || (mask_kind != 0) != (mask != NULL)) return OR_BAD_ARG;
    if (zero_num < 0 || copy_num < 0 || (copy_num > 0 && !ori_x)) return OR_BAD_ARG;
    if (const_num < 0 || (const_num > 0 && !const_x)) return OR_BAD_ARG;
    const long long N = (long long)W * bs, S = (long long)epr * W, E = (long long)W * epr;

    long long rows = 0, active = 0;
    for (long long r = 0; r < W; ++r) rows += ep_recv_count[r * S + S - 1];
    for (long long t = 0; t < N; ++t)
        for (int k = 0; k < K; ++k) active += pair_active(mask, mask_kind, t, k, K) && ids[t * K + k] < E;
    if (rows != active) return OR_BAD_ASSIST;

    /* The source rank's window: slot[t*K + k] = index of the returned row. */
    long long *slot = malloc((size_t)(N * K > 0 ? N * K : 1) * sizeof(long long));
    for (long long i = 0; i < N * K; ++i) slot[i] = -1;

    long long row = 0;
    for (long long r = 0; r < W; ++r) {
        long long prev = 0;
        for (long long i = 0; i < S; ++i) {
            long long end = ep_recv_count[r * S + i];
            long long e = r * epr + i / W;          /* segment index = el*W + s */
            for (long long c = prev; c < end; ++c, ++row) {
                long long s = assist[row * 3 + 0], tok = assist[row * 3 + 1], k = assist[row * 3 + 2];
                if (s != i % W || tok < 0 || tok >= bs || k < 0 || k >= K) { free(slot); return OR_BAD_ASSIST; }
                long long t = s * bs + tok;
                if (!pair_active(mask, mask_kind, t, (int)k, K) || ids[t * K + k] != e || slot[t * K + k] != -1) {
                    free(slot);
                    return OR_BAD_ASSIST;
                }
                slot[t * K + k] = row;
            }
            prev = end;
        }
    }

    for (long long t = 0; t < N; ++t) {
        for (int j = 0; j < h; ++j) {
            if (dtype == OR_INT32) {
                uint32_t acc = 0;
                for (int k = 0; k < K; ++k) {
                    int32_t sc = ((const int32_t *)scales)[t * K + k];
                    long long cj = const_index(ids, mask, mask_kind, t, k, K, E, zero_num, copy_num, const_num);
                    if (slot[t * K + k] >= 0) {
                        const int32_t *y = (const int32_t *)expand_x + (size_t)slot[t * K + k] * h;
                        acc += (uint32_t)y[j] * (uint32_t)sc;
                    } else if (is_copy(ids, mask, mask_kind, t, k, K, E, zero_num, copy_num)) {
                        acc += (uint32_t)((const int32_t *)ori_x)[t * h + j] * (uint32_t)sc;
                    } else if (cj >= 0) {
                        acc += (uint32_t)((const int32_t *)const_x)[cj * h + j] * (uint32_t)sc;
                    }
                }
                ((int32_t *)x_out)[t * h + j] = (int32_t)acc;
            } else {
                float acc = 0.0f;
                for (int k = 0; k < K; ++k) {
                    float sc = ((const float *)scales)[t * K + k];
                    long long cj = const_index(ids, mask, mask_kind, t, k, K, E, zero_num, copy_num, const_num);
                    if (slot[t * K + k] >= 0)
                        acc = fmaf(load_f32(expand_x, (size_t)slot[t * K + k] * h + j, dtype), sc, acc);
                    else if (is_copy(ids, mask, mask_kind, t, k, K, E, zero_num, copy_num))
                        acc = fmaf(load_f32(ori_x, (size_t)(t * h + j), dtype), sc, acc);
                    else if (cj >= 0)
                        acc = fmaf(load_f32(const_x, (size_t)(cj * h + j), dtype), sc, acc);
                }
                ((uint16_t *)x_out)[t * h + j] = store_16(acc, dtype);
            }
        }
    }
    free(slot);
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Large-segment predicate ([P1] 方案设计)                                   */
/* ------------------------------------------------------------------------ */

/*
 * For every segment (el, s) of every rank r, flag[r*S + el*W + s] = 1 when
 *   s != r, the segment is non-empty, its payload bytes are at least
 *   threshold_bytes, and its payload bytes exceed the mean payload of rank r's
 *   remote segments. The mean is compared by cross-multiplication, with
 *   num = (rows r receives from other ranks) * h * elem_bytes and
 *   den = max(W - 1, 1) * epr, all in 64-bit integers.
 */
int oracle_large_segments(const int32_t *ep_recv_count, int W, int epr, int h, int elem_bytes,
                          long long threshold_bytes, uint8_t *flag)
{
    const long long S = (long long)epr * W;
    for (long long r = 0; r < W; ++r) {
        long long remote = 0;
        for (long long i = 0; i < S; ++i) {
            long long c = ep_recv_count[r * S + i] - (i ? ep_recv_count[r * S + i - 1] : 0);
            if (i % W != r) remote += c;
        }
        long long num = remote * h * elem_bytes;
        long long den = (long long)(W - 1 > 1 ? W - 1 : 1) * epr;
        for (long long i = 0; i < S; ++i) {
            long long c = ep_recv_count[r * S + i] - (i ? ep_recv_count[r * S + i - 1] : 0);
            long long bytes = c * h * elem_bytes;
            flag[r * S + i] = (i % W != r) && c > 0 && bytes >= threshold_bytes && bytes * den > num;
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Identity expert for int8 rows (harness, not part of the method)           */
/* ------------------------------------------------------------------------ */

/* y[i, j] = bf16(f32(q[i, j]) * scale[i]): what an identity expert hands to
 * combine when dispatch quantised its input; one fp32 product, one rounding. */
/* The same for E4M3 rows with per-group scales: bf16(f32(e4m3) * scale[g]). */
void oracle_identity_expert_dequant_fp8(const uint8_t *q, const float *scale, long long rows, int h,
                                        uint16_t *y)
{
    const int G = (h + 127) / 128;
    for (long long i = 0; i < rows; ++i)
        for (int j = 0; j < h; ++j)
            y[i * h + j] = oracle_f32_to_bf16(oracle_e4m3_to_f32(q[i * h + j]) * scale[i * G + j / 128]);
}

/* The same for MX rows: bf16(f32(e4m3) * 2^(byte - 127)), one E8M0 byte per
 * block of 32 (the product is exact in binary32 for the bytes a finite 16-bit
 * token can produce, so the bf16 conversion is the one rounding). */
void oracle_identity_expert_dequant_mx(const uint8_t *q, const uint8_t *scale, long long rows, int h,
                                       uint16_t *y)
{
    const int B = (h + MX_BLOCK - 1) / MX_BLOCK;
    for (long long i = 0; i < rows; ++i)
        for (int j = 0; j < h; ++j)
            y[i * h + j] = oracle_f32_to_bf16(ldexpf(oracle_e4m3_to_f32(q[i * h + j]),
                                                     (int)scale[i * B + j / MX_BLOCK] - 127));
}

void oracle_identity_expert_dequant(const int8_t *q, const float *scale, long long rows, int h,
                                    uint16_t *y)
{
    for (long long i = 0; i < rows; ++i)
        for (int j = 0; j < h; ++j)
            y[i * h + j] = oracle_f32_to_bf16((float)q[i * h + j] * scale[i]);
}
