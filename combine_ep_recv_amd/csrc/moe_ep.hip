// moe_ep.hip -- MoE token dispatch and combine for MI355X (gfx950, wave64).
//
// The C ABI declared in include/moe_ep.h. Pure data movement plus an axpy:
// no MFMA anywhere; every kernel is bounded by HBM bandwidth or latency.
//
// Dispatch (aclnnMoeDistributeDispatchV4, 计算公式: expandXOut = AllToAllV(X),
// with every logical rank's receive window a partition of one HBM):
//   route    one block per (source rank, 256-token chunk). Builds, in LDS, a
//            bitmap per expert over the chunk's tokens (ds_or_b64), then
//            writes the chunk's per-expert counts and, for every (t, k), the
//            number of earlier tokens of the chunk routed to the same expert
//            (a popcount of the bitmap below the token). Bit-set order does
//            not matter, so the result is deterministic with no sort.
//   scan     one block of 1024 threads, one expert column per thread: the
//            row offset of every (chunk, expert) block, ep_recv_count
//            (inclusive, el-major, per rank; combine_doubleplane README
//            功能说明), and, when asked, the large-segment predicate of the
//            README's 方案设计 and the segment work plan.
//   scatter  token-major (default): one block per token reads its row once
//            with 128-bit loads and writes the K copies (optionally int8
//            quantised with one fp32 scale per token) plus assist_info.
//            Segment-major (optional): a metadata pass, then blocks walk
//            expand_x in destination order following the plan.
// Combine (README 功能说明, check formula): one block per token recovers
//   row(t, k) from ep_recv_count and assist_info, gathers the K rows with
//   128-bit loads and accumulates in fp32 with one FMA per k (k ascending),
//   rounding once to the output type.

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "moe_ep.h"

namespace {

constexpr int kThreads = 256;              // route / scatter / combine block size
constexpr int kScanThreads = 1024;         // the single scan block (>= max experts)
constexpr int kRouteTokens = 256;          // tokens per route block
constexpr int kRouteWords = kRouteTokens / 64;
constexpr int kMaxExperts = 1024;          // moeExpertNum upper bound
constexpr int kMinWorld = 2, kMaxWorld = 768;   // epWorldSize range
constexpr int kSegLdsMax = 11264;          // W*S limit for the LDS-resident segment counts
constexpr long long kMaxTokens = (1ll << 24) - 1;   // N blocks of 256 threads stay below 2^32 items
constexpr int kPlanRows = 8;               // rows per segment-schedule work item
constexpr int kSegGrid = 4096;             // blocks of the segment-major payload pass
constexpr int64_t kReadmeLargeBytes = 2 * 1024 * 1024;
constexpr int kRowUnroll = 4;              // 16-byte chunks held per thread in the scatter

// --------------------------------------------------------------------------
// element conversions (gfx950: v_cvt_f32_f16 / v_cvt_f16_f32 / v_cvt_pk_bf16_f32,
// all round-to-nearest-even)
// --------------------------------------------------------------------------

struct F16 {
    static __device__ __forceinline__ float load(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
    static __device__ __forceinline__ uint16_t store(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
};
struct BF16 {
    static __device__ __forceinline__ float load(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
    static __device__ __forceinline__ uint16_t store(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
};

// --------------------------------------------------------------------------
// block-level helpers
// --------------------------------------------------------------------------

__device__ __forceinline__ int wave_incl_scan(int v)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int o = __shfl_up(v, d, 64);
        if (lane >= d) v += o;
    }
    return v;
}

// Exclusive prefix of one int per thread over the block; *total gets the sum.
// tmp: >= 33 ints of LDS. Every thread of the block must call it.
__device__ int block_excl_scan(int v, int *tmp, int *total)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int incl = wave_incl_scan(v);
    if (lane == 63) tmp[wid] = incl;
    __syncthreads();
    if (wid == 0) {
        const int w = lane < nw ? tmp[lane] : 0;
        const int wi = wave_incl_scan(w);
        if (lane < nw) tmp[lane] = wi - w;
        if (lane == nw - 1) tmp[32] = wi;
    }
    __syncthreads();
    const int res = tmp[wid] + incl - v;
    *total = tmp[32];
    __syncthreads();
    return res;
}

__device__ __forceinline__ float block_max(float v, float *tmp)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
    if (lane == 0) tmp[wid] = v;
    __syncthreads();
    float m = tmp[0];
    for (int i = 1; i < nw; ++i) m = fmaxf(m, tmp[i]);
    __syncthreads();
    return m;
}

// Exclusive prefix over ranks of the rank totals ep_recv_count[r][S-1]:
// out[r] = first row of rank r's window; out[W] = all rows.
__device__ void rank_bases(const int32_t *__restrict__ erc, int W, int S, int32_t *out, int *tmp)
{
    const int per = (W + (int)blockDim.x - 1) / (int)blockDim.x;   // <= 3 for W <= 768
    const int i0 = threadIdx.x * per;
    int v[3] = {0, 0, 0};
    int sum = 0;
#pragma unroll
    for (int j = 0; j < 3; ++j)
        if (j < per && i0 + j < W) { v[j] = erc[(size_t)(i0 + j) * S + S - 1]; sum += v[j]; }
    int total;
    int ex = block_excl_scan(sum, tmp, &total);
#pragma unroll
    for (int j = 0; j < 3; ++j)
        if (j < per && i0 + j < W) { out[i0 + j] = ex; ex += v[j]; }
    if (threadIdx.x == 0) out[W] = total;
}

// --------------------------------------------------------------------------
// route
// --------------------------------------------------------------------------

__global__ __launch_bounds__(kThreads) void route_kernel(const int32_t *__restrict__ ids, int W, int bs,
                                                         int epr, int K, int nbs,
                                                         int32_t *__restrict__ cnt,
                                                         int32_t *__restrict__ lr)
{
    extern __shared__ unsigned long long bm[];   // [E][kRouteWords]
    const int E = W * epr;
    const int b = blockIdx.x, s = b / nbs, j = b % nbs;
    const int tok0 = j * kRouteTokens;
    const int ntok = min(kRouteTokens, bs - tok0);
    const int npairs = ntok * K;
    const size_t pair0 = ((size_t)s * bs + tok0) * K;

    for (int i = threadIdx.x; i < E * kRouteWords; i += blockDim.x) bm[i] = 0ull;
    __syncthreads();
    for (int p = threadIdx.x; p < npairs; p += blockDim.x) {
        const int e = ids[pair0 + p];
        if ((unsigned)e < (unsigned)E) {
            const int tl = p / K;
            atomicOr(&bm[e * kRouteWords + (tl >> 6)], 1ull << (tl & 63));
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < kRouteWords; ++w) c += __popcll(bm[e * kRouteWords + w]);
        cnt[(size_t)b * E + e] = c;
    }
    for (int p = threadIdx.x; p < npairs; p += blockDim.x) {
        const int e = ids[pair0 + p];
        int rank = -1;
        if ((unsigned)e < (unsigned)E) {
            const int tl = p / K, wi = tl >> 6;
            const unsigned long long *row = &bm[e * kRouteWords];
            int c = __popcll(row[wi] & ((1ull << (tl & 63)) - 1ull));
            for (int w = 0; w < wi; ++w) c += __popcll(row[w]);
            rank = c;
        }
        lr[pair0 + p] = rank;
    }
}

// --------------------------------------------------------------------------
// scan (+ large-segment predicate and segment plan)
// --------------------------------------------------------------------------

// Walk rank r's segments in order and emit the work items of the segment
// schedule: a large segment is cut into items of its own of at most `rows`
// rows; runs of other segments are packed into items of exactly `rows` rows
// (the last one shorter). Returns the number of items; writes them when
// `plan` is non-null. The count pass and the write pass share this code.
__device__ int plan_rank(const int32_t *segc, const uint8_t *flag, int S, int row0, int rows, int2 *plan)
{
    int n = 0, row = row0, pack_start = row0, run = 0;
    for (int i = 0; i < S; ++i) {
        const int c = segc[i];
        if (flag[i]) {
            if (run) { if (plan) plan[n] = make_int2(pack_start, row); ++n; run = 0; }
            for (int q = 0; q < c; q += rows) {
                if (plan) plan[n] = make_int2(row + q, row + min(c, q + rows));
                ++n;
            }
            row += c;
            pack_start = row;
        } else {
            run += c;
            row += c;
            while (run >= rows) {
                if (plan) plan[n] = make_int2(pack_start, pack_start + rows);
                ++n;
                pack_start += rows;
                run -= rows;
            }
        }
    }
    if (run) { if (plan) plan[n] = make_int2(pack_start, row); ++n; }
    return n;
}

__global__ __launch_bounds__(kScanThreads) void scan_kernel(
    const int32_t *__restrict__ cnt, int W, int epr, int nbs, int h, int elem_bytes,
    int32_t *__restrict__ boff, int32_t *__restrict__ erc, int want_seg, long long large_bytes,
    int32_t *__restrict__ seg_flags, int2 *__restrict__ plan, int32_t *__restrict__ nplan)
{
    __shared__ int32_t eoff[kMaxExperts + 1];
    __shared__ int32_t tmp[40];
    extern __shared__ int32_t seg_lds[];          // when want_seg: int32 counts [W*S], then uint8 flags [W*S]
    const int E = W * epr, S = epr * W, NB = W * nbs;
    const int tid = threadIdx.x;

    // column totals -> exclusive offsets per expert (blockDim >= E)
    int tot = 0;
    if (tid < E)
        for (int b = 0; b < NB; ++b) tot += cnt[(size_t)b * E + tid];
    int total;
    const int ex = block_excl_scan(tot, tmp, &total);
    if (tid < E) eoff[tid] = ex;
    if (tid == 0) eoff[E] = total;
    __syncthreads();

    int32_t *segc = seg_lds;
    uint8_t *flag = reinterpret_cast<uint8_t *>(seg_lds + (size_t)W * S);
    if (tid < E) {
        const int e = tid, r = e / epr, el = e % epr;
        const int base_r = eoff[r * epr];
        int run = 0;
        for (int s = 0; s < W; ++s) {
            const int before = run;
            for (int j = 0; j < nbs; ++j) {
                const size_t b = (size_t)s * nbs + j;
                const int c = cnt[b * E + e];
                boff[b * E + e] = eoff[e] + run;
                run += c;
            }
            erc[(size_t)r * S + el * W + s] = eoff[e] + run - base_r;
            if (want_seg) segc[r * S + el * W + s] = run - before;
        }
    }
    if (!want_seg) return;
    __syncthreads();

    // large-segment predicate (combine_doubleplane README 方案设计), one rank per thread
    if (tid < W) {
        const int r = tid;
        long long remote = 0;
        for (int i = 0; i < S; ++i)
            if (i % W != r) remote += segc[r * S + i];
        const long long num = remote * h * elem_bytes;
        const long long den = (long long)(W - 1 > 1 ? W - 1 : 1) * epr;
        for (int i = 0; i < S; ++i) {
            const long long c = segc[r * S + i];
            const long long bytes = c * h * elem_bytes;
            const int large = (i % W != r) && c > 0 && bytes >= large_bytes && bytes * den > num;
            flag[r * S + i] = (uint8_t)large;
            if (seg_flags) seg_flags[(size_t)r * S + i] = large;
        }
    }
    if (!plan) return;
    __syncthreads();

    int mine = 0;
    if (tid < W) mine = plan_rank(segc + tid * S, flag + tid * S, S, eoff[tid * epr], kPlanRows, nullptr);
    int nitems;
    const int first = block_excl_scan(mine, tmp, &nitems);
    if (tid < W) plan_rank(segc + tid * S, flag + tid * S, S, eoff[tid * epr], kPlanRows, plan + first);
    if (tid == 0) *nplan = nitems;
}

// --------------------------------------------------------------------------
// dispatch payload
// --------------------------------------------------------------------------

// Row of every pair of token t (token-major schedule); writes assist_info and
// expand_scales for those rows. Invalid ids give row -1 (nothing written).
__device__ __forceinline__ void token_rows(int t, int s, int tok, const int32_t *__restrict__ ids,
                                           const int32_t *__restrict__ lr, const int32_t *__restrict__ boff,
                                           int E, int K, int nbs, int R, int32_t *rows,
                                           int32_t *__restrict__ assist, const int32_t *__restrict__ esc_in,
                                           int32_t *__restrict__ esc_out)
{
    const size_t b = (size_t)s * nbs + tok / kRouteTokens;
    for (int k = threadIdx.x; k < K; k += blockDim.x) {
        const size_t p = (size_t)t * K + k;
        const int e = ids[p], l = lr[p];
        int row = -1;
        if ((unsigned)e < (unsigned)E && l >= 0) {
            row = boff[b * E + e] + l;
            if ((unsigned)row >= (unsigned)R) row = -1;
        }
        rows[k] = row;
        if (row >= 0) {
            assist[(size_t)row * 3 + 0] = s;
            assist[(size_t)row * 3 + 1] = tok;
            assist[(size_t)row * 3 + 2] = k;
            if (esc_out) esc_out[row] = esc_in[p];
        }
    }
}

// Copy `rowbytes` bytes from src to each of the ndst destination rows.
template <bool VEC>
__device__ __forceinline__ void copy_row(const char *__restrict__ src, char *__restrict__ dst_base,
                                         const int32_t *rows, int ndst, size_t rowbytes)
{
    if (VEC) {
        const int nch = (int)(rowbytes / 16);
        for (int c0 = threadIdx.x; c0 < nch; c0 += kThreads * kRowUnroll) {
            uint4 v[kRowUnroll];
#pragma unroll
            for (int u = 0; u < kRowUnroll; ++u) {
                const int c = c0 + u * kThreads;
                if (c < nch) v[u] = reinterpret_cast<const uint4 *>(src)[c];
            }
            for (int k = 0; k < ndst; ++k) {
                const int row = rows[k];
                if (row < 0) continue;
                uint4 *dst = reinterpret_cast<uint4 *>(dst_base + (size_t)row * rowbytes);
#pragma unroll
                for (int u = 0; u < kRowUnroll; ++u) {
                    const int c = c0 + u * kThreads;
                    if (c < nch) dst[c] = v[u];
                }
            }
        }
    } else {
        const int n = (int)(rowbytes / 2);
        for (int c = threadIdx.x; c < n; c += kThreads) {
            const uint16_t v = reinterpret_cast<const uint16_t *>(src)[c];
            for (int k = 0; k < ndst; ++k)
                if (rows[k] >= 0) reinterpret_cast<uint16_t *>(dst_base + (size_t)rows[k] * rowbytes)[c] = v;
        }
    }
}

__device__ __forceinline__ int8_t quant1(float v, float scale)
{
    float q = scale == 0.0f ? 0.0f : __builtin_rintf(v / scale);
    q = fminf(fmaxf(q, -127.0f), 127.0f);
    return (int8_t)(int)q;
}

template <class T>
__device__ __forceinline__ uint2 quant8(uint4 v, float scale)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint16_t b = (uint16_t)(w[i >> 1] >> ((i & 1) * 16));
        const uint32_t q = (uint8_t)quant1(T::load(b), scale);
        o[i >> 2] |= q << ((i & 3) * 8);
    }
    return make_uint2(o[0], o[1]);
}

template <class T>
__device__ __forceinline__ float amax8(uint4 v)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(T::load((uint16_t)(w[i >> 1] >> ((i & 1) * 16)))));
    return m;
}

// Per-token dynamic int8 quantisation (aclnnMoeDistributeDispatchV4 quantMode 2):
// scale = max|x| / 127 (fp32, correctly rounded), q = rint(x / scale) clamped to
// [-127, 127] (0 for an all-zero token); q is written to every destination row.
// Returns the scale.
template <class T, bool VEC>
__device__ float quant_row(const uint16_t *__restrict__ src, int8_t *__restrict__ dst_base,
                           const int32_t *rows, int ndst, int h, float *red)
{
    float amax = 0.0f;
    if (VEC) {
        const int nch = h / 8;
        const uint4 *s4 = reinterpret_cast<const uint4 *>(src);
        if (nch <= kThreads * kRowUnroll) {
            uint4 v[kRowUnroll];
#pragma unroll
            for (int u = 0; u < kRowUnroll; ++u) {
                const int c = threadIdx.x + u * kThreads;
                if (c < nch) { v[u] = s4[c]; amax = fmaxf(amax, amax8<T>(v[u])); }
            }
            amax = block_max(amax, red);
            const float scale = amax / 127.0f;
#pragma unroll
            for (int u = 0; u < kRowUnroll; ++u) {
                const int c = threadIdx.x + u * kThreads;
                if (c < nch) {
                    const uint2 q = quant8<T>(v[u], scale);
                    for (int k = 0; k < ndst; ++k)
                        if (rows[k] >= 0) reinterpret_cast<uint2 *>(dst_base + (size_t)rows[k] * h)[c] = q;
                }
            }
            return scale;
        }
        for (int c = threadIdx.x; c < nch; c += kThreads) amax = fmaxf(amax, amax8<T>(s4[c]));
        amax = block_max(amax, red);
        const float scale = amax / 127.0f;
        for (int c = threadIdx.x; c < nch; c += kThreads) {
            const uint2 q = quant8<T>(s4[c], scale);
            for (int k = 0; k < ndst; ++k)
                if (rows[k] >= 0) reinterpret_cast<uint2 *>(dst_base + (size_t)rows[k] * h)[c] = q;
        }
        return scale;
    }
    for (int j = threadIdx.x; j < h; j += kThreads) amax = fmaxf(amax, fabsf(T::load(src[j])));
    amax = block_max(amax, red);
    const float scale = amax / 127.0f;
    for (int j = threadIdx.x; j < h; j += kThreads) {
        const int8_t q = quant1(T::load(src[j]), scale);
        for (int k = 0; k < ndst; ++k)
            if (rows[k] >= 0) dst_base[(size_t)rows[k] * h + j] = q;
    }
    return scale;
}

struct DispatchArgs {
    const char *x;
    const int32_t *ids;
    const int32_t *esc_in;
    char *expand_x;
    float *dyn;
    int32_t *assist;
    int32_t *esc_out;
    const int32_t *lr;
    const int32_t *boff;
    const int2 *plan;
    const int32_t *nplan;
    int W, bs, epr, h, K, nbs, R;
    long long rowbytes;      // bytes of one x row
};

// Token-major scatter, no quantisation.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void scatter_copy_kernel(DispatchArgs a)
{
    __shared__ int32_t rows[kMaxExperts];
    const int t = blockIdx.x, s = t / a.bs, tok = t % a.bs;
    token_rows(t, s, tok, a.ids, a.lr, a.boff, a.W * a.epr, a.K, a.nbs, a.R, rows, a.assist, a.esc_in, a.esc_out);
    __syncthreads();
    copy_row<VEC>(a.x + (size_t)t * a.rowbytes, a.expand_x, rows, a.K, (size_t)a.rowbytes);
}

// Token-major scatter with per-token dynamic int8 quantisation.
template <class T, bool VEC>
__global__ __launch_bounds__(kThreads) void scatter_quant_kernel(DispatchArgs a)
{
    __shared__ int32_t rows[kMaxExperts];
    __shared__ float red[kThreads / 64];
    const int t = blockIdx.x, s = t / a.bs, tok = t % a.bs;
    token_rows(t, s, tok, a.ids, a.lr, a.boff, a.W * a.epr, a.K, a.nbs, a.R, rows, a.assist, a.esc_in, a.esc_out);
    __syncthreads();
    const float scale = quant_row<T, VEC>(reinterpret_cast<const uint16_t *>(a.x) + (size_t)t * a.h,
                                          reinterpret_cast<int8_t *>(a.expand_x), rows, a.K, a.h, red);
    for (int k = threadIdx.x; k < a.K; k += kThreads)
        if (rows[k] >= 0) a.dyn[rows[k]] = scale;
}

// Segment schedule, pass 1: assist_info / expand_scales for every pair.
__global__ __launch_bounds__(kThreads) void segment_meta_kernel(DispatchArgs a)
{
    const size_t p = (size_t)blockIdx.x * kThreads + threadIdx.x;
    const size_t npairs = (size_t)a.W * a.bs * a.K;
    if (p >= npairs) return;
    const int E = a.W * a.epr;
    const int t = (int)(p / a.K), k = (int)(p % a.K), s = t / a.bs, tok = t % a.bs;
    const size_t b = (size_t)s * a.nbs + tok / kRouteTokens;
    const int e = a.ids[p], l = a.lr[p];
    if ((unsigned)e >= (unsigned)E || l < 0) return;
    const int row = a.boff[b * E + e] + l;
    if ((unsigned)row >= (unsigned)a.R) return;
    a.assist[(size_t)row * 3 + 0] = s;
    a.assist[(size_t)row * 3 + 1] = tok;
    a.assist[(size_t)row * 3 + 2] = k;
    if (a.esc_out) a.esc_out[row] = a.esc_in[p];
}

// Segment schedule, pass 2: blocks take plan items (row ranges of expand_x,
// a large segment's rows never sharing an item with another segment) and fill
// each row from its source token, found through assist_info.
template <int MODE, bool VEC>   // MODE 0: copy, 1: quant fp16, 2: quant bf16
__global__ __launch_bounds__(kThreads) void segment_payload_kernel(DispatchArgs a)
{
    __shared__ int32_t one[1];
    __shared__ float red[kThreads / 64];
    const int n = *a.nplan;
    for (int item = blockIdx.x; item < n; item += gridDim.x) {
        const int2 it = a.plan[item];
        const int lo = max(it.x, 0), hi = min(it.y, a.R);
        for (int row = lo; row < hi; ++row) {
            const int s = a.assist[(size_t)row * 3 + 0], tok = a.assist[(size_t)row * 3 + 1];
            if ((unsigned)s >= (unsigned)a.W || (unsigned)tok >= (unsigned)a.bs) continue;
            const size_t t = (size_t)s * a.bs + tok;
            if (threadIdx.x == 0) one[0] = row;
            __syncthreads();
            if (MODE == 0) {
                copy_row<VEC>(a.x + t * a.rowbytes, a.expand_x, one, 1, (size_t)a.rowbytes);
            } else {
                const uint16_t *src = reinterpret_cast<const uint16_t *>(a.x) + t * a.h;
                int8_t *dst = reinterpret_cast<int8_t *>(a.expand_x);
                const float scale = MODE == 1 ? quant_row<F16, VEC>(src, dst, one, 1, a.h, red)
                                              : quant_row<BF16, VEC>(src, dst, one, 1, a.h, red);
                if (threadIdx.x == 0) a.dyn[row] = scale;
            }
            __syncthreads();
        }
    }
}

// --------------------------------------------------------------------------
// combine
// --------------------------------------------------------------------------

struct CombineArgs {
    const char *expand_x;
    const int32_t *assist;
    const int32_t *erc;
    const int32_t *ids;
    const void *scales;
    char *x_out;
    int W, bs, epr, h, K, R;
    long long rowbytes;
};

// Row of pair (t, k): inside segment (el*W + s) of rank r = ids[t,k] / epr the
// rows are in ascending src_token order, so the row is the segment entry whose
// src_token equals tok; each wave tests 64 entries per step with a ballot.
__device__ __forceinline__ void combine_rows(const CombineArgs &a, int t, int s, int tok, const int32_t *rbase,
                                             int32_t *rows, uint32_t *sc)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int E = a.W * a.epr, S = a.epr * a.W;
    for (int k = wid; k < a.K; k += nw) {
        const size_t p = (size_t)t * a.K + k;
        const int e = a.ids[p];
        int row = -1;
        if ((unsigned)e < (unsigned)E) {
            const int r = e / a.epr, el = e % a.epr, i = el * a.W + s;
            int lo = rbase[r] + (i ? a.erc[(size_t)r * S + i - 1] : 0);
            int hi = rbase[r] + a.erc[(size_t)r * S + i];
            lo = max(lo, 0);
            hi = min(hi, a.R);
            for (int base = lo; base < hi; base += 64) {
                const int idx = base + lane;
                const int v = idx < hi ? a.assist[(size_t)idx * 3 + 1] : -1;
                const unsigned long long m = __ballot(v == tok);
                if (m) { row = base + __ffsll((long long)m) - 1; break; }
            }
        }
        if (lane == 0) {
            rows[k] = row;
            sc[k] = reinterpret_cast<const uint32_t *>(a.scales)[p];
        }
    }
}

template <class T, bool VEC>
__global__ __launch_bounds__(kThreads) void combine_half_kernel(CombineArgs a)
{
    __shared__ int32_t rbase[kMaxWorld + 1];
    __shared__ int32_t rows[kMaxExperts];
    __shared__ uint32_t sc[kMaxExperts];
    __shared__ int tmp[40];
    const int t = blockIdx.x, s = t / a.bs, tok = t % a.bs;
    rank_bases(a.erc, a.W, a.epr * a.W, rbase, tmp);
    __syncthreads();
    combine_rows(a, t, s, tok, rbase, rows, sc);
    __syncthreads();

    const int K = a.K;
    if (VEC) {
        const int nch = a.h / 8;
        constexpr int U = 2, KB = 8;
        for (int c0 = threadIdx.x; c0 < nch; c0 += kThreads * U) {
            float acc[U][8];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[u][i] = 0.0f;
            for (int kb = 0; kb < K; kb += KB) {
                uint4 v[KB][U];
#pragma unroll
                for (int kk = 0; kk < KB; ++kk) {
                    const int k = kb + kk;
                    const int row = k < K ? rows[k] : -1;
                    const uint4 *src = reinterpret_cast<const uint4 *>(a.expand_x + (size_t)(row < 0 ? 0 : row) * a.rowbytes);
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int c = c0 + u * kThreads;
                        v[kk][u] = (row >= 0 && c < nch) ? src[c] : make_uint4(0u, 0u, 0u, 0u);
                    }
                }
#pragma unroll
                for (int kk = 0; kk < KB; ++kk) {
                    if (kb + kk < K && rows[kb + kk] >= 0) {
                        const float w = __uint_as_float(sc[kb + kk]);
#pragma unroll
                        for (int u = 0; u < U; ++u) {
                            const uint32_t q[4] = {v[kk][u].x, v[kk][u].y, v[kk][u].z, v[kk][u].w};
#pragma unroll
                            for (int i = 0; i < 8; ++i)
                                acc[u][i] = __builtin_fmaf(T::load((uint16_t)(q[i >> 1] >> ((i & 1) * 16))), w, acc[u][i]);
                        }
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * kThreads;
                if (c < nch) {
                    uint32_t o[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        o[i] = (uint32_t)T::store(acc[u][2 * i]) | ((uint32_t)T::store(acc[u][2 * i + 1]) << 16);
                    reinterpret_cast<uint4 *>(a.x_out + (size_t)t * a.rowbytes)[c] = make_uint4(o[0], o[1], o[2], o[3]);
                }
            }
        }
    } else {
        for (int j = threadIdx.x; j < a.h; j += kThreads) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                const int row = rows[k];
                if (row < 0) continue;
                const uint16_t y = reinterpret_cast<const uint16_t *>(a.expand_x)[(size_t)row * a.h + j];
                acc = __builtin_fmaf(T::load(y), __uint_as_float(sc[k]), acc);
            }
            reinterpret_cast<uint16_t *>(a.x_out)[(size_t)t * a.h + j] = T::store(acc);
        }
    }
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void combine_i32_kernel(CombineArgs a)
{
    __shared__ int32_t rbase[kMaxWorld + 1];
    __shared__ int32_t rows[kMaxExperts];
    __shared__ uint32_t sc[kMaxExperts];
    __shared__ int tmp[40];
    const int t = blockIdx.x, s = t / a.bs, tok = t % a.bs;
    rank_bases(a.erc, a.W, a.epr * a.W, rbase, tmp);
    __syncthreads();
    combine_rows(a, t, s, tok, rbase, rows, sc);
    __syncthreads();

    const int K = a.K;
    if (VEC) {
        const int nch = a.h / 4;
        for (int c = threadIdx.x; c < nch; c += kThreads) {
            uint32_t acc[4] = {0u, 0u, 0u, 0u};
            for (int k = 0; k < K; ++k) {
                const int row = rows[k];
                if (row < 0) continue;
                const uint4 v = reinterpret_cast<const uint4 *>(a.expand_x + (size_t)row * a.rowbytes)[c];
                acc[0] += v.x * sc[k];
                acc[1] += v.y * sc[k];
                acc[2] += v.z * sc[k];
                acc[3] += v.w * sc[k];
            }
            reinterpret_cast<uint4 *>(a.x_out + (size_t)t * a.rowbytes)[c] = make_uint4(acc[0], acc[1], acc[2], acc[3]);
        }
    } else {
        for (int j = threadIdx.x; j < a.h; j += kThreads) {
            uint32_t acc = 0u;
            for (int k = 0; k < K; ++k) {
                const int row = rows[k];
                if (row < 0) continue;
                acc += reinterpret_cast<const uint32_t *>(a.expand_x)[(size_t)row * a.h + j] * sc[k];
            }
            reinterpret_cast<uint32_t *>(a.x_out)[(size_t)t * a.h + j] = acc;
        }
    }
}

// --------------------------------------------------------------------------
// host side
// --------------------------------------------------------------------------

size_t elem_size(int dtype) { return dtype == MOE_INT32 ? 4 : 2; }

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int check_scalars(int W, int bs, int epr, int h, int K, int dtype)
{
    if (dtype != MOE_INT32 && dtype != MOE_FP16 && dtype != MOE_BF16) return MOE_ERR_DTYPE;
    if (W < kMinWorld || W > kMaxWorld || epr < 1 || bs < 0 || h < 1 || K < 1) return MOE_ERR_SHAPE;
    const long long E = (long long)W * epr;
    if (E > kMaxExperts || K > E) return MOE_ERR_SHAPE;
    const long long N = (long long)W * bs;
    if (N * K >= (1ll << 31) || N > kMaxTokens) return MOE_ERR_SHAPE;
    return MOE_OK;
}

struct DispatchLayout {
    int nbs, NB;
    size_t cnt, boff, lr, plan, nplan, total;
};

DispatchLayout dispatch_layout(int W, int bs, int epr, int K)
{
    DispatchLayout L;
    const size_t E = (size_t)W * epr, N = (size_t)W * bs, S = (size_t)epr * W;
    L.nbs = (bs + kRouteTokens - 1) / kRouteTokens;
    L.NB = W * L.nbs;
    const size_t plan_cap = N * K / kPlanRows + 2 * (size_t)W * S + W + 1;
    size_t off = 0;
    L.cnt = off;   off = round_up(off + (size_t)L.NB * E * 4, 256);
    L.boff = off;  off = round_up(off + (size_t)L.NB * E * 4, 256);
    L.lr = off;    off = round_up(off + N * K * 4, 256);
    L.plan = off;  off = round_up(off + plan_cap * 8, 256);
    L.nplan = off; off = round_up(off + 4, 256);
    L.total = off;
    return L;
}

}  // namespace

extern "C" {

const char *moe_status_str(int status)
{
    switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULLPTR: return "a required pointer is NULL, or a forbidden one is not";
    case MOE_ERR_SHAPE: return "a size is out of range or a size product overflows";
    case MOE_ERR_DTYPE: return "unknown token dtype";
    case MOE_ERR_QUANT: return "unknown quant mode, or quantisation of int32 data";
    case MOE_ERR_WORKSPACE: return "workspace smaller than the queried size";
    case MOE_ERR_LAUNCH: return "the HIP runtime refused a kernel launch";
    case MOE_ERR_SCHEDULE: return "unknown schedule mode, or segment schedule too large for this shape";
    case MOE_ERR_ALIGN: return "a pointer is not aligned to its element size";
    default: return "unknown status";
    }
}

int moe_dispatch_workspace_size(int ep_world, int bs, int experts_per_rank, int h, int topk, int dtype,
                                int quant_mode, size_t *bytes)
{
    if (!bytes) return MOE_ERR_NULLPTR;
    int rc = check_scalars(ep_world, bs, experts_per_rank, h, topk, dtype);
    if (rc) return rc;
    if (quant_mode != MOE_QUANT_NONE && quant_mode != MOE_QUANT_DYN_TOKEN) return MOE_ERR_QUANT;
    if (quant_mode == MOE_QUANT_DYN_TOKEN && dtype == MOE_INT32) return MOE_ERR_QUANT;
    *bytes = dispatch_layout(ep_world, bs, experts_per_rank, topk).total;
    return MOE_OK;
}

int moe_dispatch(const void *x, const int32_t *expert_ids, const void *expert_scales, int ep_world, int bs,
                 int experts_per_rank, int h, int topk, int dtype, int quant_mode, void *expand_x,
                 float *dynamic_scales, int32_t *assist_info, int32_t *ep_recv_count, void *expand_scales,
                 const moe_schedule *schedule, void *workspace, size_t workspace_bytes, void *stream)
{
    size_t need = 0;
    int rc = moe_dispatch_workspace_size(ep_world, bs, experts_per_rank, h, topk, dtype, quant_mode, &need);
    if (rc) return rc;
    const int W = ep_world, epr = experts_per_rank, K = topk;
    const long long N = (long long)W * bs;
    const bool quant = quant_mode == MOE_QUANT_DYN_TOKEN;
    if (!ep_recv_count || !workspace) return MOE_ERR_NULLPTR;
    if (N > 0 && (!x || !expert_ids || !expand_x || !assist_info)) return MOE_ERR_NULLPTR;
    if (quant != (dynamic_scales != nullptr) && N > 0) return MOE_ERR_NULLPTR;
    if (!quant && dynamic_scales) return MOE_ERR_NULLPTR;
    if (expand_scales && !expert_scales) return MOE_ERR_NULLPTR;
    if (workspace_bytes < need) return MOE_ERR_WORKSPACE;

    const int mode = schedule ? schedule->mode : MOE_SCHED_TOKEN;
    long long large = schedule ? schedule->large_segment_bytes : -1;
    if (large < 0) large = kReadmeLargeBytes;
    int32_t *seg_flags = schedule ? schedule->segment_is_large : nullptr;
    if (mode != MOE_SCHED_TOKEN && mode != MOE_SCHED_SEGMENT) return MOE_ERR_SCHEDULE;
    const long long S = (long long)epr * W;
    const bool want_seg = mode == MOE_SCHED_SEGMENT || seg_flags;
    if (want_seg && (long long)W * S > kSegLdsMax) return MOE_ERR_SCHEDULE;

    const size_t xs = elem_size(dtype);
    const size_t rowbytes = (size_t)h * xs;
    if (!aligned(x, xs) || !aligned(expert_ids, 4) || !aligned(expert_scales, 4) ||
        !aligned(expand_x, quant ? 1 : xs) || !aligned(dynamic_scales, 4) || !aligned(assist_info, 4) ||
        !aligned(ep_recv_count, 4) || !aligned(expand_scales, 4) || !aligned(workspace, 16) ||
        !aligned(seg_flags, 4))
        return MOE_ERR_ALIGN;

    const DispatchLayout L = dispatch_layout(W, bs, epr, K);
    char *ws = static_cast<char *>(workspace);
    int32_t *cnt = reinterpret_cast<int32_t *>(ws + L.cnt);
    int32_t *boff = reinterpret_cast<int32_t *>(ws + L.boff);
    int32_t *lr = reinterpret_cast<int32_t *>(ws + L.lr);
    int2 *plan = reinterpret_cast<int2 *>(ws + L.plan);
    int32_t *nplan = reinterpret_cast<int32_t *>(ws + L.nplan);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int E = W * epr;

    (void)hipGetLastError();
    if (N > 0)
        hipLaunchKernelGGL(route_kernel, dim3(L.NB), dim3(kThreads), (size_t)E * kRouteWords * 8, st,
                           expert_ids, W, bs, epr, K, L.nbs, cnt, lr);
    const int elem_out = quant ? 1 : (int)xs;
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), want_seg ? (size_t)W * S * 5 : 0, st,
                       cnt, W, epr, L.nbs, h, elem_out, boff, ep_recv_count, want_seg ? 1 : 0, large,
                       seg_flags, (mode == MOE_SCHED_SEGMENT && N > 0) ? plan : nullptr, nplan);
    if (N > 0) {
        DispatchArgs a;
        a.x = static_cast<const char *>(x);
        a.ids = expert_ids;
        a.esc_in = static_cast<const int32_t *>(expert_scales);
        a.expand_x = static_cast<char *>(expand_x);
        a.dyn = dynamic_scales;
        a.assist = assist_info;
        a.esc_out = static_cast<int32_t *>(expand_scales);
        a.lr = lr;
        a.boff = boff;
        a.plan = plan;
        a.nplan = nplan;
        a.W = W; a.bs = bs; a.epr = epr; a.h = h; a.K = K; a.nbs = L.nbs; a.R = (int)(N * K);
        a.rowbytes = (long long)rowbytes;
        const bool vec = quant ? (h % 8 == 0 && aligned(x, 16) && aligned(expand_x, 8))
                               : (rowbytes % 16 == 0 && aligned(x, 16) && aligned(expand_x, 16));
        if (mode == MOE_SCHED_TOKEN) {
            const dim3 g((unsigned)N), b(kThreads);
            if (!quant) {
                if (vec) hipLaunchKernelGGL(scatter_copy_kernel<true>, g, b, 0, st, a);
                else hipLaunchKernelGGL(scatter_copy_kernel<false>, g, b, 0, st, a);
            } else if (dtype == MOE_FP16) {
                if (vec) hipLaunchKernelGGL((scatter_quant_kernel<F16, true>), g, b, 0, st, a);
                else hipLaunchKernelGGL((scatter_quant_kernel<F16, false>), g, b, 0, st, a);
            } else {
                if (vec) hipLaunchKernelGGL((scatter_quant_kernel<BF16, true>), g, b, 0, st, a);
                else hipLaunchKernelGGL((scatter_quant_kernel<BF16, false>), g, b, 0, st, a);
            }
        } else {
            const long long npairs = N * K;
            hipLaunchKernelGGL(segment_meta_kernel, dim3((unsigned)((npairs + kThreads - 1) / kThreads)),
                               dim3(kThreads), 0, st, a);
            const dim3 g(kSegGrid), b(kThreads);
            const int qm = !quant ? 0 : (dtype == MOE_FP16 ? 1 : 2);
            if (qm == 0) {
                if (vec) hipLaunchKernelGGL((segment_payload_kernel<0, true>), g, b, 0, st, a);
                else hipLaunchKernelGGL((segment_payload_kernel<0, false>), g, b, 0, st, a);
            } else if (qm == 1) {
                if (vec) hipLaunchKernelGGL((segment_payload_kernel<1, true>), g, b, 0, st, a);
                else hipLaunchKernelGGL((segment_payload_kernel<1, false>), g, b, 0, st, a);
            } else {
                if (vec) hipLaunchKernelGGL((segment_payload_kernel<2, true>), g, b, 0, st, a);
                else hipLaunchKernelGGL((segment_payload_kernel<2, false>), g, b, 0, st, a);
            }
        }
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

int moe_combine_workspace_size(int ep_world, int bs, int experts_per_rank, int h, int topk, int dtype,
                               size_t *bytes)
{
    if (!bytes) return MOE_ERR_NULLPTR;
    int rc = check_scalars(ep_world, bs, experts_per_rank, h, topk, dtype);
    if (rc) return rc;
    *bytes = 0;
    return MOE_OK;
}

int moe_combine(const void *expand_x, const int32_t *assist_info, const int32_t *ep_recv_count,
                const int32_t *expert_ids, const void *expert_scales, int ep_world, int bs, int experts_per_rank,
                int h, int topk, int dtype, void *x_out, void *workspace, size_t workspace_bytes, void *stream)
{
    size_t need = 0;
    int rc = moe_combine_workspace_size(ep_world, bs, experts_per_rank, h, topk, dtype, &need);
    if (rc) return rc;
    const int W = ep_world, K = topk;
    const long long N = (long long)W * bs;
    if (!ep_recv_count) return MOE_ERR_NULLPTR;
    if (N > 0 && (!expand_x || !assist_info || !expert_ids || !expert_scales || !x_out)) return MOE_ERR_NULLPTR;
    if (workspace_bytes < need) return MOE_ERR_WORKSPACE;
    (void)workspace;
    const size_t xs = elem_size(dtype);
    if (!aligned(expand_x, xs) || !aligned(assist_info, 4) || !aligned(ep_recv_count, 4) ||
        !aligned(expert_ids, 4) || !aligned(expert_scales, 4) || !aligned(x_out, xs))
        return MOE_ERR_ALIGN;
    if (N == 0) return MOE_OK;

    CombineArgs a;
    a.expand_x = static_cast<const char *>(expand_x);
    a.assist = assist_info;
    a.erc = ep_recv_count;
    a.ids = expert_ids;
    a.scales = expert_scales;
    a.x_out = static_cast<char *>(x_out);
    a.W = W; a.bs = bs; a.epr = experts_per_rank; a.h = h; a.K = K; a.R = (int)(N * K);
    a.rowbytes = (long long)((size_t)h * xs);
    const bool vec = (size_t)a.rowbytes % 16 == 0 && aligned(expand_x, 16) && aligned(x_out, 16);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 g((unsigned)N), b(kThreads);
    (void)hipGetLastError();
    if (dtype == MOE_INT32) {
        if (vec) hipLaunchKernelGGL(combine_i32_kernel<true>, g, b, 0, st, a);
        else hipLaunchKernelGGL(combine_i32_kernel<false>, g, b, 0, st, a);
    } else if (dtype == MOE_FP16) {
        if (vec) hipLaunchKernelGGL((combine_half_kernel<F16, true>), g, b, 0, st, a);
        else hipLaunchKernelGGL((combine_half_kernel<F16, false>), g, b, 0, st, a);
    } else {
        if (vec) hipLaunchKernelGGL((combine_half_kernel<BF16, true>), g, b, 0, st, a);
        else hipLaunchKernelGGL((combine_half_kernel<BF16, false>), g, b, 0, st, a);
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // extern "C"
