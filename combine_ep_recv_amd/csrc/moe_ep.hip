// moe_ep.hip -- MoE token dispatch and combine for MI355X (gfx950, wave64).
//
// The C ABI declared in include/moe_ep.h. Pure data movement plus an axpy:
// no MFMA anywhere; every kernel is bounded by HBM bandwidth or by latency.
//
// Dispatch (aclnnMoeDistributeDispatchV4, 计算公式: expandXOut = AllToAllV(X),
// with every logical rank's receive window a partition of one HBM):
//   route    one block per (source rank, 256-token chunk) b. Builds, in LDS, a
//            bitmap per expert over the chunk's tokens (ds_or_b64), then
//            writes, per expert e, the exclusive and inclusive prefix of the
//            chunk's counts over experts (pc[b][e], pci[b][e]) and, for every
//            (t, k), the number of earlier tokens of the chunk routed to the
//            same expert (a popcount below the token's bit). Bit-set order is
//            irrelevant, so the result is deterministic without a sort.
//            Inactive pairs (token masks, xActiveMaskOptional) and pairs of
//            special experts (ids past the E real ones) are routed nowhere.
//   scatter  token-major: the first row of pair (t, k) routed to e from
//            chunk b is  sum_{b' < b} pci[b'][e] + sum_{b' >= b} pc[b'][e]
//            (all rows of lower experts, plus this expert's rows from earlier
//            chunks), so each block sums those few L2-resident words for its K
//            pairs instead of waiting for a grid-wide scan. Rows are moved with
//            128-bit loads/stores; quantisation (quantMode 1: static int8 with
//            one coefficient or one per column; quantMode 2: per-token int8;
//            quantMode 3: per-128-group FP8 E4M3) runs one wavefront per token
//            (max by DPP shuffles, no block barrier). Static int8 with one
//            coefficient per expert and column instead writes the metadata
//            first, then walks the rows expert-major in groups of source ranks.
//            ep_recv_count (combine_doubleplane README 功能说明) is formed the
//            same way by the first threads of the grid.
//   scan     single block; only for more than 64 chunks, and for the segment
//            schedule (the README's 方案设计 large-segment predicate + plan).
// Combine (README 功能说明, check formula; 实现逻辑 return path + weighted sum):
//   slots    every expand_x row announces itself in its source's window: the
//            row index goes to slot (src_token, topk_id) of rank src_rank;
//            pairs without a row get -1 (inactive, zero expert) or -2 (copy
//            expert: the token itself).
//   gather   one block per (token, 2 KiB slice) reads the K rows named by its
//            slots with 128-bit loads and accumulates in fp32, one FMA per k
//            with k ascending, rounding once to the output type.

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <limits.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "moe_ep.h"

namespace {

constexpr int kScanThreads = 1024;         // the single scan block (>= max experts)
constexpr int kScanBatch = 32;             // chunks whose counts the scan loads at once
constexpr int kRouteThreads = 256;
constexpr int kRouteTokens = 256;          // tokens per route chunk
constexpr int kRouteWords = kRouteTokens / 64;
constexpr int kMaxExperts = 1024;          // moeExpertNum upper bound
constexpr int kMinWorld = 2, kMaxWorld = 768;   // epWorldSize range
constexpr int kDirectMaxChunks = 64;       // chunk count up to which blocks sum the prefixes themselves
constexpr int kChunkBatch = 16;            // chunk counts such a sum loads at once
constexpr int kSegLdsMax = 11264;          // W*S limit for the LDS-resident segment counts
constexpr long long kMaxTokens = (1ll << 24) - 1;   // N blocks of 256 threads stay below 2^32 items
constexpr int kPlanRows = 8;               // rows per segment-schedule work item
static_assert(kPlanRows <= 64, "a plan item's rows are held one per lane");
constexpr int kSegGrid = 4096;             // blocks of the segment-major payload pass
constexpr size_t kDeviceStoreBytes = 64ull << 20;   // gather: the tail of x_out stored device-scope
constexpr int kAdaptiveSegGrid = 1024;     // most blocks of the adaptive schedule's large-segment pass
constexpr int64_t kReadmeLargeBytes = 2 * 1024 * 1024;

constexpr int kCopyThreads = 128;          // token-major copy: block = (token, slice)
constexpr int kCopyUnroll = 2;             // 16-byte chunks per thread per slice
constexpr int kCopyWaveMinTokens = 1024;   // from here on the copy runs one wavefront per token ...
constexpr long long kCopyWaveMaxBytes = 640ll << 20;    // ... up to this much expand_x
constexpr long long kMixedStoreMaxBytes = 320ll << 20;  // rows written up to which half the stores are plain
constexpr long long kQuarterPlainMaxBytes = 512ll << 20; // ... a quarter of them; none beyond
constexpr int kQuantThreads = 256;         // one wavefront per token
constexpr int kQuantMaxK = 64;             // wavefront-per-token quantiser handles topk <= 64 ...
constexpr int kQuantMaxH = 16384;          // ... and h <= 16384 (16 pieces of 16 elements per lane)
constexpr int kBlockThreads = 256;         // generic block-per-token kernels
constexpr int kGatherThreads = 128;        // combine: block = (token, 128-chunk slice)
constexpr int kSlotThreads = 256;
constexpr int kCopySlot = -2;             // slot of a copy-expert pair: the token itself
constexpr int kConstSlot0 = -3;           // slot of a pair of const expert j: kConstSlot0 - j
// shapes of the static quantisation coefficients: 1, h or E*h values
constexpr int kStaticOne = 0, kStaticColumn = 1, kStaticExpert = 2;
constexpr int kXcds = 8;                   // gfx950 XCDs; consecutive workgroups go to consecutive XCDs
constexpr long long kStaticGroupBytes = 2ll << 20;   // token slices per XCD in one source group (L2 is 4 MB)

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

// Streaming (non-temporal) 16-byte accesses for data that is touched once. They
// pay where reads dominate (the combine's gather; its x_out stores are
// device-scope, see store_device) and in the (token, slice) copy. The write-dominated wavefront scatters (the
// quantisers, the wavefront copy) split their stores: a checkerboard over
// (1 KiB chunk, copy) goes non-temporal, the rest plain. At
// 16 ranks x 256 tokens, h = 7168 (294 MB moved) that kernel takes 45 us,
// against 51 us with plain stores only and 55 us with non-temporal ones only;
// a pure 235 MB scattered-row write reaches ~6.3 TB/s plain and ~4.8 TB/s
// non-temporal. The mix is no slower on small outputs either. As the rows
// written outgrow the Infinity Cache (256 MB) the plain share must shrink
// (store_mix). The int8 dispatch at 16 ranks, h = 7168 takes:
// - 384 tokens per rank (352 MB of rows): 76 us with a quarter of the stores
//   plain, 82 us with half, 84 us with none;
// - 512 tokens (470 MB): 102 / 125 / 112 us;
// - 576 tokens (528 MB): 117 / 142 / 118 us;
// - 640 tokens (587 MB): 134 us with a quarter, 130 us with none;
// - 1024 tokens: 252 us with a quarter, 198 us with none.
// So the quantisers keep half of their stores plain up to 320 MiB of rows, a
// quarter up to 512 MiB, and none beyond. The wavefront copy (bf16 rows twice
// as long) is best with half plain up to its 640 MiB limit: at 256 and 320
// tokens per rank (470 and 587 MB) it takes 85 and 116 us that way, against
// 91 and 139 us with a quarter or none.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_stream(uint4 *p, uint4 v)
{
    u32x4_t t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x4_t *>(p));
}
// Device-scope 16-byte store (sc1): the line is written through the XCD's L2
// rather than left dirty there for the launch's closing writeback. The
// combine's x_out is written once and read by no later wave of the launch, so
// that writeback is pure wait at the end of the kernel: at 16 ranks x 256
// tokens, h = 7168 (58.7 MB of x_out) the cold dispatch + combine step takes
// ~142.4 us with it against ~146 us with non-temporal stores, back to back
// unchanged. The lines stay in the Infinity Cache, though, and a larger
// output written this way evicts what the next launch would find there (at
// 512 tokens per rank: back to back 335 against 289 us, and 302 against 298
// us timed), so only the last 64 MiB of x_out (all of it up to that size) is
// stored device-scope, the rest non-temporally: 298 and 309 us there. The dispatch's scatter is not helped: sc1 on its non-temporal
// half takes the back-to-back step from 141 to 165 us, on its plain half it
// changes nothing. There is no clang builtin for the scope bits, hence the
// asm; the s_nop covers the wait states a VALU write to the store's data
// registers needs after a 128-bit store, which the compiler does not see
// across an asm statement. The store is a kernel's last memory access (no
// later load's vmcnt wait miscounts it).
__device__ __forceinline__ void store_device(uint4 *p, uint4 v)
{
    const u32x4_t t = {v.x, v.y, v.z, v.w};
    asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" ::"v"(p), "v"(t) : "memory");
}
__device__ __forceinline__ uint4 load_stream(const uint4 *p)
{
    u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

// n / d for 0 <= n < 2^23 and d >= 1, with rcp = 1.0f / d: the float quotient is
// within (n / d) * 2^-23 < 1 of the true one, so one integer correction in
// either direction makes it exact. Integer division by a runtime divisor costs
// tens of instructions; this costs six.
__device__ __forceinline__ int div_small(int n, int d, float rcp)
{
    int q = (int)((float)n * rcp);
    const int r = n - q * d;
    q += (r >= d) - (r < 0);
    return q;
}

// --------------------------------------------------------------------------
// wave / block helpers
// --------------------------------------------------------------------------

// Inclusive prefix sum over the 64 lanes of a wavefront: a Hillis-Steele scan
// inside each 16-lane row by DPP row shifts (a lane whose source lies outside
// its row adds 0), then the totals of the lower rows, read with readlane.
__device__ __forceinline__ int wave_incl_scan(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
    const int lane = threadIdx.x & 63;
    const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
              r2 = __builtin_amdgcn_readlane(v, 47);
    return v + (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
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

// Inclusive scan of one int per thread over the block, through buf
// (blockDim.x ints of LDS): the max over this and lower threads, or (REV) the
// min over this and higher threads. Shuffles inside each wavefront, then the
// wavefront totals; buf holds every thread's result on return. Every thread
// of the block calls it.
template <bool REV>
__device__ int block_incl_minmax(int v, int *buf)
{
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6, nw = blockDim.x >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = REV ? __shfl_down(v, d, 64) : __shfl_up(v, d, 64);
        if (REV ? lane + d < 64 : lane >= d) v = REV ? min(v, y) : max(v, y);
    }
    if (lane == (REV ? 0 : 63)) buf[wid] = v;        // the wavefront's total
    __syncthreads();
    for (int w = 0; w < nw; ++w)
        if (REV ? w > wid : w < wid) v = REV ? min(v, buf[w]) : max(v, buf[w]);
    __syncthreads();
    buf[t] = v;
    __syncthreads();
    return v;
}

__device__ __forceinline__ int wave_sum_i(int v)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
    return v;
}

__device__ __forceinline__ float block_max(float v, float *tmp)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    v = wave_max(v);
    if (lane == 0) tmp[wid] = v;
    __syncthreads();
    float m = tmp[0];
    for (int i = 1; i < nw; ++i) m = fmaxf(m, tmp[i]);
    __syncthreads();
    return m;
}

// --------------------------------------------------------------------------
// route
// --------------------------------------------------------------------------

// Rank of bit `bit` among the set bits of a kRouteWords-word bitmap: the set
// bits of the lower words plus those below it in its own word. All words are
// read (one LDS round trip) and masked, so there is no loop.
__device__ __forceinline__ int bitmap_rank(const unsigned long long *row, int bit)
{
    const int wi = bit >> 6;
    int r = 0;
#pragma unroll
    for (int w = 0; w < kRouteWords; ++w) {
        const unsigned long long m = w < wi ? ~0ull : (w == wi ? (1ull << (bit & 63)) - 1ull : 0ull);
        r += __popcll(row[w] & m);
    }
    return r;
}

// MK: the token-mask kind, a template parameter so that the unmasked kernel
// carries no mask code (it cost 0.6 us of latency at 16 chunks).
template <int MK>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(const int32_t *__restrict__ ids, int W, int bs,
                                                              int epr, int K, int nbs,
                                                              const uint8_t *__restrict__ mask,
                                                              int32_t *__restrict__ pc, int32_t *__restrict__ pci,
                                                              int32_t *__restrict__ lr)
{
    extern __shared__ unsigned long long bm[];   // [E][kRouteWords]
    __shared__ int tmp[40];
    constexpr int U = 8;
    const int E = W * epr;
    const int b = blockIdx.x, s = b / nbs, j = b % nbs;
    const int tok0 = j * kRouteTokens;
    const int ntok = min(kRouteTokens, bs - tok0);
    const int npairs = ntok * K;
    const size_t pair0 = ((size_t)s * bs + tok0) * K;
    const float rK = 1.0f / K;

    // one pass of U pairs per thread covers the chunk whenever ntok * K <= 2048;
    // the ids and token indices then stay in registers for the rank pass. The
    // first pass's ids are requested before the bitmaps are cleared.
    // An inactive pair (token masks) is routed nowhere: its id reads as -1, so
    // it sets no bit, is not counted and gets rank -1, and no kernel after this
    // one writes a row for it.
    // A pass loads U ids, then (with a mask) their U mask bytes, at clamped
    // indices (npairs >= 1), and only then tests them: a mask test between two
    // loads makes the compiler wait for each pair before issuing the next.
    const size_t tok_base = (size_t)s * bs + tok0;
    int e[U], tl[U], mk[U];
    auto load_pass = [&](int p0) {
#pragma unroll
        for (int u = 0; u < U; ++u) e[u] = ids[pair0 + min(p0 + u * kRouteThreads, npairs - 1)];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = min(p0 + u * kRouteThreads, npairs - 1);
            if constexpr (MK == MOE_MASK_TOKEN) mk[u] = mask[tok_base + div_small(p, K, rK)];
            if constexpr (MK == MOE_MASK_PAIR) mk[u] = mask[pair0 + p];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = p0 + u * kRouteThreads;
            tl[u] = div_small(p, K, rK);
            if (p >= npairs) e[u] = -1;
            if constexpr (MK != MOE_MASK_NONE) if (!mk[u]) e[u] = -1;
        }
    };
    const bool one_pass = npairs <= kRouteThreads * U;
    load_pass(threadIdx.x);
    for (int i = threadIdx.x; i < E * kRouteWords; i += blockDim.x) bm[i] = 0ull;
    __syncthreads();
    for (int p0 = threadIdx.x; p0 < npairs; p0 += kRouteThreads * U) {
        if (p0 != (int)threadIdx.x) load_pass(p0);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if ((unsigned)e[u] < (unsigned)E) atomicOr(&bm[e[u] * kRouteWords + (tl[u] >> 6)], 1ull << (tl[u] & 63));
    }
    __syncthreads();

    // per-expert counts of this chunk and their prefix over experts (E <= 4 * 256);
    // every thread reads its four experts' words at once (clamped, then masked)
    int c[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int x = threadIdx.x * 4 + q;
        const unsigned long long *row = &bm[min(x, E - 1) * kRouteWords];
        int n = 0;
#pragma unroll
        for (int w = 0; w < kRouteWords; ++w) n += __popcll(row[w]);
        c[q] = x < E ? n : 0;
        sum += c[q];
    }
    int total;
    int ex = block_excl_scan(sum, tmp, &total);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int x = threadIdx.x * 4 + q;
        if (x < E) {
            pc[(size_t)b * E + x] = ex;
            pci[(size_t)b * E + x] = ex + c[q];
        }
        ex += c[q];
    }

    for (int p0 = threadIdx.x; p0 < npairs; p0 += kRouteThreads * U) {
        if (!one_pass) load_pass(p0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = p0 + u * kRouteThreads;
            if (p >= npairs) continue;
            lr[pair0 + p] = (unsigned)e[u] < (unsigned)E ? bitmap_rank(&bm[e[u] * kRouteWords], tl[u]) : -1;
        }
    }
}

// --------------------------------------------------------------------------
// scan (many chunks, or the segment schedule)
// --------------------------------------------------------------------------

// The large-segment predicate (combine_doubleplane README, 方案设计): segment
// (el, s) of rank r with c rows is large iff it comes from another rank, is
// non-empty, its payload c*h*elem_bytes reaches T, and that payload exceeds
// the mean payload r receives per remote segment, num / den with num = (rows r
// receives from other ranks)*h*elem_bytes and den = max(W-1, 1)*epr. The last
// test is evaluated as c*den > remote rows: both sides of payload*den > num
// carry the factor h*elem_bytes > 0, and without it no product can leave 64
// bits.
__device__ __forceinline__ bool segment_large(bool from_other_rank, long long c, long long remote_rows,
                                              long long row_bytes, long long large_bytes, long long den)
{
    return from_other_rank && c > 0 && c * row_bytes >= large_bytes && c * den > remote_rows;
}

__global__ __launch_bounds__(kScanThreads) void scan_kernel(
    const int32_t *__restrict__ pc, const int32_t *__restrict__ pci, int W, int epr, int nbs, int h,
    int elem_bytes, int32_t *__restrict__ boff, int32_t *__restrict__ erc, int want_seg, long long large_bytes,
    int32_t *__restrict__ seg_flags, int2 *__restrict__ plan, int32_t *__restrict__ nplan)
{
    __shared__ int32_t eoff[kMaxExperts + 1];
    __shared__ int32_t part[kScanThreads];        // [q][e]: chunk-range partial counts, then their prefixes
    __shared__ int32_t tmp[40];
    extern __shared__ int32_t seg_lds[];          // when want_seg: int32 counts [W*S], then uint8 flags [W*S]
    const int E = W * epr, S = epr * W, NB = W * nbs;
    const int tid = threadIdx.x;
    // T threads per expert (kScanThreads / E, rounded down to a power of two);
    // thread (e, q) = tid % E, tid / E owns chunks [q * NB / T, (q + 1) * NB / T)
    int T = 1;
    while (2 * T * E <= kScanThreads) T *= 2;
    const int e = tid % E, q = tid / E;
    const bool act = q < T;
    const int bq0 = act ? (int)((long long)q * NB / T) : 0, bq1 = act ? (int)((long long)(q + 1) * NB / T) : 0;

    // partial column sums; kScanBatch chunks' counts are loaded together, and
    // the first batch stays in registers for the offsets below
    int mine = 0, c0[kScanBatch];
    for (int b0 = bq0; b0 < bq1; b0 += kScanBatch) {
        int c[kScanBatch];
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u) {
            const size_t b = (size_t)min(b0 + u, bq1 - 1);
            c[u] = b0 + u < bq1 ? pci[b * E + e] - pc[b * E + e] : 0;
        }
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u) mine += c[u];
        if (b0 == bq0) {
#pragma unroll
            for (int u = 0; u < kScanBatch; ++u) c0[u] = c[u];
        }
    }
    if (act) part[q * E + e] = mine;
    __syncthreads();
    // column totals -> exclusive offsets per expert (the q = 0 threads, tid = e)
    int tot = 0;
    if (tid < E) {
        for (int k = 0; k < T; ++k) {
            const int v = part[k * E + tid];
            part[k * E + tid] = tot;                  // now: offset of range k inside column e
            tot += v;
        }
    }
    int total;
    const int ex = block_excl_scan(tot, tmp, &total);
    if (tid < E) eoff[tid] = ex;
    if (tid == 0) eoff[E] = total;
    __syncthreads();

    // chunk offsets, and ep_recv_count at the last chunk of every source rank
    if (act) {
        const int r = e / epr, el = e % epr;
        const int base_r = eoff[r * epr];
        int run = part[q * E + e];
        for (int b0 = bq0; b0 < bq1; b0 += kScanBatch) {
            int c[kScanBatch];
#pragma unroll
            for (int u = 0; u < kScanBatch; ++u) {
                const size_t b = (size_t)min(b0 + u, bq1 - 1);
                c[u] = b0 == bq0 ? c0[u] : pci[b * E + e] - pc[b * E + e];
            }
#pragma unroll
            for (int u = 0; u < kScanBatch; ++u) {
                const int b = b0 + u;
                if (b >= bq1) continue;
                boff[(size_t)b * E + e] = eoff[e] + run;
                run += c[u];
                if ((b + 1) % nbs == 0)               // last chunk of source rank b / nbs
                    erc[(size_t)r * S + el * W + b / nbs] = eoff[e] + run - base_r;
            }
        }
        if (nbs == 0 && q == 0)                       // empty batch: zero counts
            for (int s = 0; s < W; ++s) erc[(size_t)r * S + el * W + s] = 0;
    }
    if (!want_seg) return;
    __syncthreads();
    // segment counts: differences of consecutive inclusive counts within a rank
    const int G = W * S;
    int32_t *segc = seg_lds;
    uint8_t *flag = reinterpret_cast<uint8_t *>(seg_lds + (size_t)G);
    for (int i = tid; i < G; i += blockDim.x) segc[i] = erc[i] - (i % S > 0 ? erc[i - 1] : 0);
    // rows each rank receives from the other ranks (part[] is free from here on)
    for (int r = tid; r < W; r += blockDim.x) part[r] = 0;
    __syncthreads();
    for (int i = tid; i < G; i += blockDim.x)
        if ((i % S) % W != i / S && segc[i]) atomicAdd(&part[i / S], segc[i]);
    __syncthreads();

    // large-segment predicate (combine_doubleplane README 方案设计), one segment
    // per thread: segment i of rank r comes from source rank i % W
    const long long den = (long long)(W - 1 > 1 ? W - 1 : 1) * epr;
    for (int g = tid; g < G; g += blockDim.x) {
        const int r = g / S, i = g % S;
        const int large = segment_large(i % W != r, segc[g], part[r], (long long)h * elem_bytes, large_bytes, den);
        flag[g] = (uint8_t)large;
        if (seg_flags) seg_flags[g] = large;
    }
    if (!plan) return;
    __syncthreads();

    // The plan. Every rank's rows fall into blocks: a block opens at the rank's
    // first segment, at a large segment and at the segment after one, so a
    // large segment is a block of its own and the others pack into blocks
    // between them. Each block is cut into kPlanRows-row items from its start
    // (the last one shorter). Items are numbered by start row, as walking each
    // rank's segments in turn would emit them. Thread tid owns the segments
    // [g0, g1); the start and the end of each segment's block come from
    // block-wide max and min scans over the openers' row offsets, which grow
    // with the segment index.
    constexpr int PT = (kSegLdsMax + kScanThreads - 1) / kScanThreads;
    const int per = (G + (int)blockDim.x - 1) / (int)blockDim.x;     // <= PT: G <= kSegLdsMax
    const int g0 = min(tid * per, G), g1 = min(g0 + per, G);
    auto opener = [&](int g) { return g % S == 0 || flag[g] != 0 || flag[g - 1] != 0; };
    int csum = 0;
    for (int g = g0; g < g1; ++g) csum += segc[g];
    int total_rows;
    const int off0 = block_excl_scan(csum, tmp, &total_rows);        // row offset of segment g0
    int o[PT];
    int last = -1, first = INT_MAX;
    {
        int run = off0;
#pragma unroll
        for (int k = 0; k < PT; ++k) {
            const int g = g0 + k;
            o[k] = run;
            if (g < g1) {
                if (opener(g)) {
                    first = min(first, run);
                    last = run;
                }
                run += segc[g];
            }
        }
    }
    block_incl_minmax<false>(last, part);
    const int carry_f = tid > 0 ? part[tid - 1] : -1;                // last opener before g0
    __syncthreads();
    block_incl_minmax<true>(first, part);
    const int carry_b = tid + 1 < (int)blockDim.x ? part[tid + 1] : INT_MAX;   // first opener after g1 - 1
    int eb[PT];
    {
        int nxt = carry_b == INT_MAX ? total_rows : carry_b;
#pragma unroll
        for (int k = PT - 1; k >= 0; --k) {
            const int g = g0 + k;
            eb[k] = nxt;
            if (g < g1 && opener(g)) nxt = o[k];
        }
    }
    int sb[PT], nmine = 0;
    {
        int cur = carry_f;
#pragma unroll
        for (int k = 0; k < PT; ++k) {
            const int g = g0 + k;
            if (g < g1 && opener(g)) cur = o[k];
            sb[k] = cur;
            if (g < g1) {
                const int lo = o[k] - cur, hi = lo + segc[g];
                nmine += (hi + kPlanRows - 1) / kPlanRows - (lo + kPlanRows - 1) / kPlanRows;
            }
        }
    }
    int nitems;
    int idx = block_excl_scan(nmine, tmp, &nitems);
#pragma unroll
    for (int k = 0; k < PT; ++k) {
        const int g = g0 + k;
        if (g >= g1) continue;
        const int lo = o[k] - sb[k], hi = lo + segc[g];
        for (int m = (lo + kPlanRows - 1) / kPlanRows; m < (hi + kPlanRows - 1) / kPlanRows; ++m) {
            const int st = sb[k] + kPlanRows * m;
            plan[idx++] = make_int2(st, min(st + kPlanRows, eb[k]));
        }
    }
    if (tid == 0) *nplan = nitems;
}

// --------------------------------------------------------------------------
// dispatch payload
// --------------------------------------------------------------------------

struct DispatchArgs {
    const char *x;
    const int32_t *ids;
    const int32_t *esc_in;
    char *expand_x;
    float *dyn;
    int32_t *assist;
    int32_t *esc_out;
    int32_t *erc;
    const int32_t *lr;
    const int32_t *pc;
    const int32_t *pci;
    const int32_t *boff;      // scan path only
    const int2 *plan;
    const int32_t *nplan;
    int W, bs, epr, h, K, nbs, R, E, S, NB;
    int direct;               // 1: blocks sum pc/pci themselves and write ep_recv_count
    int nsl;                  // copy kernel: slices per token
    long long rowbytes;       // bytes of one x row
    const float *qs;          // static quantisation coefficients
    int qkind;                // their shape: kStaticOne, kStaticColumn or kStaticExpert
    int store_mix;            // wavefront scatters: 0 half the stores plain, 1 a quarter, 2 none
    const uint8_t *mask;      // token mask (one-launch dispatch; the route kernel takes its own)
    int mask_kind;
    // adaptive schedule: per expand_x row, 1 if the row's segment is large (written by the token-major
    // kernels, which leave that row's payload out) and 0 otherwise; the threshold T, the bytes of an
    // expand_x row and max(W-1, 1)*epr for the predicate
    uint8_t *lflag;
    long long large, out_row_bytes, den;
};

// Whether piece j of copy k of a wavefront scatter is stored non-temporally
// (see store_stream): every other piece, every piece but one in four, or all.
__device__ __forceinline__ bool stream_piece(const DispatchArgs &a, int j, int k)
{
    return a.store_mix == 2 || ((j + k) & (a.store_mix == 1 ? 3 : 1)) != 0;
}

// ep_recv_count[r][el*W + s] = (end row of segment (el, s) of rank r) - (first row of rank r),
// from the chunk prefixes: first row of (chunk b, expert e) = sum_{b'<b} pci + sum_{b'>=b} pc.
__device__ void write_erc_direct(const DispatchArgs &a, size_t gtid, size_t nthreads)
{
    const size_t total = (size_t)a.W * a.S;
    for (size_t q = gtid; q < total; q += nthreads) {
        const int r = (int)(q / a.S), i = (int)(q % a.S), el = i / a.W, s = i % a.W;
        const int e = r * a.epr + el, e0 = r * a.epr, bend = (s + 1) * a.nbs;
        int end = 0, base = 0;
        // every chunk count of a pass is loaded before any is added (clamped
        // indices, the extra values dropped), so a pass costs one round trip
        for (int b0 = 0; b0 < a.NB; b0 += kChunkBatch) {
            int ve[kChunkBatch], vb[kChunkBatch];
#pragma unroll
            for (int j = 0; j < kChunkBatch; ++j) {
                const int b = min(b0 + j, a.NB - 1);
                ve[j] = (b < bend ? a.pci : a.pc)[(size_t)b * a.E + e];
                vb[j] = a.pc[(size_t)b * a.E + e0];
            }
#pragma unroll
            for (int j = 0; j < kChunkBatch; ++j) {
                end += b0 + j < a.NB ? ve[j] : 0;
                base += b0 + j < a.NB ? vb[j] : 0;
            }
        }
        a.erc[q] = end - base;
    }
}

// Rows of segment (expert e, source rank s): its source's route chunks' counts
// for e. The first four chunks' counts (all of them up to 1024 tokens per
// rank) are loaded together, so the caller can issue them with its other
// loads; further chunks take a loop.
__device__ __forceinline__ int segment_rows(const DispatchArgs &a, int e, int s)
{
    const int b0 = s * a.nbs, last = b0 + a.nbs - 1;
    int vi[4], vx[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const size_t idx = (size_t)min(b0 + u, last) * a.E + e;
        vi[u] = a.pci[idx];
        vx[u] = a.pc[idx];
    }
    int c = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) c += u < a.nbs ? vi[u] - vx[u] : 0;
    for (int b = b0 + 4; b <= last; ++b) c += a.pci[(size_t)b * a.E + e] - a.pc[(size_t)b * a.E + e];
    return c;
}

// The large-segment predicate (segment_large) for the segment of expert e
// from source rank s with c rows, from the route's chunk counts. Only a
// segment that passes the size test sums the rows its rank receives from the
// other ranks: over every route chunk of another source, that chunk's pairs to
// the rank's experts (an inclusive minus an exclusive prefix over experts).
__device__ bool pair_segment_large(const DispatchArgs &a, int e, int s, int c)
{
    const int r = e / a.epr;
    if (r == s || c <= 0 || (long long)c * a.out_row_bytes < a.large) return false;
    const int e0 = r * a.epr, e1 = e0 + a.epr - 1;
    long long remote = 0;
    for (int b = 0; b < a.NB; ++b)
        if (b / a.nbs != r) remote += a.pci[(size_t)b * a.E + e1] - a.pc[(size_t)b * a.E + e0];
    return segment_large(true, c, remote, a.out_row_bytes, a.large, a.den);
}

// Rows of the K pairs of token t, cooperatively over the calling threads
// [tid0, tid0 + nthr). ek/lk/off/rows: K ints of LDS each. The caller
// synchronises between the three phases (load / sum / finish).
__device__ __forceinline__ void pairs_load(const DispatchArgs &a, int t, int *ek, int *lk, int *off, int lt, int nthr)
{
    for (int k = lt; k < a.K; k += nthr) {
        const size_t p = (size_t)t * a.K + k;
        ek[k] = a.ids[p];
        lk[k] = a.lr[p];
        off[k] = 0;
    }
}

__device__ __forceinline__ void pairs_sum(const DispatchArgs &a, int t, const int *ek, int *off, int lt, int nthr)
{
    const int s = t / a.bs, tok = t % a.bs;
    const int bt = s * a.nbs + tok / kRouteTokens;
    if (a.direct) {
        const int n = a.K * a.NB;
        for (int i = lt; i < n; i += nthr) {
            const int k = i / a.NB, b = i % a.NB, e = ek[k];
            if ((unsigned)e < (unsigned)a.E) atomicAdd(&off[k], (b < bt ? a.pci : a.pc)[(size_t)b * a.E + e]);
        }
    } else {
        for (int k = lt; k < a.K; k += nthr) {
            const int e = ek[k];
            if ((unsigned)e < (unsigned)a.E) off[k] = a.boff[(size_t)bt * a.E + e];
        }
    }
}

// Final rows (-1 for an invalid pair); optionally writes assist_info / expand_scales.
// SKIP (adaptive schedule): a pair in a large segment also gets -1, after its
// meta, and its row's flag; the large-segment pass writes its payload.
template <bool SKIP = false>
__device__ __forceinline__ void pairs_finish(const DispatchArgs &a, int t, const int *ek, const int *lk,
                                             const int *off, int *rows, bool meta, int lt, int nthr)
{
    const int s = t / a.bs, tok = t % a.bs;
    for (int k = lt; k < a.K; k += nthr) {
        int row = -1;
        if ((unsigned)ek[k] < (unsigned)a.E && lk[k] >= 0) {
            row = off[k] + lk[k];
            if ((unsigned)row >= (unsigned)a.R) row = -1;
        }
        bool big = false;
        if constexpr (SKIP)
            if (row >= 0) big = pair_segment_large(a, ek[k], s, segment_rows(a, ek[k], s));
        rows[k] = big ? -1 : row;    // a large segment's row: meta here, payload by its own wavefronts
        if (meta && row >= 0) {
            a.assist[(size_t)row * 3 + 0] = s;
            a.assist[(size_t)row * 3 + 1] = tok;
            a.assist[(size_t)row * 3 + 2] = k;
            if (a.esc_out) a.esc_out[row] = a.esc_in[(size_t)t * a.K + k];
            if constexpr (SKIP) a.lflag[row] = big ? 1 : 0;
        }
    }
}

// Row of pair (t, lane) for lanes < K (-1 for other lanes and invalid pairs), from
// registers only: the chunk prefixes are summed by the lane itself (direct path)
// or read from the scan's table. Writes assist_info / expand_scales when asked.
// SKIP (adaptive schedule): as pairs_finish.
template <bool SKIP = false>
__device__ __forceinline__ int lane_pair_row(const DispatchArgs &a, int t, int lane, int e, int l, bool meta)
{
    const int s = t / a.bs, tok = t - s * a.bs;
    int row = -1;
    bool big = false;
    if (lane < a.K && (unsigned)e < (unsigned)a.E && l >= 0) {
        const int bt = s * a.nbs + tok / kRouteTokens;
        int c = 0;
        if constexpr (SKIP) c = segment_rows(a, e, s);    // loaded with the offsets below
        int off = 0;
        if (a.direct) {
            // all chunk counts of a pass loaded before any is added: one round trip per pass
            for (int b0 = 0; b0 < a.NB; b0 += kChunkBatch) {
                int v[kChunkBatch];
#pragma unroll
                for (int j = 0; j < kChunkBatch; ++j) {
                    const int b = min(b0 + j, a.NB - 1);
                    v[j] = (b < bt ? a.pci : a.pc)[(size_t)b * a.E + e];
                }
#pragma unroll
                for (int j = 0; j < kChunkBatch; ++j) off += b0 + j < a.NB ? v[j] : 0;
            }
        } else {
            off = a.boff[(size_t)bt * a.E + e];
        }
        row = off + l;
        if ((unsigned)row >= (unsigned)a.R) row = -1;
        if constexpr (SKIP) big = row >= 0 && pair_segment_large(a, e, s, c);
    }
    if (meta && row >= 0) {
        a.assist[(size_t)row * 3 + 0] = s;
        a.assist[(size_t)row * 3 + 1] = tok;
        a.assist[(size_t)row * 3 + 2] = lane;
        if (a.esc_out) a.esc_out[row] = a.esc_in[(size_t)t * a.K + lane];
        if constexpr (SKIP) a.lflag[row] = big ? 1 : 0;
    }
    return big ? -1 : row;       // a large segment's row: meta here, payload by its own wavefronts
}

// Token-major copy: block = (token, slice of kCopyThreads * kCopyUnroll chunks).
// For topk <= 64 each wavefront resolves the K rows in its own lanes (pair k in
// lane k, loaded before the payload) and reads them back with readlane: no LDS and
// no barrier; larger topk goes through LDS.
template <bool VEC, bool SKIP = false>
__global__ __launch_bounds__(kCopyThreads) void scatter_copy_kernel(DispatchArgs a)
{
    extern __shared__ int dsm[];                  // ek, lk, off, rows: 4 * K ints (topk > 64 only)
    const int t = blockIdx.x / a.nsl, sl = blockIdx.x % a.nsl;
    const int tid = threadIdx.x, lane = tid & 63;
    constexpr int SC = kCopyThreads * kCopyUnroll;

    if (a.direct) write_erc_direct(a, (size_t)blockIdx.x * kCopyThreads + tid, (size_t)gridDim.x * kCopyThreads);

    const bool small_k = a.K <= 64;
    int e = -1, l = -1;
    if (small_k) {
        const size_t pk = (size_t)t * a.K + (lane < a.K ? lane : 0);
        e = a.ids[pk];
        l = a.lr[pk];
    }
    const char *src = a.x + (size_t)t * a.rowbytes;
    const int n = VEC ? (int)(a.rowbytes / 16) : (int)(a.rowbytes / 2);
    const int c0 = sl * SC + tid;
    uint4 v[kCopyUnroll];
    uint16_t w[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int c = c0 + u * kCopyThreads;
        if constexpr (VEC) v[u] = c < n ? reinterpret_cast<const uint4 *>(src)[c] : make_uint4(0u, 0u, 0u, 0u);
        else w[u] = c < n ? reinterpret_cast<const uint16_t *>(src)[c] : (uint16_t)0;
    }

    if (small_k) {
        const int my_row = lane_pair_row<SKIP>(a, t, lane, e, l, sl == 0 && tid < 64);
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const int c = c0 + u * kCopyThreads;
            for (int k = 0; k < a.K; ++k) {
                const int row = __builtin_amdgcn_readlane(my_row, k);
                if (row < 0 || c >= n) continue;
                char *dst = a.expand_x + (size_t)row * a.rowbytes;
                if constexpr (VEC) store_stream(reinterpret_cast<uint4 *>(dst) + c, v[u]);
                else reinterpret_cast<uint16_t *>(dst)[c] = w[u];
            }
        }
        return;
    }

    int *ek = dsm, *lk = dsm + a.K, *off = dsm + 2 * a.K, *rows = dsm + 3 * a.K;
    pairs_load(a, t, ek, lk, off, tid, kCopyThreads);
    __syncthreads();
    pairs_sum(a, t, ek, off, tid, kCopyThreads);
    __syncthreads();
    pairs_finish<SKIP>(a, t, ek, lk, off, rows, sl == 0, tid, kCopyThreads);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int c = c0 + u * kCopyThreads;
        if (c >= n) continue;
        for (int k = 0; k < a.K; ++k) {
            const int row = rows[k];
            if (row < 0) continue;
            char *dst = a.expand_x + (size_t)row * a.rowbytes;
            if constexpr (VEC) store_stream(reinterpret_cast<uint4 *>(dst) + c, v[u]);
            else reinterpret_cast<uint16_t *>(dst)[c] = w[u];
        }
    }
}

template <bool FAST>
__device__ __forceinline__ int8_t quant1(float v, float scale, float inv)
{
    if (scale == 0.0f) return 0;
    float q;
    if (FAST) {
        const float q0 = v * inv;
        const float r = __builtin_fmaf(-q0, scale, v);
        q = __builtin_rintf(__builtin_fmaf(r, inv, q0));
    } else {
        q = __builtin_rintf(v / scale);
    }
    q = fminf(fmaxf(q, -127.0f), 127.0f);
    return (int8_t)(int)q;
}

constexpr float kFastQuantMinScale = 0x1p-100f;

template <class T>
__device__ __forceinline__ float amax_u4(uint4 v)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(T::load((uint16_t)(w[i >> 1] >> ((i & 1) * 16)))));
    return m;
}

// 8 elements -> 8 int8 codes packed into two words. FAST (scale >= 2^-100): after
// the FMA correction step, adding 1.5 * 2^23 rounds the quotient to an integer
// (ties to even) and leaves its two's-complement low byte in the low mantissa
// byte; |code| <= 127 always holds (|x| <= amax), so no clamp is needed. Both
// facts were checked exhaustively over all 16-bit (x, amax) pairs.
template <class T, bool FAST>
__device__ __forceinline__ uint2 quant_u4(uint4 v, float scale, float inv)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float x = T::load((uint16_t)(w[i >> 1] >> ((i & 1) * 16)));
        uint32_t q;
        if (FAST) {
            const float q0 = x * inv;
            const float r = __builtin_fmaf(-q0, scale, x);
            q = __float_as_uint(__builtin_fmaf(r, inv, q0) + 0x1.8p23f) & 0xffu;
        } else {
            q = (uint8_t)quant1<false>(x, scale, inv);
        }
        o[i >> 2] |= q << ((i & 3) * 8);
    }
    return make_uint2(o[0], o[1]);
}

// Quantise one token held by the wavefront (v: its row, 16 elements per lane
// and chunk) and store it to the K rows named by lanes 0..K-1 of my_row, plus
// the row scales.
template <class T, int J>
__device__ __forceinline__ void quant_store_wave(const DispatchArgs &a, int lane, const uint4 (&v)[J][2], int my_row)
{
    const int K = a.K, noc = a.h / 16;
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j)
        if (lane + 64 * j < noc) amax = fmaxf(amax, fmaxf(amax_u4<T>(v[j][0]), amax_u4<T>(v[j][1])));
    amax = wave_max(amax);
    const float scale = amax / 127.0f;
    const float inv = 1.0f / scale;
    const bool fast = scale >= kFastQuantMinScale;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        if (lane + 64 * j >= noc) continue;
        uint2 lo, hi;
        if (fast) {
            lo = quant_u4<T, true>(v[j][0], scale, inv);
            hi = quant_u4<T, true>(v[j][1], scale, inv);
        } else {
            lo = quant_u4<T, false>(v[j][0], scale, inv);
            hi = quant_u4<T, false>(v[j][1], scale, inv);
        }
        const uint4 q = make_uint4(lo.x, lo.y, hi.x, hi.y);
        for (int k = 0; k < K; ++k) {
            const int row = __builtin_amdgcn_readlane(my_row, k);
            if (row < 0) continue;
            uint4 *dst = reinterpret_cast<uint4 *>(a.expand_x + (size_t)row * a.h) + lane + 64 * j;
            if (stream_piece(a, j, k)) store_stream(dst, q);   // see store_stream
            else *dst = q;
        }
    }
    if (my_row >= 0) a.dyn[my_row] = scale;
}

// Static quantisation of 8 elements with their 8 coefficients: q = rint(x * c)
// of the exact product, ties to even, saturated to [-128, 127]. One fused
// multiply-add with M = 1.5 * 2^23 rounds x * c + M once; for |x * c| < 2^22
// that sum lies in [2^23, 2^24), where binary32 spacing is 1, so the result is
// M + rint(x * c) (M is even, so ties go to even as well), and larger
// magnitudes land outside [M - 128, M + 127]. Clamping to that range (a NaN
// clamps to M - 128) saturates, and the low mantissa byte is then the code in
// two's complement. Three byte permutes pack four codes.
template <class T>
__device__ __forceinline__ uint2 static_u4(uint4 v, float4 c0, float4 c1)
{
    constexpr float M = 0x1.8p23f;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    uint32_t r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float x = T::load((uint16_t)(w[i >> 1] >> ((i & 1) * 16)));
        r[i] = __float_as_uint(fminf(fmaxf(__builtin_fmaf(x, c[i], M), M - 128.0f), M + 127.0f));
    }
    // v_perm_b32 (a, b, sel): byte n of the result is byte sel.n of the 8-byte
    // value a:b (b in bytes 0-3); 0x0c gives a zero byte
    uint32_t o[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t lo = __builtin_amdgcn_perm(r[4 * h + 1], r[4 * h], 0x0c0c0400u);
        const uint32_t hi = __builtin_amdgcn_perm(r[4 * h + 3], r[4 * h + 2], 0x0c0c0400u);
        o[h] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
    return make_uint2(o[0], o[1]);
}

// Static quantisation of one token held by the wavefront with one coefficient
// or one per column (the same codes for every row, formed once), stored to the
// K rows named by lanes 0..K-1 of my_row.
template <class T, int J>
__device__ __forceinline__ void quant_store_wave_static(const DispatchArgs &a, int lane, const uint4 (&v)[J][2],
                                                        int my_row)
{
    const int K = a.K, noc = a.h / 16;
    const float c = a.qs[0];
    const float4 cc = make_float4(c, c, c, c);
    const float4 *cb = reinterpret_cast<const float4 *>(a.qs);
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int oc = lane + 64 * j;
        if (oc >= noc) continue;
        float4 c0 = cc, c1 = cc, c2 = cc, c3 = cc;
        if (a.qkind == kStaticColumn) {       // a single value has no element past qs[0]
            c0 = cb[4 * oc];
            c1 = cb[4 * oc + 1];
            c2 = cb[4 * oc + 2];
            c3 = cb[4 * oc + 3];
        }
        const uint2 lo = static_u4<T>(v[j][0], c0, c1);
        const uint2 hi = static_u4<T>(v[j][1], c2, c3);
        const uint4 q = make_uint4(lo.x, lo.y, hi.x, hi.y);
        for (int k = 0; k < K; ++k) {
            const int row = __builtin_amdgcn_readlane(my_row, k);
            if (row < 0) continue;
            uint4 *dst = reinterpret_cast<uint4 *>(a.expand_x + (size_t)row * a.h) + oc;
            if (stream_piece(a, j, k)) store_stream(dst, q);
            else *dst = q;
        }
    }
}

// Token-major copy for many tokens: one wavefront per token holds the row in
// registers (J 16-byte pieces per lane) and writes its K copies, like the
// quantising scatter, with the same checkerboard of plain and non-temporal
// stores (at 16 ranks x 256 tokens of bf16: 84 us; 109 us all non-temporal,
// 130 us all plain).
template <int J, bool SKIP = false>
__global__ __launch_bounds__(kQuantThreads) void scatter_copy_wave_kernel(DispatchArgs a)
{
    const int lane = threadIdx.x & 63;
    const int N = a.W * a.bs, K = a.K, nc = (int)(a.rowbytes / 16);
    if (a.direct) write_erc_direct(a, (size_t)blockIdx.x * kQuantThreads + threadIdx.x,
                                   (size_t)gridDim.x * kQuantThreads);
    const int nwaves = gridDim.x * (kQuantThreads / 64);
    for (int t = blockIdx.x * (kQuantThreads / 64) + (threadIdx.x >> 6); t < N; t += nwaves) {
        const size_t pk = (size_t)t * K + (lane < K ? lane : 0);
        const int e = a.ids[pk], l = a.lr[pk];
        const uint4 *src = reinterpret_cast<const uint4 *>(a.x + (size_t)t * a.rowbytes);
        uint4 v[J];
#pragma unroll
        for (int j = 0; j < J; ++j) v[j] = load_stream(src + min(lane + 64 * j, nc - 1));
        const int my_row = lane_pair_row<SKIP>(a, t, lane, e, l, true);
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int c = lane + 64 * j;
            if (c >= nc) continue;
            for (int k = 0; k < K; ++k) {
                const int row = __builtin_amdgcn_readlane(my_row, k);
                if (row < 0) continue;
                uint4 *dst = reinterpret_cast<uint4 *>(a.expand_x + (size_t)row * a.rowbytes) + c;
                if (stream_piece(a, j, k)) store_stream(dst, v[j]);
                else *dst = v[j];
            }
        }
    }
}

// ---- quantMode 3: per-group (128 elements) dynamic FP8 E4M3 ----
// 8 elements -> 8 E4M3 bytes, scale > 0. The quotient |x| / scale (FAST: the
// one-step corrected |x| * inv) is clamped to 448 and converted, with x's sign,
// by v_cvt_pk_fp8_f32 (OCP E4M3 on gfx950, round to nearest even). Two checks
// make the codes those of the definition: for every 16-bit (x, group max) pair,
// the corrected quotient rounded to E4M3 equals the E4M3 rounding of the
// correctly rounded binary32 quotient (checked exhaustively on the CPU; where
// that quotient lands on an E4M3 midpoint it is that binary32 value, not the
// exact rational one, whose tie decides); and on gfx950 the instruction
// equals that rounding for every binary32 |v| <= 448 (all 2,277,507,074 such
// values compared).
template <class T, bool FAST>
__device__ __forceinline__ uint2 fp8_u4(uint4 v, float scale, float inv)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint16_t bits = (uint16_t)(w[i >> 1] >> ((i & 1) * 16));
        const float ax = fabsf(T::load(bits));
        float q;
        if (FAST) {
            const float q0 = ax * inv;
            const float r = __builtin_fmaf(-q0, scale, ax);
            q = __builtin_fmaf(r, inv, q0);
        } else {
            q = ax / scale;
        }
        c[i] = __uint_as_float(__float_as_uint(fminf(q, 448.0f)) | ((uint32_t)(bits & 0x8000u) << 16));
    }
    uint32_t o[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        int p = __builtin_amdgcn_cvt_pk_fp8_f32(c[4 * h], c[4 * h + 1], 0, false);
        p = __builtin_amdgcn_cvt_pk_fp8_f32(c[4 * h + 2], c[4 * h + 3], p, true);
        o[h] = (uint32_t)p;
    }
    return make_uint2(o[0], o[1]);
}

// The wavefront holds one token (16 elements per lane and chunk); a group of
// 128 elements is 8 neighbouring lanes of one chunk, so its max is three xor
// shuffles. Per group: scale = max / 448 (0 -> codes 0), written for each of
// the K rows (dynamic_scales [rows, ceil(h/128)]).
template <class T, int J>
__device__ __forceinline__ void quant_store_wave_fp8(const DispatchArgs &a, int lane, const uint4 (&v)[J][2],
                                                     int my_row)
{
    const int K = a.K, noc = a.h / 16, G = (a.h + 127) / 128;
    float gs[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int c = lane + 64 * j;
        const bool live = c < noc;
        float amax = live ? fmaxf(amax_u4<T>(v[j][0]), amax_u4<T>(v[j][1])) : 0.0f;
        amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
        const float scale = amax / 448.0f;
        gs[j] = scale;
        const float inv = 1.0f / scale;
        uint4 q = make_uint4(0u, 0u, 0u, 0u);
        if (scale != 0.0f) {
            uint2 lo, hi;
            if (scale >= kFastQuantMinScale) {
                lo = fp8_u4<T, true>(v[j][0], scale, inv);
                hi = fp8_u4<T, true>(v[j][1], scale, inv);
            } else {
                lo = fp8_u4<T, false>(v[j][0], scale, inv);
                hi = fp8_u4<T, false>(v[j][1], scale, inv);
            }
            q = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
        if (!live) continue;
        for (int k = 0; k < K; ++k) {
            const int row = __builtin_amdgcn_readlane(my_row, k);
            if (row < 0) continue;
            uint4 *dst = reinterpret_cast<uint4 *>(a.expand_x + (size_t)row * a.h) + c;
            if (stream_piece(a, j, k)) store_stream(dst, q);   // see store_stream
            else *dst = q;
        }
    }
    // the row's group scales, one store per row: lane g takes group g's scale
    // from lane 8 * (g % 8) of chunk g / 8 (one 224-byte store per row at h =
    // 7168 instead of seven of 32 bytes: 52.3 against 53.5 us per dispatch)
    for (int g0 = 0; g0 < G; g0 += 64) {
        const int g = g0 + lane;
        float mys = 0.0f;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const float sj = __shfl(gs[j], (g & 7) << 3, 64);
            if ((g >> 3) == j) mys = sj;
        }
        if (g >= G) continue;
        for (int k = 0; k < K; ++k) {
            const int row = __builtin_amdgcn_readlane(my_row, k);
            if (row >= 0) a.dyn[(size_t)row * G + g] = mys;
        }
    }
}

// ---- quantMode 4: MX (OCP Microscaling v1.0), E4M3 elements, blocks of 32 ----
// 8 elements -> 8 E4M3 bytes. mult = 2^-shared is a power of two, so |x| * mult
// is exact (or, below 2^-126, rounds to a value whose E4M3 code is 0 anyway);
// it is clamped to 448 and converted with x's sign by v_cvt_pk_fp8_f32, the
// conversion checked for every binary32 |v| <= 448 (see fp8_u4).
template <class T>
__device__ __forceinline__ uint2 mx_u4(uint4 v, float mult)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint16_t bits = (uint16_t)(w[i >> 1] >> ((i & 1) * 16));
        const float q = fabsf(T::load(bits)) * mult;
        c[i] = __uint_as_float(__float_as_uint(fminf(q, 448.0f)) | ((uint32_t)(bits & 0x8000u) << 16));
    }
    uint32_t o[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        int p = __builtin_amdgcn_cvt_pk_fp8_f32(c[4 * h], c[4 * h + 1], 0, false);
        p = __builtin_amdgcn_cvt_pk_fp8_f32(c[4 * h + 2], c[4 * h + 3], p, true);
        o[h] = (uint32_t)p;
    }
    return make_uint2(o[0], o[1]);
}

// A block of 32 elements is two neighbouring lanes of one chunk (16 elements
// each), so its max is one xor shuffle. The shared exponent floor(log2 max) - 8,
// clamped below at -127, is the max's binary32 exponent field minus 8 (at least
// 0), which is also the E8M0 byte: a subnormal or zero max has field 0, and a
// 16-bit token's max keeps the byte at or below 246, so 2^(127 - byte) is a
// normal binary32 number. The row's bytes leave as 4-byte words: lane r*8 of
// chunk j packs blocks 32j + 4r .. + 3 with three shuffles, and lane g of the
// store loop takes word g (one 224-byte store per row at h = 7168); where the
// row's byte count or the buffer's address is not a multiple of 4, each word
// leaves as byte stores instead.
template <class T, int J>
__device__ __forceinline__ void quant_store_wave_mx(const DispatchArgs &a, int lane, const uint4 (&v)[J][2],
                                                    int my_row)
{
    const int K = a.K, noc = a.h / 16, B = (a.h + 31) / 32, G4 = (B + 3) / 4;
    uint8_t *sbytes = reinterpret_cast<uint8_t *>(a.dyn);
    uint32_t dw[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int c = lane + 64 * j;
        const bool live = c < noc;
        float amax = live ? fmaxf(amax_u4<T>(v[j][0]), amax_u4<T>(v[j][1])) : 0.0f;
        amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
        const uint32_t byte = (uint32_t)max((int)(__float_as_uint(amax) >> 23) - 8, 0);
        const float mult = __uint_as_float((254u - byte) << 23);
        dw[j] = byte | ((uint32_t)__shfl_down((int)byte, 2, 64) << 8) |
                ((uint32_t)__shfl_down((int)byte, 4, 64) << 16) | ((uint32_t)__shfl_down((int)byte, 6, 64) << 24);
        if (!live) continue;
        const uint2 lo = mx_u4<T>(v[j][0], mult), hi = mx_u4<T>(v[j][1], mult);
        const uint4 q = make_uint4(lo.x, lo.y, hi.x, hi.y);
        for (int k = 0; k < K; ++k) {
            const int row = __builtin_amdgcn_readlane(my_row, k);
            if (row < 0) continue;
            uint4 *dst = reinterpret_cast<uint4 *>(a.expand_x + (size_t)row * a.h) + c;
            if (stream_piece(a, j, k)) store_stream(dst, q);   // see store_stream
            else *dst = q;
        }
    }
    const bool words = (B & 3) == 0 && (reinterpret_cast<uintptr_t>(sbytes) & 3) == 0;
    for (int g0 = 0; g0 < G4; g0 += 64) {
        const int g = g0 + lane;
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const uint32_t wj = (uint32_t)__shfl((int)dw[j], (g & 7) << 3, 64);
            if ((g >> 3) == j) word = wj;
        }
        if (g >= G4) continue;
        for (int k = 0; k < K; ++k) {
            const int row = __builtin_amdgcn_readlane(my_row, k);
            if (row < 0) continue;
            uint8_t *dst = sbytes + (size_t)row * B + 4 * g;
            if (words) {
                *reinterpret_cast<uint32_t *>(dst) = word;
            } else {
                for (int i = 0; i < 4; ++i)
                    if (4 * g + i < B) dst[i] = (uint8_t)(word >> (8 * i));
            }
        }
    }
}

// The quantising scatter (aclnnMoeDistributeDispatchV4 quantMode 1, 2, 3 and 4),
// one wavefront per token. QM 1: the static codes above (one coefficient or one
// per column; per-expert coefficients take the source-group kernel below); QM 2:
// scale = max|x| / 127 over the token (fp32, correctly rounded),
// q = rint(x / scale) (0 for an all-zero token); QM 3: the per-group FP8 codes
// above; QM 4: the MX codes and scale bytes above. Codes go to every destination row. Lane k loads pair k's id and
// in-chunk rank before the row's 16-byte loads, so both are in flight together;
// rows reach the store loop through readlane. No LDS, no barrier. Needs
// h % 16 == 0, h <= 1024 * J, topk <= kQuantMaxK.
template <class T, int J, int QM, bool SKIP = false>
__global__ __launch_bounds__(kQuantThreads) void scatter_quant_wave_kernel(DispatchArgs a)
{
    const int lane = threadIdx.x & 63;
    const int N = a.W * a.bs, K = a.K, noc = a.h / 16;
    if (a.direct) write_erc_direct(a, (size_t)blockIdx.x * kQuantThreads + threadIdx.x,
                                   (size_t)gridDim.x * kQuantThreads);
    const int nwaves = gridDim.x * (kQuantThreads / 64);
    for (int t = blockIdx.x * (kQuantThreads / 64) + (threadIdx.x >> 6); t < N; t += nwaves) {
        const size_t pk = (size_t)t * K + (lane < K ? lane : 0);
        // the pair loads go out before the token's, and the row resolution waits for
        // them alone: its chunk-count loads then overlap the token loads
        const int e = a.ids[pk], l = a.lr[pk];
        __builtin_amdgcn_sched_barrier(0);
        const uint4 *src = reinterpret_cast<const uint4 *>(a.x + (size_t)t * a.rowbytes);
        uint4 v[J][2];
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int oc = min(lane + 64 * j, noc - 1);     // duplicate loads past the row end are ignored
            v[j][0] = src[2 * oc];
            v[j][1] = src[2 * oc + 1];
        }
        __builtin_amdgcn_sched_barrier(0);
        const int my_row = lane_pair_row<SKIP>(a, t, lane, e, l, true);
        if constexpr (QM == MOE_QUANT_DYN_GROUP) quant_store_wave_fp8<T, J>(a, lane, v, my_row);
        else if constexpr (QM == MOE_QUANT_MX) quant_store_wave_mx<T, J>(a, lane, v, my_row);
        else if constexpr (QM == MOE_QUANT_STATIC) quant_store_wave_static<T, J>(a, lane, v, my_row);
        else quant_store_wave<T, J>(a, lane, v, my_row);
    }
}

// Rows, assist_info, expand_scales (and, on the direct path, ep_recv_count)
// without the payload: one wavefront per token. It runs before a payload pass
// that walks expand_x in expert-major order, and also reads its token once,
// contiguously, so that the payload pass's scattered re-reads of token slices
// find them in the Infinity Cache instead of HBM. At 16 ranks x 256 bf16 tokens
// with per-expert static coefficients that read takes a timed step (after the
// 1 GiB eviction) from 192.7 to 169.5 us; back to back, with the tokens
// already cached, it costs 6 us (157 -> 163 us).
__global__ __launch_bounds__(kQuantThreads) void dispatch_meta_kernel(DispatchArgs a)
{
    const int lane = threadIdx.x & 63;
    const int N = a.W * a.bs, K = a.K;
    if (a.direct) write_erc_direct(a, (size_t)blockIdx.x * kQuantThreads + threadIdx.x,
                                   (size_t)gridDim.x * kQuantThreads);
    const int t = blockIdx.x * (kQuantThreads / 64) + (threadIdx.x >> 6);
    if (t >= N) return;
    const size_t pk = (size_t)t * K + (lane < K ? lane : 0);
    lane_pair_row(a, t, lane, a.ids[pk], a.lr[pk], true);
    const uint4 *src = reinterpret_cast<const uint4 *>(a.x + (size_t)t * a.rowbytes);
    const int nc = (int)(a.rowbytes / 16);
    uint32_t sink = 0;
    for (int c = lane; c < nc; c += 64) {
        const uint4 v = src[c];
        sink ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    asm volatile("" ::"v"(sink));      // keeps the loads: their only purpose is to leave the lines cached
}

// Static quantisation with one coefficient per expert and column, expert-major
// in source-rank groups. Inside expert e's rows (rank r, local expert el) the
// order is source rank, then token, so the rows of e from source ranks
// [s0, s1) are one contiguous range whose bounds ep_recv_count gives.
// Workgroup b serves column slice g = b % kXcds of the rows of expert
// e = (b / kXcds) % E from source group grp (part of them when a group's rows
// are many); workgroups run group by group. Per XCD the group's token slices
// (kStaticGroupBytes: about 1170 tokens at h = 7168) and the coefficient slice
// then fit in L2: each lane keeps its piece of expert e's coefficients in
// registers and re-reads token pieces from L2. At 16 ranks x 256 bf16 tokens
// the dispatch takes about 64.5 us; token-major waves that read each row's
// coefficients took 118 us, a hidden-dimension split without groups 85-95 us,
// and expert-major without groups (tokens re-read from the Infinity Cache)
// 92 us. Needs assist_info and ep_recv_count written (dispatch_meta_kernel)
// and h <= 2048 * kXcds (PL = 1 up to 1024 * kXcds).
template <class T, int PL>
__global__ __launch_bounds__(kQuantThreads) void scatter_static_group_kernel(DispatchArgs a, int spg, int parts)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, noc = a.h / 16;
    const int g = (int)(blockIdx.x % kXcds);
    const int q = (int)(blockIdx.x / kXcds), e = q % a.E, q2 = q / a.E, part = q2 % parts, grp = q2 / parts;
    const int per = (noc + kXcds - 1) / kXcds;
    const int s0 = grp * spg, s1 = min(s0 + spg, a.W);
    if (s0 >= s1) return;
    const int r = e / a.epr, el = e - r * a.epr;
    int b = 0;                                     // first row of rank r
    for (int x = lane; x < r; x += 64) b += a.erc[(size_t)x * a.S + a.S - 1];
    b = wave_sum_i(b);
    const int i0 = el * a.W + s0, i1 = el * a.W + s1 - 1;
    const int row0 = b + (i0 > 0 ? a.erc[(size_t)r * a.S + i0 - 1] : 0);
    const int row1 = min(b + a.erc[(size_t)r * a.S + i1], a.R);
    if (row0 >= row1) return;
    // PL 16-element pieces per lane: piece p of the slice is lane + 64 * p
    int oc[PL];
    bool mine[PL];
    float4 c[PL][4];
#pragma unroll
    for (int p = 0; p < PL; ++p) {
        oc[p] = g * per + lane + 64 * p;
        mine[p] = lane + 64 * p < per && oc[p] < noc;
        const float4 *cb = reinterpret_cast<const float4 *>(a.qs + (size_t)e * a.h) + 4 * min(oc[p], noc - 1);
        c[p][0] = cb[0];
        c[p][1] = cb[1];
        c[p][2] = cb[2];
        c[p][3] = cb[3];
    }
    const int wstep = parts * (kQuantThreads / 64);
    const int rfirst = row0 + part * (kQuantThreads / 64) + wave;
    const int nmine = rfirst < row1 ? (row1 - rfirst + wstep - 1) / wstep : 0;
    for (int base = 0; base < nmine; base += 64) {
        // lane i holds the token of the wave's row base + i, so each row costs one
        // dependent load (its token slice) instead of two: 64.5 against 67-70 us
        // per dispatch at 16 ranks x 256 bf16 tokens (two rows in flight: 65.2 us)
        int my_src = -1;
        if (base + lane < nmine) {
            const int row = rfirst + (base + lane) * wstep;
            const int s = a.assist[(size_t)row * 3 + 0], tok = a.assist[(size_t)row * 3 + 1];
            if ((unsigned)s < (unsigned)a.W && (unsigned)tok < (unsigned)a.bs) my_src = s * a.bs + tok;
        }
        const int cnt = min(64, nmine - base);
        for (int i = 0; i < cnt; ++i) {
            const int t = __builtin_amdgcn_readlane(my_src, i);
            if (t < 0) continue;
            const int row = rfirst + (base + i) * wstep;
            const uint4 *src = reinterpret_cast<const uint4 *>(a.x + (size_t)t * a.rowbytes);
#pragma unroll
            for (int p = 0; p < PL; ++p) {
                if (!mine[p]) continue;
                const uint2 lo = static_u4<T>(src[2 * oc[p]], c[p][0], c[p][1]);
                const uint2 hi = static_u4<T>(src[2 * oc[p] + 1], c[p][2], c[p][3]);
                uint4 *dst = reinterpret_cast<uint4 *>(a.expand_x + (size_t)row * a.h) + oc[p];
                // non-temporal only: 70 us against 78 us with the mixed stores at 16 x 256 tokens
                store_stream(dst, make_uint4(lo.x, lo.y, hi.x, hi.y));
            }
        }
    }
}

// The same quantisation, one block per token, any h and topk (8-byte stores
// when h % 8 == 0 and the pointers allow, single bytes otherwise).
template <class T, bool VEC>
__device__ float quant_row_block(const uint16_t *__restrict__ src, int8_t *__restrict__ dst_base,
                                 const int *rows, int ndst, int h, float *red)
{
    float amax = 0.0f;
    if (VEC) {
        const int nch = h / 8;
        const uint4 *s4 = reinterpret_cast<const uint4 *>(src);
        for (int c = threadIdx.x; c < nch; c += blockDim.x) amax = fmaxf(amax, amax_u4<T>(s4[c]));
        amax = block_max(amax, red);
        const float scale = amax / 127.0f, inv = 1.0f / scale;
        const bool fast = scale >= kFastQuantMinScale;
        for (int c = threadIdx.x; c < nch; c += blockDim.x) {
            const uint2 q = fast ? quant_u4<T, true>(s4[c], scale, inv) : quant_u4<T, false>(s4[c], scale, inv);
            for (int k = 0; k < ndst; ++k)
                if (rows[k] >= 0) reinterpret_cast<uint2 *>(dst_base + (size_t)rows[k] * h)[c] = q;
        }
        return scale;
    }
    for (int j = threadIdx.x; j < h; j += blockDim.x) amax = fmaxf(amax, fabsf(T::load(src[j])));
    amax = block_max(amax, red);
    const float scale = amax / 127.0f, inv = 1.0f / scale;
    const bool fast = scale >= kFastQuantMinScale;
    for (int j = threadIdx.x; j < h; j += blockDim.x) {
        const float x = T::load(src[j]);
        const int8_t q = fast ? quant1<true>(x, scale, inv) : quant1<false>(x, scale, inv);
        for (int k = 0; k < ndst; ++k)
            if (rows[k] >= 0) dst_base[(size_t)rows[k] * h + j] = q;
    }
    return scale;
}

template <class T, bool VEC, bool SKIP = false>
__global__ __launch_bounds__(kBlockThreads) void scatter_quant_block_kernel(DispatchArgs a)
{
    extern __shared__ int dsm[];
    __shared__ float red[kBlockThreads / 64];
    int *ek = dsm, *lk = dsm + a.K, *off = dsm + 2 * a.K, *rows = dsm + 3 * a.K;
    const int t = blockIdx.x;
    if (a.direct) write_erc_direct(a, (size_t)blockIdx.x * kBlockThreads + threadIdx.x,
                                   (size_t)gridDim.x * kBlockThreads);
    pairs_load(a, t, ek, lk, off, threadIdx.x, kBlockThreads);
    __syncthreads();
    pairs_sum(a, t, ek, off, threadIdx.x, kBlockThreads);
    __syncthreads();
    pairs_finish<SKIP>(a, t, ek, lk, off, rows, true, threadIdx.x, kBlockThreads);
    __syncthreads();
    const float scale = quant_row_block<T, VEC>(reinterpret_cast<const uint16_t *>(a.x) + (size_t)t * a.h,
                                                reinterpret_cast<int8_t *>(a.expand_x), rows, a.K, a.h, red);
    for (int k = threadIdx.x; k < a.K; k += kBlockThreads)
        if (rows[k] >= 0) a.dyn[rows[k]] = scale;
}

// Segment schedule, pass 1: assist_info / expand_scales for every pair (scan path offsets).
__global__ __launch_bounds__(kBlockThreads) void segment_meta_kernel(DispatchArgs a)
{
    const size_t p = (size_t)blockIdx.x * kBlockThreads + threadIdx.x;
    const size_t npairs = (size_t)a.W * a.bs * a.K;
    if (p >= npairs) return;
    const int t = (int)(p / a.K), k = (int)(p % a.K), s = t / a.bs, tok = t % a.bs;
    const size_t b = (size_t)s * a.nbs + tok / kRouteTokens;
    const int e = a.ids[p], l = a.lr[p];
    if ((unsigned)e >= (unsigned)a.E || l < 0) return;
    const int row = a.boff[b * a.E + e] + l;
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
__global__ __launch_bounds__(kBlockThreads) void segment_payload_kernel(DispatchArgs a)
{
    __shared__ int one[1];
    __shared__ float red[kBlockThreads / 64];
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
                const char *src = a.x + t * a.rowbytes;
                char *dst = a.expand_x + (size_t)row * a.rowbytes;
                if (VEC) {
                    for (int c = threadIdx.x; c < (int)(a.rowbytes / 16); c += kBlockThreads)
                        reinterpret_cast<uint4 *>(dst)[c] = reinterpret_cast<const uint4 *>(src)[c];
                } else {
                    for (int c = threadIdx.x; c < (int)(a.rowbytes / 2); c += kBlockThreads)
                        reinterpret_cast<uint16_t *>(dst)[c] = reinterpret_cast<const uint16_t *>(src)[c];
                }
            } else {
                const uint16_t *src = reinterpret_cast<const uint16_t *>(a.x) + t * a.h;
                int8_t *dst = reinterpret_cast<int8_t *>(a.expand_x);
                const float scale = MODE == 1 ? quant_row_block<F16, VEC>(src, dst, one, 1, a.h, red)
                                              : quant_row_block<BF16, VEC>(src, dst, one, 1, a.h, red);
                if (threadIdx.x == 0) a.dyn[row] = scale;
            }
            __syncthreads();
        }
    }
}

// Segment schedule, pass 2 on the wavefront path (rows of at most 16 KiB in
// 16-byte pieces, or per-token int8 with h % 16 == 0 and h <= 16384): a
// workgroup takes plan items, its lanes load the item's source tokens from
// assist_info at once (one row per lane), and wavefront w fills rows lo + w,
// lo + w + 4, ... with the token-major kernels' per-wavefront code (the
// same stores, and for int8 the same codes and scale). 16 ranks x 256 bf16
// tokens, int8: 132 us per dispatch (292 us with a workgroup walking its
// item's rows one at a time), against 50 us for the token-major schedule,
// which reads each token once instead of once per destination row.
__device__ __forceinline__ int item_row_token(const DispatchArgs &a, int lo, int hi, int lane)
{
    int t = -1;
    if (lane < hi - lo) {
        const int row = lo + lane;
        const int s = a.assist[(size_t)row * 3 + 0], tok = a.assist[(size_t)row * 3 + 1];
        if ((unsigned)s < (unsigned)a.W && (unsigned)tok < (unsigned)a.bs) t = s * a.bs + tok;
    }
    return t;
}

template <int J>
__global__ __launch_bounds__(kQuantThreads) void segment_copy_wave_kernel(DispatchArgs a)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n16 = (int)(a.rowbytes / 16), n = *a.nplan;
    for (int item = blockIdx.x; item < n; item += gridDim.x) {
        const int2 it = a.plan[item];
        const int lo = max(it.x, 0), hi = min(it.y, a.R);
        const int my_t = item_row_token(a, lo, hi, lane);
        for (int i = wave; i < min(hi - lo, 64); i += kQuantThreads / 64) {
            const int t = __builtin_amdgcn_readlane(my_t, i);
            if (t < 0) continue;
            const uint4 *src = reinterpret_cast<const uint4 *>(a.x + (size_t)t * a.rowbytes);
            uint4 *dst = reinterpret_cast<uint4 *>(a.expand_x + (size_t)(lo + i) * a.rowbytes);
            uint4 v[J];
#pragma unroll
            for (int j = 0; j < J; ++j) v[j] = src[min(lane + 64 * j, n16 - 1)];
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int c = lane + 64 * j;
                if (c >= n16) continue;
                if (j & 1) store_stream(dst + c, v[j]);    // the token-major copy's mix
                else dst[c] = v[j];
            }
        }
    }
}

template <class T, int J>
__global__ __launch_bounds__(kQuantThreads) void segment_quant_wave_kernel(DispatchArgs a)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int noc = a.h / 16, n = *a.nplan;
    DispatchArgs one = a;          // one destination row per token visit
    one.K = 1;
    for (int item = blockIdx.x; item < n; item += gridDim.x) {
        const int2 it = a.plan[item];
        const int lo = max(it.x, 0), hi = min(it.y, a.R);
        const int my_t = item_row_token(a, lo, hi, lane);
        for (int i = wave; i < min(hi - lo, 64); i += kQuantThreads / 64) {
            const int t = __builtin_amdgcn_readlane(my_t, i);
            if (t < 0) continue;
            const uint4 *src = reinterpret_cast<const uint4 *>(a.x + (size_t)t * a.rowbytes);
            uint4 v[J][2];
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int oc = min(lane + 64 * j, noc - 1);
                v[j][0] = src[2 * oc];
                v[j][1] = src[2 * oc + 1];
            }
            quant_store_wave<T, J>(one, lane, v, lane == 0 ? lo + i : -1);
        }
    }
}

// Adaptive schedule, after the token-major scatter: the rows of the large
// segments. A large segment's rows are consecutive in expand_x, so each
// wavefront takes windows of kPlanRows consecutive rows and fills every row of
// its window that the token-major kernels left out (flagged), in row order,
// from the token its assist_info names, with their per-wavefront copy or
// quantiser.
// Rows at and past the active total (the ranks' ep_recv_count totals) were
// not written by this call and are not read.
__device__ __forceinline__ int active_rows(const DispatchArgs &a, int lane)
{
    int v = 0;
    for (int r = lane; r < a.W; r += 64) v += a.erc[(size_t)r * a.S + a.S - 1];
    return min(wave_sum_i(v), a.R);
}

// Lane i of window w0 (WR rows): the flag of row w0 + i, loaded at a clamped
// index without waiting for the active total; window_token then drops rows at
// and past it, and reads the token of each flagged row from assist_info.
template <int WR>
__device__ __forceinline__ int window_load(const DispatchArgs &a, int w0, int lane)
{
    return a.lflag[min(w0 + (lane < WR ? lane : 0), a.R - 1)];
}

template <int WR>
__device__ __forceinline__ int window_token(const DispatchArgs &a, int v, int w0, int A, int lane)
{
    int t = -1;
    if (lane < WR && w0 + lane < A && v != 0) {
        const size_t row = (size_t)(w0 + lane);
        const int s = a.assist[row * 3 + 0], tok = a.assist[row * 3 + 1];
        if ((unsigned)s < (unsigned)a.W && (unsigned)tok < (unsigned)a.bs) t = s * a.bs + tok;
    }
    return t;
}

template <int J>
__global__ __launch_bounds__(kQuantThreads) void large_copy_wave_kernel(DispatchArgs a)
{
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * (kQuantThreads / 64) + (threadIdx.x >> 6), nw = gridDim.x * (kQuantThreads / 64);
    const int n16 = (int)(a.rowbytes / 16);
    const int v0 = window_load<kPlanRows>(a, gw * kPlanRows, lane), A = active_rows(a, lane);
    for (int w0 = gw * kPlanRows; w0 < A; w0 += nw * kPlanRows) {
        const int my_t = window_token<kPlanRows>(a, w0 == gw * kPlanRows ? v0 : window_load<kPlanRows>(a, w0, lane),
                                                 w0, A, lane);
        for (unsigned long long m = __builtin_amdgcn_ballot_w64(my_t >= 0); m; m &= m - 1) {
            const int i = __builtin_ctzll(m);
            const int t = __builtin_amdgcn_readlane(my_t, i);
            const uint4 *src = reinterpret_cast<const uint4 *>(a.x + (size_t)t * a.rowbytes);
            uint4 *dst = reinterpret_cast<uint4 *>(a.expand_x + (size_t)(w0 + i) * a.rowbytes);
            uint4 v[J];
#pragma unroll
            for (int j = 0; j < J; ++j) v[j] = src[min(lane + 64 * j, n16 - 1)];
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int c = lane + 64 * j;
                if (c >= n16) continue;
                if (j & 1) store_stream(dst + c, v[j]);    // the token-major copy's mix
                else dst[c] = v[j];
            }
        }
    }
}

template <class T, int J>
__global__ __launch_bounds__(kQuantThreads) void large_quant_wave_kernel(DispatchArgs a)
{
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * (kQuantThreads / 64) + (threadIdx.x >> 6), nw = gridDim.x * (kQuantThreads / 64);
    const int noc = a.h / 16;
    const int v0 = window_load<kPlanRows>(a, gw * kPlanRows, lane), A = active_rows(a, lane);
    DispatchArgs one = a;          // one destination row per token visit
    one.K = 1;
    for (int w0 = gw * kPlanRows; w0 < A; w0 += nw * kPlanRows) {
        const int my_t = window_token<kPlanRows>(a, w0 == gw * kPlanRows ? v0 : window_load<kPlanRows>(a, w0, lane),
                                                 w0, A, lane);
        for (unsigned long long m = __builtin_amdgcn_ballot_w64(my_t >= 0); m; m &= m - 1) {
            const int i = __builtin_ctzll(m);
            const int t = __builtin_amdgcn_readlane(my_t, i);
            const uint4 *src = reinterpret_cast<const uint4 *>(a.x + (size_t)t * a.rowbytes);
            uint4 v[J][2];
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int oc = min(lane + 64 * j, noc - 1);
                v[j][0] = src[2 * oc];
                v[j][1] = src[2 * oc + 1];
            }
            quant_store_wave<T, J>(one, lane, v, lane == 0 ? w0 + i : -1);
        }
    }
}

// The same for rows off the wavefront path: the block takes windows, and fills
// each left-out row with the whole block.
template <int MODE, bool VEC>   // MODE 0: copy, 1: quant fp16, 2: quant bf16
__global__ __launch_bounds__(kBlockThreads) void large_payload_block_kernel(DispatchArgs a)
{
    __shared__ int one[1], win[kPlanRows], act[1];
    __shared__ float red[kBlockThreads / 64];
    if (threadIdx.x < 64) {
        const int A = active_rows(a, threadIdx.x);
        if (threadIdx.x == 0) act[0] = A;
    }
    __syncthreads();
    const int A = act[0];
    for (int w0 = blockIdx.x * kPlanRows; w0 < A; w0 += gridDim.x * kPlanRows) {
        if (threadIdx.x < kPlanRows)
            win[threadIdx.x] = window_token<kPlanRows>(a, window_load<kPlanRows>(a, w0, threadIdx.x), w0, A, threadIdx.x);
        __syncthreads();
        for (int i = 0; i < kPlanRows; ++i) {
            const int t = win[i];
            if (t < 0) continue;
            const int row = w0 + i;
            if (threadIdx.x == 0) one[0] = row;
            __syncthreads();
            if (MODE == 0) {
                const char *src = a.x + (size_t)t * a.rowbytes;
                char *dst = a.expand_x + (size_t)row * a.rowbytes;
                if (VEC) {
                    for (int c = threadIdx.x; c < (int)(a.rowbytes / 16); c += kBlockThreads)
                        reinterpret_cast<uint4 *>(dst)[c] = reinterpret_cast<const uint4 *>(src)[c];
                } else {
                    for (int c = threadIdx.x; c < (int)(a.rowbytes / 2); c += kBlockThreads)
                        reinterpret_cast<uint16_t *>(dst)[c] = reinterpret_cast<const uint16_t *>(src)[c];
                }
            } else {
                const uint16_t *src = reinterpret_cast<const uint16_t *>(a.x) + (size_t)t * a.h;
                int8_t *dst = reinterpret_cast<int8_t *>(a.expand_x);
                const float scale = MODE == 1 ? quant_row_block<F16, VEC>(src, dst, one, 1, a.h, red)
                                              : quant_row_block<BF16, VEC>(src, dst, one, 1, a.h, red);
                if (threadIdx.x == 0) a.dyn[row] = scale;
            }
            __syncthreads();
        }
        __syncthreads();
    }
}

void launch_segment_copy_wave(int J, dim3 g, dim3 b, hipStream_t st, const DispatchArgs &a)
{
    if (J <= 1) hipLaunchKernelGGL((segment_copy_wave_kernel<1>), g, b, 0, st, a);
    else if (J <= 2) hipLaunchKernelGGL((segment_copy_wave_kernel<2>), g, b, 0, st, a);
    else if (J <= 4) hipLaunchKernelGGL((segment_copy_wave_kernel<4>), g, b, 0, st, a);
    else if (J <= 8) hipLaunchKernelGGL((segment_copy_wave_kernel<8>), g, b, 0, st, a);
    else if (J <= 14) hipLaunchKernelGGL((segment_copy_wave_kernel<14>), g, b, 0, st, a);
    else hipLaunchKernelGGL((segment_copy_wave_kernel<16>), g, b, 0, st, a);
}

template <class T>
void launch_segment_quant_wave(int J, dim3 g, dim3 b, hipStream_t st, const DispatchArgs &a)
{
    if (J <= 1) hipLaunchKernelGGL((segment_quant_wave_kernel<T, 1>), g, b, 0, st, a);
    else if (J <= 2) hipLaunchKernelGGL((segment_quant_wave_kernel<T, 2>), g, b, 0, st, a);
    else if (J <= 4) hipLaunchKernelGGL((segment_quant_wave_kernel<T, 4>), g, b, 0, st, a);
    else if (J <= 7) hipLaunchKernelGGL((segment_quant_wave_kernel<T, 7>), g, b, 0, st, a);
    else if (J <= 8) hipLaunchKernelGGL((segment_quant_wave_kernel<T, 8>), g, b, 0, st, a);
    else if (J <= 12) hipLaunchKernelGGL((segment_quant_wave_kernel<T, 12>), g, b, 0, st, a);
    else hipLaunchKernelGGL((segment_quant_wave_kernel<T, 16>), g, b, 0, st, a);
}

void launch_large_copy_wave(int J, dim3 g, dim3 b, hipStream_t st, const DispatchArgs &a)
{
    if (J <= 1) hipLaunchKernelGGL((large_copy_wave_kernel<1>), g, b, 0, st, a);
    else if (J <= 2) hipLaunchKernelGGL((large_copy_wave_kernel<2>), g, b, 0, st, a);
    else if (J <= 4) hipLaunchKernelGGL((large_copy_wave_kernel<4>), g, b, 0, st, a);
    else if (J <= 8) hipLaunchKernelGGL((large_copy_wave_kernel<8>), g, b, 0, st, a);
    else if (J <= 14) hipLaunchKernelGGL((large_copy_wave_kernel<14>), g, b, 0, st, a);
    else hipLaunchKernelGGL((large_copy_wave_kernel<16>), g, b, 0, st, a);
}

template <class T>
void launch_large_quant_wave(int J, dim3 g, dim3 b, hipStream_t st, const DispatchArgs &a)
{
    if (J <= 1) hipLaunchKernelGGL((large_quant_wave_kernel<T, 1>), g, b, 0, st, a);
    else if (J <= 2) hipLaunchKernelGGL((large_quant_wave_kernel<T, 2>), g, b, 0, st, a);
    else if (J <= 4) hipLaunchKernelGGL((large_quant_wave_kernel<T, 4>), g, b, 0, st, a);
    else if (J <= 7) hipLaunchKernelGGL((large_quant_wave_kernel<T, 7>), g, b, 0, st, a);
    else if (J <= 8) hipLaunchKernelGGL((large_quant_wave_kernel<T, 8>), g, b, 0, st, a);
    else if (J <= 12) hipLaunchKernelGGL((large_quant_wave_kernel<T, 12>), g, b, 0, st, a);
    else hipLaunchKernelGGL((large_quant_wave_kernel<T, 16>), g, b, 0, st, a);
}


// --------------------------------------------------------------------------
// one launch per call for small batches
// --------------------------------------------------------------------------
//
// Rows by counting. Rows are ordered by expert, then source rank, then token,
// and for pairs of one expert that is the order of their flat index p = t*K + k
// (a token names each expert once). With key(p) = e*N*K + p for a pair that is
// exchanged (active, routed to one of the E real experts), the row of pair p is
// the number of exchanged pairs whose key is smaller. A workgroup that needs
// the rows of token t's K pairs reads every pair's expert id (N*K int32, in L2
// after the first workgroups), compares those keys with its K targets and sums
// the counts over the workgroup: a wavefront counts with one ballot per key and
// target (the population of the lane mask is the wavefront's count, so nothing
// is summed across lanes), and the workgroup adds its wavefronts' counts. The
// dispatch then needs no route launch and the combine no slot pass; at 8 ranks
// x 32 tokens, top-8, a dispatch thread compares 8 keys. The combine counts
// less: the first row of a pair's segment comes from ep_recv_count, so it only
// counts the same source rank's earlier pairs of the same expert.

constexpr int kFusedThreads = 256;        // one-launch dispatch: workgroup = (token, slice)
constexpr int kFusedUnroll = 2;           // 16-byte chunks per thread: a slice is 8 KiB
constexpr int kFusedMaxPairs = 4096;      // N*K up to which dispatch runs as one launch
constexpr int kFusedMaxCounts = 4096;     // W*E segment counts of its ep_recv_count workgroup (LDS)
constexpr int kFusedMaxK = 16;
constexpr int kFusedCombinePairs = 65535; // one-launch combine: N*K (the range its tests cover) ...
constexpr int kFusedCombineSrcPairs = 1024;   // ... and bs*K (pairs a workgroup may count)
constexpr int kFusedCombineLdsCounts = 2048;  // W*E up to which a workgroup stages ep_recv_count in LDS
static_assert(kFusedCombineLdsCounts == 16 * kGatherThreads, "the deepest staging loads 16 counts per thread");

// Expert ids and mask bytes of L pairs p[j], in two phases: pair_loads issues
// every load before any value is used, so that the L latencies overlap, and
// pair_experts then keeps the expert of each pair that is exchanged (below n,
// active, routed to one of the E real experts) and writes -1 for the others.
// MASKED (a token or pair mask) is a template parameter: without a mask no
// mask byte is loaded, and with one the loads are the same for both kinds,
// with no branch between them (a mask test between two id loads makes the
// compiler wait for the first before it issues the second, and loads on some
// paths only make it drain every load at the first wait). Pairs at or past n
// are read at n - 1 (at 0 if n is 0: the caller guarantees one pair).
template <int L, bool MASKED>
__device__ __forceinline__ void pair_loads(const int32_t *ids, const uint8_t *mask, int mask_kind, const int (&p)[L],
                                           int n, int K, float rK, int (&e)[L], int (&m)[L])
{
    const int last = n > 0 ? n - 1 : 0;
#pragma unroll
    for (int j = 0; j < L; ++j) e[j] = ids[min(p[j], last)];
    if constexpr (MASKED) {
#pragma unroll
        for (int j = 0; j < L; ++j) {
            const int q = min(p[j], last);
            m[j] = mask[mask_kind == MOE_MASK_TOKEN ? div_small(q, K, rK) : q];
        }
    }
}

template <int L, bool MASKED>
__device__ __forceinline__ void pair_experts(const int (&p)[L], int n, int E, int (&e)[L], const int (&m)[L])
{
#pragma unroll
    for (int j = 0; j < L; ++j)
        e[j] = p[j] < n && (!MASKED || m[j] != 0) && (unsigned)e[j] < (unsigned)E ? e[j] : -1;
}

// ep_recv_count workgroup of the one-launch dispatch: segment counts by LDS
// atomics over every exchanged pair, one exclusive scan over all W*E segments
// in (rank, el*W + s) order, and per rank that scan minus its value at the
// rank's first segment (a rank has S = E segments).
template <bool MASKED>
__device__ void fused_counts(const DispatchArgs &a)
{
    extern __shared__ int cnt[];                 // [W * E]
    __shared__ int tmp[40];
    const int G = a.W * a.E, NK = a.R, tid = threadIdx.x, nt = blockDim.x;
    const float rK = 1.0f / a.K, rbs = 1.0f / a.bs, repr = 1.0f / a.epr, rE = 1.0f / a.E;
    for (int i = tid; i < G; i += nt) cnt[i] = 0;
    __syncthreads();
    constexpr int CL = 8;                        // pairs per thread and pass, loads first
    for (int p0 = tid; p0 < NK; p0 += CL * nt) {
        int p[CL], e[CL], m[CL];
#pragma unroll
        for (int j = 0; j < CL; ++j) p[j] = p0 + j * nt;
        pair_loads<CL, MASKED>(a.ids, a.mask, a.mask_kind, p, NK, a.K, rK, e, m);
        pair_experts<CL, MASKED>(p, NK, a.E, e, m);
#pragma unroll
        for (int j = 0; j < CL; ++j) {
            if (e[j] < 0) continue;
            const int s = div_small(div_small(p[j], a.K, rK), a.bs, rbs);
            const int r = div_small(e[j], a.epr, repr);
            atomicAdd(&cnt[r * a.E + (e[j] - r * a.epr) * a.W + s], 1);
        }
    }
    __syncthreads();
    const int per = (G + nt - 1) / nt;
    const int g0 = min(tid * per, G), g1 = min(g0 + per, G);
    int sum = 0;
    for (int g = g0; g < g1; ++g) sum += cnt[g];
    int total;
    int run = block_excl_scan(sum, tmp, &total);
    for (int g = g0; g < g1; ++g) {
        run += cnt[g];
        cnt[g] = run;                            // inclusive prefix over all segments
    }
    __syncthreads();
    for (int g = tid; g < G; g += nt) {
        const int r = div_small(g, a.E, rE);
        a.erc[g] = cnt[g] - (r > 0 ? cnt[r * a.E - 1] : 0);
    }
}

// One-launch dispatch (copies): workgroups (token t, 8 KiB slice) plus one
// ep_recv_count workgroup at the end of the grid. Each thread issues the loads
// of L of the N*K expert ids (L * kFusedThreads >= N*K) and of token t's pair
// `lane` first, then those of its slice chunks, so that the count waits for the
// ids only; lane k of every wavefront holds the key of token t's pair k. After the count, every
// thread stores its chunks to the K rows; slice 0 writes assist_info and
// expand_scales. Needs rows in 16-byte pieces, K <= KT and N*K <= L * 256.
template <int KT, int L, bool MASKED>
__global__ __launch_bounds__(kFusedThreads) void dispatch_fused_kernel(DispatchArgs a)
{
    constexpr int NW = kFusedThreads / 64;
    __shared__ int red[NW * 64];
    const int N = a.W * a.bs, NK = a.R;
    if ((int)blockIdx.x >= N * a.nsl) {
        fused_counts<MASKED>(a);
        return;
    }
    const int tid = threadIdx.x, lane = tid & 63;
    const int t = blockIdx.x / a.nsl, sl = blockIdx.x - t * a.nsl;
    const float rK = 1.0f / a.K;
    const int nc = (int)(a.rowbytes / 16), c0 = sl * (kFusedThreads * kFusedUnroll) + tid;
    const uint4 *src = reinterpret_cast<const uint4 *>(a.x + (size_t)t * a.rowbytes);
    int p[L + 1], e[L + 1], m[L + 1];            // [L]: pair `lane` of token t
#pragma unroll
    for (int j = 0; j < L; ++j) p[j] = tid + j * kFusedThreads;
    p[L] = t * a.K + (lane < a.K ? lane : 0);
    pair_loads<L + 1, MASKED>(a.ids, a.mask, a.mask_kind, p, NK, a.K, rK, e, m);
    uint4 v[kFusedUnroll];
#pragma unroll
    for (int u = 0; u < kFusedUnroll; ++u) v[u] = src[min(c0 + u * kFusedThreads, nc - 1)];
    __builtin_amdgcn_sched_barrier(0);           // keep the slice loads above the waits for the ids
    pair_experts<L + 1, MASKED>(p, NK, a.E, e, m);
    int key[L];
#pragma unroll
    for (int j = 0; j < L; ++j) key[j] = e[j] >= 0 ? e[j] * NK + p[j] : INT_MAX;
    const int pt = p[L];
    const int tkey = lane < a.K && e[L] >= 0 ? e[L] * NK + pt : INT_MAX;
    // every thread is active here: the ballots see the whole wavefront. Lane k
    // keeps the wavefront's count for target k, selected as each is formed; every
    // lane writes its slot (only the first KT are read), since a write under a
    // lane test lets the compiler sink the counts into it and keep all L * KT lane
    // masks live until then.
    int mine = 0;
#pragma unroll
    for (int k = 0; k < KT; ++k) {
        const int tk = __builtin_amdgcn_readlane(tkey, k);
        int c = 0;
#pragma unroll
        for (int j = 0; j < L; ++j) c += __popcll(__builtin_amdgcn_ballot_w64(key[j] < tk));
        mine = lane == k ? c : mine;
    }
    red[tid] = mine;
    __syncthreads();
    int rows[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) {
        int row = 0;
#pragma unroll
        for (int q = 0; q < NW; ++q) row += red[q * 64 + k];
        const bool has = k < a.K && __builtin_amdgcn_readlane(tkey, k) != INT_MAX;
        rows[k] = has && row < a.R ? row : -1;
    }
    if (sl == 0 && tid < a.K) {
        int row = -1;
#pragma unroll
        for (int k = 0; k < KT; ++k)
            if (tid == k) row = rows[k];
        if (row >= 0) {
            const int s = t / a.bs;
            a.assist[(size_t)row * 3 + 0] = s;
            a.assist[(size_t)row * 3 + 1] = t - s * a.bs;
            a.assist[(size_t)row * 3 + 2] = tid;
            if (a.esc_out) a.esc_out[row] = a.esc_in[pt];
        }
    }
#pragma unroll
    for (int u = 0; u < kFusedUnroll; ++u) {
        const int c = c0 + u * kFusedThreads;
        if (c >= nc) continue;
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            if (rows[k] < 0) continue;
            store_stream(reinterpret_cast<uint4 *>(a.expand_x + (size_t)rows[k] * a.rowbytes) + c, v[u]);
        }
    }
}

// --------------------------------------------------------------------------
// combine
// --------------------------------------------------------------------------

struct CombineArgs {
    const char *expand_x;
    const int32_t *assist;
    const void *scales;
    const int32_t *slot;      // [N*K] row of pair (t, k), written by combine_slots_kernel
    int32_t *slot_out;
    char *x_out;
    const int32_t *erc;       // ep_recv_count [W, S]: with a mask, the row total comes from it
    const uint8_t *mask;
    const int32_t *ids;       // expert_ids [N, K]: special experts are recognised by id
    const char *ori_x;        // [N, h]: the tokens, for copy experts
    const char *const_x;      // [const experts, h]: the const experts' outputs
    int mask_kind;
    int pair_pass;            // a mask or special experts: mark pairs that have no row
    // special ids: [E, zero_end) zero, [zero_end, copy_end) copy, [copy_end, const_end) const
    int E, zero_end, copy_end, const_end;
    int W, bs, h, K, R, S, nsl, epr;
    long long rowbytes;
    int dev_from;             // gather: tokens from here on store x_out device-scope (see store_device)
};

// Return path (README 实现逻辑): row i of expand_x belongs to slot
// (src_token, topk_id) of source rank src_rank. Only its index travels.
// Under a token mask or with special experts only the first A rows exist (A =
// sum over ranks of the last inclusive count). A pair without a row gets slot
// -1 (inactive, or a zero expert: the gather skips it), -2 (a copy expert:
// the gather reads the token itself) or -3 - j (const expert j: the gather
// reads row j of the const table). A thread handles row i and pair i.
__global__ __launch_bounds__(kSlotThreads) void combine_slots_kernel(CombineArgs a)
{
    __shared__ int tmp[40];
    const int i = blockIdx.x * kSlotThreads + threadIdx.x;
    // Row i's assist_info entry, and in the pair pass pair i's id, its mask byte
    // and the first rank totals, are loaded first, unconditionally, at clamped
    // indices (R >= 1, W >= 1): none depends on another, and loads on some paths
    // only would make the compiler's first wait drain them all.
    const size_t ic = (size_t)min(i, a.R - 1);
    const int s = a.assist[ic * 3 + 0], tok = a.assist[ic * 3 + 1], k = a.assist[ic * 3 + 2];
    int rows = a.R;
    if (a.pair_pass) {
        const int e = a.ids[ic];
        const int tot0 = a.erc[(size_t)min((int)threadIdx.x, a.W - 1) * a.S + a.S - 1];
        const uint8_t *mp = a.mask_kind == MOE_MASK_TOKEN  ? a.mask + ic / a.K
                            : a.mask_kind == MOE_MASK_PAIR ? a.mask + ic
                                                           : reinterpret_cast<const uint8_t *>(a.ids + ic);
        const int mb = a.mask_kind == MOE_MASK_NONE ? 1 : *mp;
        int part = (int)threadIdx.x < a.W ? tot0 : 0;
        for (int r = threadIdx.x + kSlotThreads; r < a.W; r += kSlotThreads) part += a.erc[(size_t)r * a.S + a.S - 1];
        block_excl_scan(part, tmp, &rows);
        if (i < a.R) {
            if (mb == 0 || (e >= a.E && e < a.zero_end)) a.slot_out[i] = -1;
            else if (e >= a.zero_end && e < a.copy_end) a.slot_out[i] = kCopySlot;
            else if (e >= a.copy_end && e < a.const_end) a.slot_out[i] = kConstSlot0 - (e - a.copy_end);
        }
    }
    if (i >= rows || i >= a.R) return;
    if ((unsigned)s < (unsigned)a.W && (unsigned)tok < (unsigned)a.bs && (unsigned)k < (unsigned)a.K)
        a.slot_out[((size_t)s * a.bs + tok) * a.K + k] = i;
}

__device__ __forceinline__ void gather_prologue(const CombineArgs &a, int t, int *rows, uint32_t *sc)
{
    for (int k = threadIdx.x; k < a.K; k += blockDim.x) {
        const size_t p = (size_t)t * a.K + k;
        const int row = a.slot[p];
        // -2 (copy expert) and -3 - j (const expert j) are honoured only when this
        // call has such experts, so a stale or foreign slot never sends the gather
        // to a missing ori_x or past the const table
        const bool cst = row <= kConstSlot0 && a.const_x && kConstSlot0 - row < a.const_end - a.copy_end;
        rows[k] = (unsigned)row < (unsigned)a.R ? row : ((row == kCopySlot && a.ori_x) || cst ? row : -1);
        sc[k] = reinterpret_cast<const uint32_t *>(a.scales)[p];
    }
    __syncthreads();
}

// The row a slot names: an expand_x row, token t of ori_x (copy expert) or
// row j of the const table (const expert j).
__device__ __forceinline__ const char *slot_row(const CombineArgs &a, int t, int row)
{
    if (row >= 0) return a.expand_x + (size_t)row * a.rowbytes;
    if (row == kCopySlot) return a.ori_x + (size_t)t * a.rowbytes;
    return a.const_x + (size_t)(kConstSlot0 - row) * a.rowbytes;
}

// fp16 / bf16: block = (token, slice of kGatherThreads 16-byte chunks)
template <class T, bool VEC>
__global__ __launch_bounds__(kGatherThreads) void combine_gather_half_kernel(CombineArgs a)
{
    extern __shared__ int dsm[];
    int *rows = dsm;
    uint32_t *sc = reinterpret_cast<uint32_t *>(dsm + a.K);
    const int t = blockIdx.x / a.nsl, sl = blockIdx.x % a.nsl;
    gather_prologue(a, t, rows, sc);
    const int K = a.K;
    if (VEC) {
        const int nch = a.h / 8, c = sl * kGatherThreads + threadIdx.x;
        if (c >= nch) return;
        constexpr int KB = 8;
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
        for (int kb = 0; kb < K; kb += KB) {
            uint4 v[KB];
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) {
                const int k = kb + kk;
                const int row = k < K ? rows[k] : -1;
                v[kk] = row != -1 ? load_stream(reinterpret_cast<const uint4 *>(slot_row(a, t, row)) + c)
                                  : make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) {
                const int k = kb + kk;
                if (k < K && rows[k] != -1) {
                    const float wgt = __uint_as_float(sc[k]);
                    const uint32_t q[4] = {v[kk].x, v[kk].y, v[kk].z, v[kk].w};
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        acc[i] = __builtin_fmaf(T::load((uint16_t)(q[i >> 1] >> ((i & 1) * 16))), wgt, acc[i]);
                }
            }
        }
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (uint32_t)T::store(acc[2 * i]) | ((uint32_t)T::store(acc[2 * i + 1]) << 16);
        uint4 *dst = reinterpret_cast<uint4 *>(a.x_out + (size_t)t * a.rowbytes) + c;
        if (t >= a.dev_from) store_device(dst, make_uint4(o[0], o[1], o[2], o[3]));
        else store_stream(dst, make_uint4(o[0], o[1], o[2], o[3]));
    } else {
        const int j = sl * kGatherThreads + threadIdx.x;
        if (j >= a.h) return;
        float acc = 0.0f;
        for (int k = 0; k < K; ++k) {
            const int row = rows[k];
            if (row == -1) continue;
            const uint16_t y = reinterpret_cast<const uint16_t *>(slot_row(a, t, row))[j];
            acc = __builtin_fmaf(T::load(y), __uint_as_float(sc[k]), acc);
        }
        reinterpret_cast<uint16_t *>(a.x_out)[(size_t)t * a.h + j] = T::store(acc);
    }
}

// int32: wrapping 32-bit arithmetic, k ascending
template <bool VEC>
__global__ __launch_bounds__(kGatherThreads) void combine_gather_i32_kernel(CombineArgs a)
{
    extern __shared__ int dsm[];
    int *rows = dsm;
    uint32_t *sc = reinterpret_cast<uint32_t *>(dsm + a.K);
    const int t = blockIdx.x / a.nsl, sl = blockIdx.x % a.nsl;
    gather_prologue(a, t, rows, sc);
    const int K = a.K;
    if (VEC) {
        const int nch = a.h / 4, c = sl * kGatherThreads + threadIdx.x;
        if (c >= nch) return;
        uint32_t acc[4] = {0u, 0u, 0u, 0u};
        for (int k = 0; k < K; ++k) {
            const int row = rows[k];
            if (row == -1) continue;
            const uint4 v = reinterpret_cast<const uint4 *>(slot_row(a, t, row))[c];
            acc[0] += v.x * sc[k];
            acc[1] += v.y * sc[k];
            acc[2] += v.z * sc[k];
            acc[3] += v.w * sc[k];
        }
        reinterpret_cast<uint4 *>(a.x_out + (size_t)t * a.rowbytes)[c] = make_uint4(acc[0], acc[1], acc[2], acc[3]);
    } else {
        const int j = sl * kGatherThreads + threadIdx.x;
        if (j >= a.h) return;
        uint32_t acc = 0u;
        for (int k = 0; k < K; ++k) {
            const int row = rows[k];
            if (row == -1) continue;
            acc += reinterpret_cast<const uint32_t *>(slot_row(a, t, row))[j] * sc[k];
        }
        reinterpret_cast<uint32_t *>(a.x_out)[(size_t)t * a.h + j] = acc;
    }
}


// One-launch combine: workgroup = (token t, slice of kGatherThreads 16-byte
// chunks), with the gather and the fp32 weighted sum of the gather kernels
// above. The slot of token t's pair k is found in the workgroup (lane k of
// every wavefront holds it): a real expert's row is the first row of its
// segment, from ep_recv_count (the rows of all lower ranks, plus the rank's
// inclusive count before segment (el, s)), plus the pairs of source rank s's
// earlier tokens routed to the same expert, counted over those tokens' ids. A
// copy expert reads token t, const expert j row j of the const table. With
// PS > 0 the workgroup stages ep_recv_count in LDS, PS values per thread
// (W*E <= PS * kGatherThreads), so that the segment start needs no second
// dependent load; PS is 4 or 16 so that small tables do not pay for 16 loads
// per thread. Needs rows in 16-byte pieces, K <= KT and N*K < 2^16.
template <class T, int KT, int PS, bool MASKED>
__global__ __launch_bounds__(kGatherThreads) void combine_fused_kernel(CombineArgs a)
{
    constexpr bool PRE = PS > 0;
    constexpr int NW = kGatherThreads / 64;
    extern __shared__ int erc_lds[];              // PRE: ep_recv_count [W * S]
    __shared__ int red[kGatherThreads];
    const int tid = threadIdx.x, lane = tid & 63;
    const int t = blockIdx.x / a.nsl, sl = blockIdx.x - t * a.nsl;
    const int K = a.K;
    const int s = t / a.bs;
    const float rK = 1.0f / K;
    // Every load of the prologue that depends on no other is issued first, in
    // this order, and only then is any value used, so that their latencies
    // overlap: lane k's pair k of token t (id, weight, mask byte), the first 64
    // rank totals, the first SB source pairs of each thread, and (PRE) the
    // ep_recv_count values the thread stages. These loads are issued whatever
    // the sizes, at clamped indices, and the values not needed are ignored: a
    // load under a condition makes the compiler's waits assume the path
    // without it, and the first wait would then drain every load.
    const int pt = t * K + (lane < K ? lane : 0);
    const int e = a.ids[pt];
    const uint32_t wbits = reinterpret_cast<const uint32_t *>(a.scales)[pt];
    const int mb = MASKED ? a.mask[a.mask_kind == MOE_MASK_TOKEN ? (size_t)t : (size_t)pt] : 1;
    const int tot0 = a.erc[(size_t)min(lane, a.W - 1) * a.S + a.S - 1];
    constexpr int SB = 4;                          // source pairs per thread and pass
    const int p1 = t * K;                          // token t's first pair
    int sp[SB], se[SB], sm[SB];
#pragma unroll
    for (int u = 0; u < SB; ++u) sp[u] = s * a.bs * K + tid + u * kGatherThreads;
    pair_loads<SB, MASKED>(a.ids, a.mask, a.mask_kind, sp, p1, K, rK, se, sm);
    const int WS = a.W * a.S;
    int ercv[PRE ? PS : 1];
    if (PRE) {
#pragma unroll
        for (int u = 0; u < PS; ++u) ercv[u] = a.erc[min(tid + u * kGatherThreads, WS - 1)];
    }
    const bool on = lane < K && mb != 0;
    const bool real = on && (unsigned)e < (unsigned)a.E;
    const int r = real ? div_small(e, a.epr, 1.0f / a.epr) : -1;
    const int seg = real ? (e - r * a.epr) * a.W + s : 0;     // segment (el, s) inside rank r
    int base = 0;
    if (!PRE && real && seg > 0) base = a.erc[(size_t)r * a.S + seg - 1];
    const int ek = real ? e : INT_MIN;             // an inactive pair below reads as -1, never INT_MIN
    // Every lane's values that other lanes need are read here, with the whole
    // wavefront active: a lane that is switched off inside the loops below may
    // not hold them there.
    int ek_u[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) ek_u[k] = __builtin_amdgcn_readlane(ek, k);
    // Rows of the ranks below lane k's rank r: every wavefront scans the W rank
    // totals, 64 at a time (the first 64 loaded above), and lane k reads the
    // prefix before r from the scan (ds_bpermute). Loop bounds are uniform.
    int below = 0;
    for (int q0 = 0; q0 < a.W; q0 += 64) {
        const int q = q0 + lane;
        const int tot = q0 == 0 ? (lane < a.W ? tot0 : 0)
                                : (q < a.W ? a.erc[(size_t)q * a.S + a.S - 1] : 0);
        const int sc = wave_incl_scan(tot);
        const int n = min(r - q0, 64);           // ranks of this chunk below r (r = -1: none)
        const int got = __builtin_amdgcn_ds_bpermute(max(n - 1, 0) << 2, sc);
        below += n > 0 ? got : 0;
    }
    // Pairs of source rank s's earlier tokens routed to the same expert: every
    // wavefront counts its share with one ballot per pair slot and target, lane
    // k keeps target k's count, and the workgroup adds its wavefronts' counts.
    // The loop is uniform, so the ballots see every lane.
    int mine = 0;
    const int pfirst = s * a.bs * K;
    for (int pb = pfirst; pb < p1; pb += SB * kGatherThreads) {
        if (pb != pfirst) {                       // the first pass's loads were issued above
#pragma unroll
            for (int u = 0; u < SB; ++u) sp[u] = pb + tid + u * kGatherThreads;
            pair_loads<SB, MASKED>(a.ids, a.mask, a.mask_kind, sp, p1, K, rK, se, sm);
        }
        pair_experts<SB, MASKED>(sp, p1, a.E, se, sm);
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            int c = 0;
#pragma unroll
            for (int u = 0; u < SB; ++u) c += __popcll(__builtin_amdgcn_ballot_w64(se[u] == ek_u[k]));
            mine += lane == k ? c : 0;
        }
    }
    if (PRE) {
#pragma unroll
        for (int u = 0; u < PS; ++u) {
            const int i = tid + u * kGatherThreads;
            if (i < WS) erc_lds[i] = ercv[u];
        }
    }
    red[tid] = mine;                              // every lane (only the first KT are read): see dispatch_fused_kernel
    __syncthreads();                              // (also publishes erc_lds)
    if (PRE && real && seg > 0) base = erc_lds[r * a.S + seg - 1];
    int cnt = below;
#pragma unroll
    for (int q = 0; q < NW; ++q) cnt += red[q * 64 + lane];
    // the slot of lane k's pair: a row, kCopySlot, kConstSlot0 - j, or -1 (nothing to add)
    int slot = -1;
    if (real) {
        slot = cnt + base;
        if ((unsigned)slot >= (unsigned)a.R) slot = -1;
    } else if (on && e >= a.zero_end && e < a.copy_end && a.ori_x) {
        slot = kCopySlot;
    } else if (on && e >= a.copy_end && e < a.const_end && a.const_x) {
        slot = kConstSlot0 - (e - a.copy_end);
    }
    int slot_u[KT];
    uint32_t w_u[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) {
        slot_u[k] = k < K ? __builtin_amdgcn_readlane(slot, k) : -1;
        w_u[k] = __builtin_amdgcn_readlane(wbits, k);
    }
    constexpr bool I32 = std::is_same<T, int32_t>::value;
    const int nch = I32 ? a.h / 4 : a.h / 8, c = sl * kGatherThreads + tid;
    if (c >= nch) return;
    constexpr int KB = 8;
    float acc[8];
    uint32_t iacc[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) iacc[i] = 0u;
#pragma unroll
    for (int kb = 0; kb < KT; kb += KB) {
        if (kb >= K) break;
        uint4 v[KB];
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
            const int k = kb + kk;
            v[kk] = slot_u[k] != -1 ? load_stream(reinterpret_cast<const uint4 *>(slot_row(a, t, slot_u[k])) + c)
                                    : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
            const int k = kb + kk;
            if (slot_u[k] == -1) continue;
            const uint32_t wk = w_u[k];
            const uint32_t q[4] = {v[kk].x, v[kk].y, v[kk].z, v[kk].w};
            if constexpr (I32) {
#pragma unroll
                for (int i = 0; i < 4; ++i) iacc[i] += q[i] * wk;
            } else {
                const float wgt = __uint_as_float(wk);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    acc[i] = __builtin_fmaf(T::load((uint16_t)(q[i >> 1] >> ((i & 1) * 16))), wgt, acc[i]);
            }
        }
    }
    uint4 out;
    if constexpr (I32) {
        out = make_uint4(iacc[0], iacc[1], iacc[2], iacc[3]);
    } else {
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (uint32_t)T::store(acc[2 * i]) | ((uint32_t)T::store(acc[2 * i + 1]) << 16);
        out = make_uint4(o[0], o[1], o[2], o[3]);
    }
    store_stream(reinterpret_cast<uint4 *>(a.x_out + (size_t)t * a.rowbytes) + c, out);
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
    // every (token, slice) grid below has at most N * ceil(h / 128) blocks of <= 128 threads,
    // and a launch must stay below 2^32 work-items
    if (N * (((long long)h + 127) / 128) >= (1ll << 25)) return MOE_ERR_SHAPE;
    return MOE_OK;
}

// Special experts: counts >= 0, every id below 2^31.
int check_special(const moe_special_experts *sp, long long E)
{
    if (!sp) return MOE_OK;
    if (sp->zero_expert_num < 0 || sp->copy_expert_num < 0 || sp->const_expert_num < 0) return MOE_ERR_SHAPE;
    if (E + sp->zero_expert_num + sp->copy_expert_num + (long long)sp->const_expert_num >= (1ll << 31))
        return MOE_ERR_SHAPE;
    return MOE_OK;
}

struct DispatchLayout {
    int nbs, NB;
    size_t pc, pci, boff, lr, plan, nplan, total;
};

DispatchLayout dispatch_layout(int W, int bs, int epr, int K)
{
    DispatchLayout L;
    const size_t E = (size_t)W * epr, N = (size_t)W * bs, S = (size_t)epr * W;
    L.nbs = (bs + kRouteTokens - 1) / kRouteTokens;
    L.NB = W * L.nbs;
    // plan items of the segment schedule; the adaptive schedule keeps its per-row flags (N * K bytes) there
    const size_t plan_cap = N * K / kPlanRows + 2 * (size_t)W * S + W + 1;
    static_assert(kPlanRows == 8, "the plan region holds one byte per row");
    size_t off = 0;
    L.pc = off;    off = round_up(off + (size_t)L.NB * E * 4, 256);
    L.pci = off;   off = round_up(off + (size_t)L.NB * E * 4, 256);
    L.boff = off;  off = round_up(off + (size_t)L.NB * E * 4, 256);
    L.lr = off;    off = round_up(off + N * K * 4, 256);
    L.plan = off;  off = round_up(off + plan_cap * 8, 256);
    L.nplan = off; off = round_up(off + 4, 256);
    L.total = off;
    return L;
}

template <bool SKIP>
void launch_copy_wave(int J, dim3 g, dim3 b, hipStream_t st, const DispatchArgs &a)
{
    if (J <= 1) hipLaunchKernelGGL((scatter_copy_wave_kernel<1, SKIP>), g, b, 0, st, a);
    else if (J <= 2) hipLaunchKernelGGL((scatter_copy_wave_kernel<2, SKIP>), g, b, 0, st, a);
    else if (J <= 4) hipLaunchKernelGGL((scatter_copy_wave_kernel<4, SKIP>), g, b, 0, st, a);
    else if (J <= 8) hipLaunchKernelGGL((scatter_copy_wave_kernel<8, SKIP>), g, b, 0, st, a);
    else if (J <= 14) hipLaunchKernelGGL((scatter_copy_wave_kernel<14, SKIP>), g, b, 0, st, a);
    else hipLaunchKernelGGL((scatter_copy_wave_kernel<16, SKIP>), g, b, 0, st, a);
}

template <class T, int QM, bool SKIP = false>
void launch_quant_wave(int J, dim3 g, dim3 b, hipStream_t st, const DispatchArgs &a)
{
    if (J <= 1) hipLaunchKernelGGL((scatter_quant_wave_kernel<T, 1, QM, SKIP>), g, b, 0, st, a);
    else if (J <= 2) hipLaunchKernelGGL((scatter_quant_wave_kernel<T, 2, QM, SKIP>), g, b, 0, st, a);
    else if (J <= 4) hipLaunchKernelGGL((scatter_quant_wave_kernel<T, 4, QM, SKIP>), g, b, 0, st, a);
    else if (J <= 7) hipLaunchKernelGGL((scatter_quant_wave_kernel<T, 7, QM, SKIP>), g, b, 0, st, a);
    else if (J <= 8) hipLaunchKernelGGL((scatter_quant_wave_kernel<T, 8, QM, SKIP>), g, b, 0, st, a);
    else if (J <= 12) hipLaunchKernelGGL((scatter_quant_wave_kernel<T, 12, QM, SKIP>), g, b, 0, st, a);
    else hipLaunchKernelGGL((scatter_quant_wave_kernel<T, 16, QM, SKIP>), g, b, 0, st, a);
}

// ---- scratch of the allocation-free dispatch (moe_dispatch_noalloc) ----
// One file-scope device array: every GPU the library runs on holds its own
// copy, at its own address, until the process ends. Host code must not use
// the array's name as a device address (on the host it names a stand-in): the
// address is looked up per device with hipGetSymbolAddress and kept here.
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];             // device address of `scratch` per device, once looked up

// The scratch's device address on the current device (looked up on the first
// call there, with that device current), or nullptr when the lookup fails.
void *scratch_on_current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
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
    case MOE_ERR_QUANT:
        return "unknown quant mode, quantisation of int32 data, or a shape or coefficient count the quantiser "
               "does not take";
    case MOE_ERR_WORKSPACE: return "workspace smaller than the queried size";
    case MOE_ERR_LAUNCH: return "the HIP runtime refused a kernel launch";
    case MOE_ERR_SCHEDULE: return "unknown schedule mode, or segment schedule too large for this shape";
    case MOE_ERR_ALIGN: return "a pointer is not aligned to its element size";
    case MOE_ERR_MASK: return "unknown mask kind, or the mask pointer does not match it";
    default: return "unknown status";
    }
}

int moe_dispatch_workspace_size(int ep_world, int bs, int experts_per_rank, int h, int topk, int dtype,
                                int quant_mode, size_t *bytes)
{
    if (!bytes) return MOE_ERR_NULLPTR;
    int rc = check_scalars(ep_world, bs, experts_per_rank, h, topk, dtype);
    if (rc) return rc;
    if (quant_mode < MOE_QUANT_NONE || quant_mode > MOE_QUANT_MX) return MOE_ERR_QUANT;
    if (quant_mode != MOE_QUANT_NONE && dtype == MOE_INT32) return MOE_ERR_QUANT;
    // the static, per-group and MX quantisers are the wavefront-per-token kernel only
    if ((quant_mode == MOE_QUANT_STATIC || quant_mode == MOE_QUANT_DYN_GROUP || quant_mode == MOE_QUANT_MX) &&
        (h % 16 != 0 || h > kQuantMaxH || topk > kQuantMaxK))
        return MOE_ERR_QUANT;
    *bytes = dispatch_layout(ep_world, bs, experts_per_rank, topk).total;
    return MOE_OK;
}

int moe_dispatch(const void *x, const int32_t *expert_ids, const void *expert_scales,
                 const uint8_t *x_active_mask, int mask_kind, const moe_special_experts *special,
                 int ep_world, int bs, int experts_per_rank, int h, int topk, int dtype, int quant_mode,
                 const float *quant_scales, int64_t quant_scales_numel, void *expand_x, void *dynamic_scales,
                 int32_t *assist_info, int32_t *ep_recv_count, void *expand_scales,
                 const moe_schedule *schedule, void *workspace, size_t workspace_bytes, void *stream)
{
    size_t need = 0;
    int rc = moe_dispatch_workspace_size(ep_world, bs, experts_per_rank, h, topk, dtype, quant_mode, &need);
    if (rc) return rc;
    const int W = ep_world, epr = experts_per_rank, K = topk;
    const long long N = (long long)W * bs;
    const bool quant = quant_mode != MOE_QUANT_NONE;
    const bool group_quant = quant_mode == MOE_QUANT_DYN_GROUP;
    const bool static_quant = quant_mode == MOE_QUANT_STATIC;
    const bool mx_quant = quant_mode == MOE_QUANT_MX;
    const bool dyn_quant = quant && !static_quant;       // writes dynamic_scales
    if (!ep_recv_count || !workspace) return MOE_ERR_NULLPTR;
    if (N > 0 && (!x || !expert_ids || !expand_x || !assist_info)) return MOE_ERR_NULLPTR;
    if (dyn_quant != (dynamic_scales != nullptr) && N > 0) return MOE_ERR_NULLPTR;
    if (!dyn_quant && dynamic_scales) return MOE_ERR_NULLPTR;
    const long long E_ = (long long)W * epr;
    int qkind = kStaticOne;
    if (static_quant) {
        if (!quant_scales && N > 0) return MOE_ERR_NULLPTR;
        if (quant_scales_numel == 1) qkind = kStaticOne;
        else if (quant_scales_numel == h) qkind = kStaticColumn;
        else if (quant_scales_numel == E_ * h) qkind = kStaticExpert;
        else return MOE_ERR_QUANT;
    } else if (quant_scales || quant_scales_numel != 0) {
        return MOE_ERR_NULLPTR;
    }
    if (expand_scales && !expert_scales) return MOE_ERR_NULLPTR;
    if (mask_kind < MOE_MASK_NONE || mask_kind > MOE_MASK_PAIR) return MOE_ERR_MASK;
    if ((mask_kind != MOE_MASK_NONE) != (x_active_mask != nullptr) && N > 0) return MOE_ERR_MASK;
    if (mask_kind == MOE_MASK_NONE && x_active_mask) return MOE_ERR_MASK;
    // special experts: their ids are legal and, like any id past the E real
    // experts, routed nowhere by the kernels
    if ((rc = check_special(special, (long long)W * epr))) return rc;
    if (workspace_bytes < need) return MOE_ERR_WORKSPACE;

    const int mode = schedule ? schedule->mode : MOE_SCHED_ADAPTIVE;
    long long large = schedule ? schedule->large_segment_bytes : -1;
    if (large < 0) large = kReadmeLargeBytes;
    int32_t *seg_flags = schedule ? schedule->segment_is_large : nullptr;
    if (mode != MOE_SCHED_TOKEN && mode != MOE_SCHED_SEGMENT && mode != MOE_SCHED_ADAPTIVE) return MOE_ERR_SCHEDULE;
    const long long S = (long long)epr * W;
    const size_t xs = elem_size(dtype);
    const int elem_out = quant ? 1 : (int)xs;
    // The adaptive schedule runs its large-segment pass only where a segment
    // can be large: a segment holds at most bs rows (ids are distinct per
    // token), so bs * h * elem_out < T rules every segment out.
    const bool adaptive = mode == MOE_SCHED_ADAPTIVE && N > 0 && (!quant || quant_mode == MOE_QUANT_DYN_TOKEN) &&
                          (long long)bs * h * elem_out >= large;
    const bool want_seg = mode == MOE_SCHED_SEGMENT || seg_flags;
    if (want_seg && (long long)W * S > kSegLdsMax) return MOE_ERR_SCHEDULE;
    if ((group_quant || static_quant || mx_quant) && mode == MOE_SCHED_SEGMENT) return MOE_ERR_SCHEDULE;

    const size_t rowbytes = (size_t)h * xs;
    if (!aligned(x, xs) || !aligned(expert_ids, 4) || !aligned(expert_scales, 4) ||
        !aligned(expand_x, quant ? 1 : xs) || !aligned(dynamic_scales, mx_quant ? 1 : 4) || !aligned(assist_info, 4) ||
        !aligned(ep_recv_count, 4) || !aligned(expand_scales, 4) || !aligned(workspace, 16) ||
        !aligned(seg_flags, 4) || !aligned(quant_scales, qkind == kStaticOne ? 4 : 16))
        return MOE_ERR_ALIGN;
    // per-token int8 takes the wavefront kernel when it can, a block kernel
    // otherwise; per-group FP8 and MX need the wavefront kernel's 16-byte rows
    const bool wave = quant && h % 16 == 0 && h <= kQuantMaxH && K <= kQuantMaxK && aligned(x, 16) &&
                      aligned(expand_x, 16);
    if ((group_quant || static_quant || mx_quant) && !wave && N > 0) return MOE_ERR_ALIGN;

    const DispatchLayout L = dispatch_layout(W, bs, epr, K);
    char *ws = static_cast<char *>(workspace);
    int32_t *pc = reinterpret_cast<int32_t *>(ws + L.pc);
    int32_t *pci = reinterpret_cast<int32_t *>(ws + L.pci);
    int32_t *boff = reinterpret_cast<int32_t *>(ws + L.boff);
    int32_t *lr = reinterpret_cast<int32_t *>(ws + L.lr);
    int2 *plan = reinterpret_cast<int2 *>(ws + L.plan);
    int32_t *nplan = reinterpret_cast<int32_t *>(ws + L.nplan);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int E = W * epr;
    // blocks sum the chunk prefixes themselves unless there are many chunks (or a
    // plan is needed); otherwise one scan block forms every offset first
    const bool direct = N > 0 && mode != MOE_SCHED_SEGMENT && L.NB <= kDirectMaxChunks;

    DispatchArgs a;
    a.x = static_cast<const char *>(x);
    a.ids = expert_ids;
    a.esc_in = static_cast<const int32_t *>(expert_scales);
    a.expand_x = static_cast<char *>(expand_x);
    a.dyn = static_cast<float *>(dynamic_scales);     // uint8 scale bytes for MX
    a.assist = assist_info;
    a.esc_out = static_cast<int32_t *>(expand_scales);
    a.erc = ep_recv_count;
    a.lr = lr;
    a.pc = pc;
    a.pci = pci;
    a.boff = boff;
    a.plan = plan;
    a.nplan = nplan;
    a.lflag = adaptive ? reinterpret_cast<uint8_t *>(ws + L.plan) : nullptr;   // the segment plan's region
    a.large = large;
    a.out_row_bytes = (long long)h * elem_out;
    a.den = (long long)(W - 1 > 1 ? W - 1 : 1) * epr;
    a.W = W; a.bs = bs; a.epr = epr; a.h = h; a.K = K; a.nbs = L.nbs; a.R = (int)(N * K);
    a.E = E; a.S = (int)S; a.NB = L.NB;
    // with a scan block present it also wrote ep_recv_count
    a.direct = (direct && !want_seg) ? 1 : 0;
    a.rowbytes = (long long)rowbytes;
    a.nsl = 1;
    a.qs = quant_scales;
    a.qkind = qkind;
    a.mask = x_active_mask;
    a.mask_kind = mask_kind;
    // the plain share of the quantisers' stores shrinks as the rows written
    // outgrow the Infinity Cache; the wavefront copy keeps half of its
    // stores plain up to its own limit (see store_stream)
    const long long qbytes = N * K * (long long)h;
    a.store_mix = !quant || qbytes <= kMixedStoreMaxBytes ? 0 : (qbytes <= kQuarterPlainMaxBytes ? 1 : 2);

    (void)hipGetLastError();
    // Small batches of copies: one launch (rows by counting, see dispatch_fused_kernel)
    const bool vec16 = rowbytes % 16 == 0 && aligned(x, 16) && aligned(expand_x, 16);
    if (N > 0 && !quant && mode != MOE_SCHED_SEGMENT && !adaptive && !want_seg && vec16 && K <= kFusedMaxK &&
        N * K <= kFusedMaxPairs && (long long)W * E <= kFusedMaxCounts) {
        const int sc = kFusedThreads * kFusedUnroll;
        a.nsl = (int)(((long long)rowbytes / 16 + sc - 1) / sc);
        const dim3 g((unsigned)(N * a.nsl + 1)), b(kFusedThreads);
        const size_t lds = (size_t)W * E * sizeof(int);
        const bool k8 = K <= 8, l8 = N * K <= 8 * kFusedThreads;
#define MOE_FUSED_DISPATCH(M)                                                                       \
        do {                                                                                        \
            if (k8 && l8) hipLaunchKernelGGL((dispatch_fused_kernel<8, 8, M>), g, b, lds, st, a);           \
            else if (k8) hipLaunchKernelGGL((dispatch_fused_kernel<8, 16, M>), g, b, lds, st, a);          \
            else if (l8) hipLaunchKernelGGL((dispatch_fused_kernel<16, 8, M>), g, b, lds, st, a);          \
            else hipLaunchKernelGGL((dispatch_fused_kernel<16, 16, M>), g, b, lds, st, a);                 \
        } while (0)
        if (a.mask_kind == MOE_MASK_NONE) MOE_FUSED_DISPATCH(false);
        else MOE_FUSED_DISPATCH(true);
#undef MOE_FUSED_DISPATCH
        return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
    }

    if (N > 0) {
        const dim3 g(L.NB), b(kRouteThreads);
        const size_t lds = (size_t)E * kRouteWords * 8;
        if (mask_kind == MOE_MASK_TOKEN)
            hipLaunchKernelGGL(route_kernel<MOE_MASK_TOKEN>, g, b, lds, st, expert_ids, W, bs, epr, K, L.nbs,
                               x_active_mask, pc, pci, lr);
        else if (mask_kind == MOE_MASK_PAIR)
            hipLaunchKernelGGL(route_kernel<MOE_MASK_PAIR>, g, b, lds, st, expert_ids, W, bs, epr, K, L.nbs,
                               x_active_mask, pc, pci, lr);
        else
            hipLaunchKernelGGL(route_kernel<MOE_MASK_NONE>, g, b, lds, st, expert_ids, W, bs, epr, K, L.nbs,
                               x_active_mask, pc, pci, lr);
    }
    if (!direct || want_seg)
        hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), want_seg ? (size_t)W * S * 5 : 0, st, pc, pci,
                           W, epr, L.nbs, h, elem_out, boff, ep_recv_count, want_seg ? 1 : 0, large, seg_flags,
                           (mode == MOE_SCHED_SEGMENT && N > 0) ? plan : nullptr, nplan);
    // the payload pass over a plan's items (segment-major, or the adaptive schedule's large segments)
    auto segment_payload = [&](unsigned blocks) {
        const int qm = !quant ? 0 : (dtype == MOE_FP16 ? 1 : 2);
        const bool vec = quant ? (h % 8 == 0 && aligned(x, 16) && aligned(expand_x, 8))
                               : (rowbytes % 16 == 0 && aligned(x, 16) && aligned(expand_x, 16));
        const int Jc = (int)((rowbytes / 16 + 63) / 64), Jq = (h / 16 + 63) / 64;
        const dim3 g(blocks), b(kBlockThreads), bw(kQuantThreads);
        if (qm == 0 && vec && Jc <= 16) {
            launch_segment_copy_wave(Jc, g, bw, st, a);
        } else if (qm != 0 && wave) {
            if (qm == 1) launch_segment_quant_wave<F16>(Jq, g, bw, st, a);
            else launch_segment_quant_wave<BF16>(Jq, g, bw, st, a);
        } else if (qm == 0) {
            if (vec) hipLaunchKernelGGL((segment_payload_kernel<0, true>), g, b, 0, st, a);
            else hipLaunchKernelGGL((segment_payload_kernel<0, false>), g, b, 0, st, a);
        } else if (qm == 1) {
            if (vec) hipLaunchKernelGGL((segment_payload_kernel<1, true>), g, b, 0, st, a);
            else hipLaunchKernelGGL((segment_payload_kernel<1, false>), g, b, 0, st, a);
        } else {
            if (vec) hipLaunchKernelGGL((segment_payload_kernel<2, true>), g, b, 0, st, a);
            else hipLaunchKernelGGL((segment_payload_kernel<2, false>), g, b, 0, st, a);
        }
    };
    // the adaptive schedule's pass over the rows the token-major kernels left out
    auto large_payload = [&]() {
        const int qm = !quant ? 0 : (dtype == MOE_FP16 ? 1 : 2);
        const bool vec = quant ? (h % 8 == 0 && aligned(x, 16) && aligned(expand_x, 8))
                               : (rowbytes % 16 == 0 && aligned(x, 16) && aligned(expand_x, 16));
        const int Jc = (int)((rowbytes / 16 + 63) / 64), Jq = (h / 16 + 63) / 64;
        const long long windows = (N * K + kPlanRows - 1) / kPlanRows;
        const dim3 gw((unsigned)std::min<long long>(kAdaptiveSegGrid, (windows + 3) / 4)), bw(kQuantThreads);
        const dim3 g((unsigned)std::min<long long>(kAdaptiveSegGrid, windows)), b(kBlockThreads);
        if (qm == 0 && vec && Jc <= 16) {
            launch_large_copy_wave(Jc, gw, bw, st, a);
        } else if (qm != 0 && wave) {
            if (qm == 1) launch_large_quant_wave<F16>(Jq, gw, bw, st, a);
            else launch_large_quant_wave<BF16>(Jq, gw, bw, st, a);
        } else if (qm == 0) {
            if (vec) hipLaunchKernelGGL((large_payload_block_kernel<0, true>), g, b, 0, st, a);
            else hipLaunchKernelGGL((large_payload_block_kernel<0, false>), g, b, 0, st, a);
        } else if (qm == 1) {
            if (vec) hipLaunchKernelGGL((large_payload_block_kernel<1, true>), g, b, 0, st, a);
            else hipLaunchKernelGGL((large_payload_block_kernel<1, false>), g, b, 0, st, a);
        } else {
            if (vec) hipLaunchKernelGGL((large_payload_block_kernel<2, true>), g, b, 0, st, a);
            else hipLaunchKernelGGL((large_payload_block_kernel<2, false>), g, b, 0, st, a);
        }
    };
    if (N > 0) {
        if (mode != MOE_SCHED_SEGMENT) {
            const size_t kdsm = (size_t)4 * K * sizeof(int);
            if (!quant) {
                const bool vec = rowbytes % 16 == 0 && aligned(x, 16) && aligned(expand_x, 16);
                const long long n = vec ? (long long)(rowbytes / 16) : (long long)(rowbytes / 2);
                const int sc = kCopyThreads * kCopyUnroll;
                const int Jc = (int)((n + 63) / 64);
                // Many tokens: one wavefront per token with mixed stores (a 529 MB bf16
                // copy at 16 ranks x 256 tokens: 84 us against 106 us for the slice
                // blocks). Few tokens: slice blocks, which keep more CUs busy (256
                // tokens at h = 7168: 11 us against 20 us). Past about 650 MB of rows
                // the slice blocks win again (16 x 1024 tokens: 378 us against 444 us).
                if (vec && K <= kQuantMaxK && Jc <= 16 && N >= kCopyWaveMinTokens &&
                    (long long)N * K * (long long)rowbytes <= kCopyWaveMaxBytes) {
                    const dim3 g((unsigned)((N + 3) / 4)), b(kQuantThreads);
                    if (adaptive) launch_copy_wave<true>(Jc, g, b, st, a);
                    else launch_copy_wave<false>(Jc, g, b, st, a);
                } else {
                    a.nsl = (int)((n + sc - 1) / sc);
                    const dim3 g((unsigned)(N * a.nsl)), b(kCopyThreads);
                    if (adaptive) {
                        if (vec) hipLaunchKernelGGL((scatter_copy_kernel<true, true>), g, b, kdsm, st, a);
                        else hipLaunchKernelGGL((scatter_copy_kernel<false, true>), g, b, kdsm, st, a);
                    } else {
                        if (vec) hipLaunchKernelGGL((scatter_copy_kernel<true, false>), g, b, kdsm, st, a);
                        else hipLaunchKernelGGL((scatter_copy_kernel<false, false>), g, b, kdsm, st, a);
                    }
                }
            } else {
                if (wave) {
                    const int J = (h / 16 + 63) / 64;
                    const dim3 g((unsigned)((N + 3) / 4)), b(kQuantThreads);
                    if (static_quant && qkind == kStaticExpert) {
                        hipLaunchKernelGGL(dispatch_meta_kernel, g, b, 0, st, a);
                        // source ranks per group: the tokens whose column slices fill kStaticGroupBytes
                        const long long slice = std::max<long long>(1, (long long)rowbytes / kXcds);
                        const long long gtok = std::max<long long>(1, kStaticGroupBytes / slice);
                        const int spg = (int)std::max<long long>(1, std::min<long long>(W, gtok / std::max(bs, 1)));
                        const int ngrp = (W + spg - 1) / spg;
                        const long long rows_per = std::max<long long>(1, N * K / ((long long)E * ngrp));
                        // parts: workgroups per (slice, expert, group); any count >= 1 covers the rows.
                        // Capped so that the grid stays below 2^32 work-items (8 * E * ngrp < 2^24 always
                        // holds: E <= 1024, ngrp <= W <= 768), which matters past ~6.7e7 pairs.
                        const long long max_parts = ((1ll << 32) / kQuantThreads - 1) / ((long long)kXcds * E * ngrp);
                        const int parts = (int)std::max<long long>(
                            1, std::min<long long>({64, std::max<long long>(1, rows_per / 32), max_parts}));
                        const dim3 gx((unsigned)((long long)kXcds * E * parts * ngrp));
                        const bool two = h > 1024 * kXcds;     // two 16-element pieces per lane
                        if (dtype == MOE_FP16) {
                            if (two) hipLaunchKernelGGL((scatter_static_group_kernel<F16, 2>), gx, b, 0, st, a, spg, parts);
                            else hipLaunchKernelGGL((scatter_static_group_kernel<F16, 1>), gx, b, 0, st, a, spg, parts);
                        } else {
                            if (two) hipLaunchKernelGGL((scatter_static_group_kernel<BF16, 2>), gx, b, 0, st, a, spg, parts);
                            else hipLaunchKernelGGL((scatter_static_group_kernel<BF16, 1>), gx, b, 0, st, a, spg, parts);
                        }
                    } else if (dtype == MOE_FP16) {
                        if (group_quant) launch_quant_wave<F16, MOE_QUANT_DYN_GROUP>(J, g, b, st, a);
                        else if (mx_quant) launch_quant_wave<F16, MOE_QUANT_MX>(J, g, b, st, a);
                        else if (static_quant) launch_quant_wave<F16, MOE_QUANT_STATIC>(J, g, b, st, a);
                        else if (adaptive) launch_quant_wave<F16, MOE_QUANT_DYN_TOKEN, true>(J, g, b, st, a);
                        else launch_quant_wave<F16, MOE_QUANT_DYN_TOKEN>(J, g, b, st, a);
                    } else {
                        if (group_quant) launch_quant_wave<BF16, MOE_QUANT_DYN_GROUP>(J, g, b, st, a);
                        else if (mx_quant) launch_quant_wave<BF16, MOE_QUANT_MX>(J, g, b, st, a);
                        else if (static_quant) launch_quant_wave<BF16, MOE_QUANT_STATIC>(J, g, b, st, a);
                        else if (adaptive) launch_quant_wave<BF16, MOE_QUANT_DYN_TOKEN, true>(J, g, b, st, a);
                        else launch_quant_wave<BF16, MOE_QUANT_DYN_TOKEN>(J, g, b, st, a);
                    }
                } else {
                    const bool vec = h % 8 == 0 && aligned(x, 16) && aligned(expand_x, 8);
                    const dim3 g((unsigned)N), b(kBlockThreads);
#define MOE_QUANT_BLOCK(T, S)                                                                      \
                    do {                                                                           \
                        if (vec) hipLaunchKernelGGL((scatter_quant_block_kernel<T, true, S>), g, b, kdsm, st, a);   \
                        else hipLaunchKernelGGL((scatter_quant_block_kernel<T, false, S>), g, b, kdsm, st, a);      \
                    } while (0)
                    if (dtype == MOE_FP16) {
                        if (adaptive) MOE_QUANT_BLOCK(F16, true);
                        else MOE_QUANT_BLOCK(F16, false);
                    } else {
                        if (adaptive) MOE_QUANT_BLOCK(BF16, true);
                        else MOE_QUANT_BLOCK(BF16, false);
                    }
#undef MOE_QUANT_BLOCK
                }
            }
            // adaptive schedule: the large segments' rows, by wavefronts of their own
            if (adaptive) large_payload();
        } else {
            const long long npairs = N * K;
            hipLaunchKernelGGL(segment_meta_kernel, dim3((unsigned)((npairs + kBlockThreads - 1) / kBlockThreads)),
                               dim3(kBlockThreads), 0, st, a);
            segment_payload(kSegGrid);
        }
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

int moe_dispatch_noalloc(const void *x, const int32_t *expert_ids, const void *expert_scales,
                         const uint8_t *x_active_mask, int mask_kind, const moe_special_experts *special,
                         int ep_world, int bs, int experts_per_rank, int h, int topk, int dtype, int quant_mode,
                         const float *quant_scales, int64_t quant_scales_numel, void *expand_x,
                         void *dynamic_scales, int32_t *assist_info, int32_t *ep_recv_count, void *expand_scales,
                         const moe_schedule *schedule, void *stream)
{
    size_t need = 0;
    int rc = moe_dispatch_workspace_size(ep_world, bs, experts_per_rank, h, topk, dtype, quant_mode, &need);
    if (rc) return rc;
    if (need > kScratchBytes) return MOE_ERR_WORKSPACE;
    void *ws = scratch_on_current_device();
    if (!ws) {
        (void)hipGetLastError();
        return MOE_ERR_LAUNCH;
    }
    // Every dispatch kernel writes the workspace words it reads (chunk counts, ranks, offsets, the
    // plan and its length) before reading them, so nothing in the scratch must start at zero.
    return moe_dispatch(x, expert_ids, expert_scales, x_active_mask, mask_kind, special, ep_world, bs,
                        experts_per_rank, h, topk, dtype, quant_mode, quant_scales, quant_scales_numel, expand_x,
                        dynamic_scales, assist_info, ep_recv_count, expand_scales, schedule, ws, kScratchBytes,
                        stream);
}

int moe_combine_workspace_size(int ep_world, int bs, int experts_per_rank, int h, int topk, int dtype,
                               size_t *bytes)
{
    if (!bytes) return MOE_ERR_NULLPTR;
    int rc = check_scalars(ep_world, bs, experts_per_rank, h, topk, dtype);
    if (rc) return rc;
    *bytes = round_up((size_t)ep_world * bs * topk * 4, 256);
    return MOE_OK;
}

int moe_combine(const void *expand_x, const int32_t *assist_info, const int32_t *ep_recv_count,
                const int32_t *expert_ids, const void *expert_scales, const uint8_t *x_active_mask,
                int mask_kind, const moe_special_experts *special, int ep_world, int bs, int experts_per_rank,
                int h, int topk, int dtype, void *x_out, void *workspace, size_t workspace_bytes, void *stream)
{
    size_t need = 0;
    int rc = moe_combine_workspace_size(ep_world, bs, experts_per_rank, h, topk, dtype, &need);
    if (rc) return rc;
    const int W = ep_world, K = topk;
    const long long N = (long long)W * bs;
    if (!ep_recv_count) return MOE_ERR_NULLPTR;
    if (N > 0 && (!expand_x || !assist_info || !expert_ids || !expert_scales || !x_out || !workspace))
        return MOE_ERR_NULLPTR;
    if (mask_kind < MOE_MASK_NONE || mask_kind > MOE_MASK_PAIR) return MOE_ERR_MASK;
    if ((mask_kind != MOE_MASK_NONE) != (x_active_mask != nullptr) && N > 0) return MOE_ERR_MASK;
    if (mask_kind == MOE_MASK_NONE && x_active_mask) return MOE_ERR_MASK;
    if ((rc = check_special(special, (long long)W * experts_per_rank))) return rc;
    const int zero_n = special ? special->zero_expert_num : 0, copy_n = special ? special->copy_expert_num : 0;
    const int const_n = special ? special->const_expert_num : 0;
    const void *ori_x = copy_n > 0 ? special->ori_x : nullptr;
    const void *const_x = const_n > 0 ? special->const_x : nullptr;
    if (copy_n > 0 && N > 0 && !ori_x) return MOE_ERR_NULLPTR;
    if (const_n > 0 && N > 0 && !const_x) return MOE_ERR_NULLPTR;
    if (workspace_bytes < need) return MOE_ERR_WORKSPACE;
    const size_t xs = elem_size(dtype);
    if (!aligned(expand_x, xs) || !aligned(assist_info, 4) || !aligned(ep_recv_count, 4) ||
        !aligned(expert_ids, 4) || !aligned(expert_scales, 4) || !aligned(x_out, xs) || !aligned(workspace, 16) ||
        !aligned(ori_x, xs) || !aligned(const_x, xs))
        return MOE_ERR_ALIGN;
    if (N == 0) return MOE_OK;

    CombineArgs a;
    a.expand_x = static_cast<const char *>(expand_x);
    a.assist = assist_info;
    a.scales = expert_scales;
    a.slot = static_cast<const int32_t *>(workspace);
    a.slot_out = static_cast<int32_t *>(workspace);
    a.x_out = static_cast<char *>(x_out);
    a.erc = ep_recv_count;
    a.mask = x_active_mask;
    a.mask_kind = mask_kind;
    a.ids = expert_ids;
    a.ori_x = static_cast<const char *>(ori_x);
    a.const_x = static_cast<const char *>(const_x);
    a.E = W * experts_per_rank;
    a.zero_end = a.E + zero_n;
    a.copy_end = a.zero_end + copy_n;
    a.const_end = a.copy_end + const_n;
    a.pair_pass = (mask_kind != MOE_MASK_NONE || zero_n + copy_n + const_n > 0) ? 1 : 0;
    a.W = W; a.bs = bs; a.h = h; a.K = K; a.R = (int)(N * K); a.S = experts_per_rank * W;
    a.epr = experts_per_rank;
    a.rowbytes = (long long)((size_t)h * xs);
    // the last kDeviceStoreBytes of x_out (all of it up to that size) go device-scope
    a.dev_from = (int)std::max<long long>(0, N - (long long)(kDeviceStoreBytes / std::max<size_t>(1, (size_t)h * xs)));
    const bool vec = (size_t)a.rowbytes % 16 == 0 && aligned(expand_x, 16) && aligned(x_out, 16) &&
                     aligned(ori_x, 16) && aligned(const_x, 16);
    const long long n = vec ? a.rowbytes / 16 : h;
    a.nsl = (int)((n + kGatherThreads - 1) / kGatherThreads);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const size_t kdsm = (size_t)2 * K * sizeof(int);
    const dim3 g((unsigned)(N * a.nsl)), b(kGatherThreads);
    (void)hipGetLastError();
    // One launch: slots found in each workgroup (see combine_fused_kernel)
    if (vec && K <= kFusedMaxK && N * K <= kFusedCombinePairs && (long long)bs * K <= kFusedCombineSrcPairs) {
        const long long ws = (long long)W * a.S;
        const int ps = ws <= 4 * kGatherThreads ? 4 : ws <= kFusedCombineLdsCounts ? 16 : 0;
        const bool k8 = K <= 8;
        const size_t lds = ps ? (size_t)ws * sizeof(int) : 0;
#define MOE_FUSED_COMBINE_M(T, M)                                                                   \
        do {                                                                                        \
            if (ps == 4 && k8) hipLaunchKernelGGL((combine_fused_kernel<T, 8, 4, M>), g, b, lds, st, a);    \
            else if (ps == 4) hipLaunchKernelGGL((combine_fused_kernel<T, 16, 4, M>), g, b, lds, st, a);    \
            else if (ps && k8) hipLaunchKernelGGL((combine_fused_kernel<T, 8, 16, M>), g, b, lds, st, a);   \
            else if (ps) hipLaunchKernelGGL((combine_fused_kernel<T, 16, 16, M>), g, b, lds, st, a);       \
            else if (k8) hipLaunchKernelGGL((combine_fused_kernel<T, 8, 0, M>), g, b, lds, st, a);         \
            else hipLaunchKernelGGL((combine_fused_kernel<T, 16, 0, M>), g, b, lds, st, a);                \
        } while (0)
#define MOE_FUSED_COMBINE(T)                                                                        \
        do {                                                                                        \
            if (a.mask_kind == MOE_MASK_NONE) MOE_FUSED_COMBINE_M(T, false);                           \
            else MOE_FUSED_COMBINE_M(T, true);                                                      \
        } while (0)
        if (dtype == MOE_INT32) MOE_FUSED_COMBINE(int32_t);
        else if (dtype == MOE_FP16) MOE_FUSED_COMBINE(F16);
        else MOE_FUSED_COMBINE(BF16);
#undef MOE_FUSED_COMBINE
#undef MOE_FUSED_COMBINE_M
        return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
    }
    hipLaunchKernelGGL(combine_slots_kernel, dim3((unsigned)((a.R + kSlotThreads - 1) / kSlotThreads)),
                       dim3(kSlotThreads), 0, st, a);
    if (dtype == MOE_INT32) {
        if (vec) hipLaunchKernelGGL(combine_gather_i32_kernel<true>, g, b, kdsm, st, a);
        else hipLaunchKernelGGL(combine_gather_i32_kernel<false>, g, b, kdsm, st, a);
    } else if (dtype == MOE_FP16) {
        if (vec) hipLaunchKernelGGL((combine_gather_half_kernel<F16, true>), g, b, kdsm, st, a);
        else hipLaunchKernelGGL((combine_gather_half_kernel<F16, false>), g, b, kdsm, st, a);
    } else {
        if (vec) hipLaunchKernelGGL((combine_gather_half_kernel<BF16, true>), g, b, kdsm, st, a);
        else hipLaunchKernelGGL((combine_gather_half_kernel<BF16, false>), g, b, kdsm, st, a);
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // extern "C"
