// Token top-k indices -> block presence -> Q->K and K->Q CSR, on the GPU.
//
// Index tensor (total_q, NHK, topk) scattered into a per-(query block, KV
// head) presence row, then compacted to per-query-block key-block lists --
// MagiAttention PR #334, Core changes item 2 -- and to the transposed
// per-key-block lists (K2Q metadata) of MagiAttention PR #331, "CSR Tile
// Mapping".  -1 marks an unused slot (xtuner PR #2096, Main Changes item 1);
// any value outside [0, Sk) is treated the same way.
//
// Kernels:
//   k_index_presence : one workgroup per (qb, hk, b); streams the block's
//                      block_q x topk indices with 16-byte loads (the next
//                      batch in flight while one is marked), sets bits of
//                      an LDS bitmap (test-then-set keeps LDS atomics rare once
//                      a block is marked), writes the uint8 presence row and
//                      its popcount.  HBM-bound on the index read.
//   k_counts         : popcount of presence rows (block-mask path only) and
//                      per-(b, h, kb) column counts (coalesced across kb, rows
//                      split over 4 waves), one launch with two block roles.
//   k_scan2          : two exclusive scans (rows, columns) -> row_ptr arrays.
//   k_fill           : one wave per CSR row of either form, ballot + prefix
//                      popcount writes the ascending column list; one launch.
//   k_csr_small      : masks of at most kCsrTotalBytes presence bytes (slices
//                      of at most kCsrSideMax x kCsrSideMax, kCsrSliceBytes;
//                      the offset counts re-read at most kCsrPrefixBytes):
//                      the whole presence -> CSR in one launch, one workgroup
//                      per (b, h) slice with the slice in LDS; its offset in
//                      the CSRs (the kept blocks of the slices before it) is
//                      counted by the workgroup itself, so none waits on another.
// The conversion is latency-bound at the benchmark's sizes, so launches are
// fused wherever no result crosses workgroups.
#include "device_common.hpp"
#include "kernels.hpp"

namespace isattn {
namespace {

constexpr int kPresThreads = 1024;
constexpr int kPresBatch = 4;                      // 16-byte index loads per thread per batch
constexpr int kScanThreads = 1024;
constexpr int kScanItems = 4;
constexpr int kCsrThreads = 1024;
// one workgroup handles a whole slice, so its time grows with the slice: at
// 64 x 64 blocks it beats the three-launch path (8 against 9 us), at
// 128 x 128 it takes twice as long (17-20 against 10 us)
constexpr int kCsrSliceBytes = 4096;
constexpr int kCsrSideMax = 1024;
constexpr int64_t kCsrTotalBytes = 256 * 1024;
constexpr int64_t kCsrPrefixBytes = 16 << 20;

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ void mark_key(uint32_t* bits, int x, int Sk, int bk, int bk_shift) {
    if (static_cast<unsigned>(x) < static_cast<unsigned>(Sk)) {
        const int kb = bk_shift >= 0 ? (x >> bk_shift) : (x / bk);
        const uint32_t bit = 1u << (kb & 31);
        uint32_t* w = bits + (kb >> 5);
        if ((__hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) & bit) == 0)
            __hip_atomic_fetch_or(w, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
}

__global__ __launch_bounds__(kPresThreads) void k_index_presence(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
    int32_t Sq, int32_t Sk, int32_t nhk, int32_t topk, int32_t bq, int32_t bk, int32_t bk_shift,
    int32_t n_qb, int32_t n_kb, int32_t vec4, uint8_t* __restrict__ presence, int32_t* __restrict__ qcnt) {
    extern __shared__ uint32_t bits[];
    __shared__ int red[kPresThreads / 64];
    const int qb = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int nwords = (n_kb + 31) >> 5;
    for (int w = tid; w < nwords; w += kPresThreads) bits[w] = 0;
    __syncthreads();

    // sequence b: index rows [first, first + Sq) and keys [0, Sk); packed
    // sequences (cu_q, cu_k) have their own lengths, at most the longest
    int64_t first = int64_t(b) * Sq;
    if (cu_q != nullptr) {
        first = cu_q[b];
        Sq = min(max(cu_q[b + 1] - cu_q[b], 0), Sq);
        Sk = min(max(cu_k[b + 1] - cu_k[b], 0), Sk);
    }
    const int r0 = qb * bq;
    const int rows = max(0, min(bq, Sq - r0));
    const int64_t row_stride = int64_t(nhk) * topk;
    const int32_t* base = idx + (first + r0) * row_stride + int64_t(hk) * topk;
    if (vec4) {
        // 16-byte loads in batches of kPresBatch per thread, the next batch in
        // flight while the current one is marked (two register buffers);
        // slots past the block's indices read as -1 (nothing selected)
        const int per_row = topk >> 2;
        const int total = rows * per_row;
        const int pr_shift = (per_row & (per_row - 1)) == 0 ? __builtin_ctz(unsigned(per_row)) : -1;
        auto fetch = [&](int u0, int4 (&x)[kPresBatch]) {
#pragma unroll
            for (int j = 0; j < kPresBatch; ++j) {
                const int uu = u0 + j * kPresThreads;
                x[j] = int4{-1, -1, -1, -1};
                if (uu < total) {
                    const int rr = pr_shift >= 0 ? uu >> pr_shift : uu / per_row;
                    const int c = uu - rr * per_row;
                    x[j] = *reinterpret_cast<const int4*>(base + rr * row_stride + 4 * c);
                }
            }
        };
        auto mark = [&](const int4 (&x)[kPresBatch]) {
#pragma unroll
            for (int j = 0; j < kPresBatch; ++j) {
                mark_key(bits, x[j].x, Sk, bk, bk_shift);
                mark_key(bits, x[j].y, Sk, bk, bk_shift);
                mark_key(bits, x[j].z, Sk, bk, bk_shift);
                mark_key(bits, x[j].w, Sk, bk, bk_shift);
            }
        };
        constexpr int kStep = kPresBatch * kPresThreads;
        int4 xa[kPresBatch], xb[kPresBatch];
        int u = tid;
        fetch(u, xa);
        while (u < total) {
            fetch(u + kStep, xb);
            mark(xa);
            u += kStep;
            if (u >= total) break;
            fetch(u + kStep, xa);
            mark(xb);
            u += kStep;
        }
    } else {
        const int total = rows * topk;
        for (int u = tid; u < total; u += kPresThreads) {
            const int rr = u / topk;
            const int c = u - rr * topk;
            mark_key(bits, base[rr * row_stride + c], Sk, bk, bk_shift);
        }
    }
    __syncthreads();

    uint8_t* out = presence + ((int64_t(b) * nhk + hk) * n_qb + qb) * int64_t(n_kb);
    for (int kb = tid; kb < n_kb; kb += kPresThreads) out[kb] = (bits[kb >> 5] >> (kb & 31)) & 1u;
    int cnt = 0;
    for (int w = tid; w < nwords; w += kPresThreads) cnt += __popc(bits[w]);
    cnt = wave_sum(cnt);
    if ((tid & 63) == 0) red[tid >> 6] = cnt;
    __syncthreads();
    if (tid == 0) {
        int t = 0;
#pragma unroll
        for (int i = 0; i < kPresThreads / 64; ++i) t += red[i];
        qcnt[(int64_t(b) * nhk + hk) * n_qb + qb] = t;
    }
}

// Row counts (blocks [0, row_blocks): 4 rows per block, one per wave) and
// column counts (the rest: block = (bh, 64-column tile), lane = column, wave
// w sums rows w, w + 4, ...) in one launch.
__global__ __launch_bounds__(256) void k_counts(const uint8_t* __restrict__ presence, int32_t rows,
                                                int32_t row_blocks, int32_t n_qb, int32_t n_kb,
                                                int32_t tiles, int32_t* __restrict__ qcnt,
                                                int32_t* __restrict__ kcnt) {
    __shared__ int part[4][64];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    if (int32_t(blockIdx.x) < row_blocks) {
        const int row = blockIdx.x * 4 + w;
        if (row >= rows) return;
        const uint8_t* p = presence + int64_t(row) * n_kb;
        int c = 0;
        for (int kb = lane; kb < n_kb; kb += 64) c += p[kb] != 0;
        c = wave_sum(c);
        if (lane == 0) qcnt[row] = c;
        return;
    }
    const int cb = blockIdx.x - row_blocks;
    const int bh = cb / tiles;
    const int kb = (cb - bh * tiles) * 64 + lane;
    int c = 0;
    if (kb < n_kb) {
        const uint8_t* p = presence + int64_t(bh) * n_qb * n_kb + kb;
#pragma unroll 4
        for (int qb = w; qb < n_qb; qb += 4) c += p[int64_t(qb) * n_kb] != 0;
    }
    part[w][lane] = c;
    __syncthreads();
    if (w == 0 && kb < n_kb) kcnt[int64_t(bh) * n_kb + kb] = part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane];
}

// Block 0 scans cnt0 -> ptr0, block 1 scans cnt1 -> ptr1 (exclusive, with
// ptr[0] = 0 and ptr[n] = total).
__global__ __launch_bounds__(kScanThreads) void k_scan2(const int32_t* __restrict__ cnt0, int32_t n0,
                                                        int32_t* __restrict__ ptr0,
                                                        const int32_t* __restrict__ cnt1, int32_t n1,
                                                        int32_t* __restrict__ ptr1) {
    const int32_t* cnt = blockIdx.x == 0 ? cnt0 : cnt1;
    const int n = blockIdx.x == 0 ? n0 : n1;
    int32_t* ptr = blockIdx.x == 0 ? ptr0 : ptr1;
    __shared__ int wsum[kScanThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    if (tid == 0) ptr[0] = 0;
    int carry = 0;
    for (int base = 0; base < n; base += kScanThreads * kScanItems) {
        int v[kScanItems];
        int s = 0;
#pragma unroll
        for (int j = 0; j < kScanItems; ++j) {
            const int i = base + tid * kScanItems + j;
            v[j] = i < n ? cnt[i] : 0;
            s += v[j];
        }
        int x = s;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        if (lane == 63) wsum[wid] = x;
        __syncthreads();
        if (wid == 0) {
            int t = lane < kScanThreads / 64 ? wsum[lane] : 0;
#pragma unroll
            for (int o = 1; o < kScanThreads / 64; o <<= 1) {
                const int y = __shfl_up(t, o, 64);
                if (lane >= o) t += y;
            }
            if (lane < kScanThreads / 64) wsum[lane] = t;
        }
        __syncthreads();
        int run = carry + (wid > 0 ? wsum[wid - 1] : 0) + (x - s);
#pragma unroll
        for (int j = 0; j < kScanItems; ++j) {
            const int i = base + tid * kScanItems + j;
            run += v[j];
            if (i < n) ptr[i + 1] = run;
        }
        carry += wsum[kScanThreads / 64 - 1];
        __syncthreads();
    }
}

// Column lists in one launch: blocks [0, q_blocks) fill the Q->K rows (one
// row per wave, lanes over 64 columns at a time), the rest the K->Q columns
// (one column per wave, lanes over 64 rows at a time); ballot + popcount
// place each kept block at its ascending position.
__global__ __launch_bounds__(256) void k_fill(const uint8_t* __restrict__ presence, int32_t rows,
                                              int32_t cols, int32_t q_blocks, int32_t n_qb,
                                              int32_t n_kb, const int32_t* __restrict__ q2k_ptr,
                                              int32_t* __restrict__ q2k_col,
                                              const int32_t* __restrict__ k2q_ptr,
                                              int32_t* __restrict__ k2q_col) {
    const int lane = threadIdx.x & 63;
    const uint64_t below = (uint64_t(1) << lane) - 1;
    if (int32_t(blockIdx.x) < q_blocks) {
        const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
        if (row >= rows) return;
        const uint8_t* p = presence + int64_t(row) * n_kb;
        int base = q2k_ptr[row];
        for (int c0 = 0; c0 < n_kb; c0 += 64) {
            const int kb = c0 + lane;
            const bool on = kb < n_kb && p[kb] != 0;
            const uint64_t m = __ballot(on);
            if (on) q2k_col[base + __popcll(m & below)] = kb;
            base += __popcll(m);
        }
        return;
    }
    const int col = (blockIdx.x - q_blocks) * 4 + (threadIdx.x >> 6);
    if (col >= cols) return;
    const int bh = col / n_kb;
    const int kb = col - bh * n_kb;
    const uint8_t* p = presence + int64_t(bh) * n_qb * n_kb + kb;
    int base = k2q_ptr[col];
    for (int q0 = 0; q0 < n_qb; q0 += 64) {
        const int qb = q0 + lane;
        const bool on = qb < n_qb && p[int64_t(qb) * n_kb] != 0;
        const uint64_t m = __ballot(on);
        if (on) k2q_col[base + __popcll(m & below)] = qb;
        base += __popcll(m);
    }
}

// Kept (nonzero) bytes of a 32-bit word.
__device__ __forceinline__ int nonzero_bytes(uint32_t w) {
    uint32_t x = w | (w >> 4);
    x |= x >> 2;
    x |= x >> 1;
    return __popc(x & 0x01010101u);
}

// Exclusive scan over the kCsrThreads threads of a workgroup (one 64-bit
// value each); *total gets the sum.  wsum holds kCsrThreads / 64 values.
__device__ int64_t csr_block_scan(int64_t v, int64_t* wsum, int64_t* total) {
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    int64_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int64_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wid] = x;
    __syncthreads();
    int64_t pre = x - v, tot = 0;
#pragma unroll
    for (int w = 0; w < kCsrThreads / 64; ++w) {
        pre += w < wid ? wsum[w] : 0;
        tot += wsum[w];
    }
    __syncthreads();
    *total = tot;
    return pre;
}

// One workgroup per slice bh = (b, h) of a presence [BH, n_qb, n_kb]
// (n_qb, n_kb <= kCsrSideMax, n_qb * n_kb <= kCsrSliceBytes): counts the
// kept blocks of the slices before it (its offset in both CSRs), stages its
// slice in LDS, counts rows (ballot per wave) and columns (LDS atomics),
// scans the three counts packed in one 64-bit value, writes its row_ptr entries and fills both column lists in
// ascending order.
__global__ __launch_bounds__(kCsrThreads) void k_csr_small(const uint8_t* __restrict__ presence, int32_t n_qb,
                                                           int32_t n_kb, int32_t* __restrict__ q2k_ptr,
                                                           int32_t* __restrict__ q2k_col,
                                                           int32_t* __restrict__ k2q_ptr,
                                                           int32_t* __restrict__ k2q_col) {
    __shared__ __attribute__((aligned(16))) uint8_t pres[kCsrSliceBytes];
    __shared__ int rcnt[kCsrSideMax];
    __shared__ int ccnt[kCsrSideMax];
    __shared__ int64_t wsum[kCsrThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    constexpr int NW = kCsrThreads / 64;
    const uint64_t below = (uint64_t(1) << lane) - 1;
    const int bh = blockIdx.x;
    const int S = n_qb * n_kb;
    const int64_t before = int64_t(bh) * S;
    const uint8_t* slice = presence + before;
    const bool vec = (reinterpret_cast<uintptr_t>(presence) & 15) == 0 && (S & 15) == 0;

    // the slice's own bytes requested first (at most one 16-byte piece per
    // thread), then the offset: kept blocks of the slices before this one
    u32x4_t own = {0u, 0u, 0u, 0u};
    if (vec && tid < S / 16) own = reinterpret_cast<const u32x4_t*>(slice)[tid];
    int c = 0;
    if (vec) {
        // eight 16-byte loads in flight per thread (the latest slice reads up to
        // kCsrTotalBytes, 16 per thread)
        const u32x4_t* p4 = reinterpret_cast<const u32x4_t*>(presence);
        const int64_t n16 = before / 16;
        for (int64_t i0 = 0; i0 < n16; i0 += 8 * kCsrThreads) {
            u32x4_t w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t i = i0 + j * kCsrThreads + tid;
                w[j] = i < n16 ? p4[i] : u32x4_t{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int j = 0; j < 8; ++j)
                c += nonzero_bytes(w[j][0]) + nonzero_bytes(w[j][1]) + nonzero_bytes(w[j][2]) + nonzero_bytes(w[j][3]);
        }
        if (tid < S / 16) reinterpret_cast<u32x4_t*>(pres)[tid] = own;
    } else {
        for (int64_t i = tid; i < before; i += kCsrThreads) c += presence[i] != 0;
        for (int i = tid; i < S; i += kCsrThreads) pres[i] = slice[i];
    }
    for (int i = tid; i < n_kb; i += kCsrThreads) ccnt[i] = 0;
    __syncthreads();

    // row counts (one wave per row) and column counts
    for (int r = wid; r < n_qb; r += NW) {
        int n = 0;
        for (int c0 = 0; c0 < n_kb; c0 += 64) {
            const int kb = c0 + lane;
            const bool on = kb < n_kb && pres[r * n_kb + kb] != 0;
            if (on) atomicAdd(&ccnt[kb], 1);
            n += __popcll(__ballot(on));
        }
        if (lane == 0) rcnt[r] = n;
    }
    __syncthreads();
    // one scan for all three: row counts (bits 0-15), column counts (bits
    // 16-31; both at most 16384 in all) and the offset count (bits 32-; only
    // its total is used)
    const int rc = tid < n_qb ? rcnt[tid] : 0;
    const int cc = tid < n_kb ? ccnt[tid] : 0;
    int64_t tot = 0;
    const int64_t x = csr_block_scan((int64_t(c) << 32) | (int64_t(cc) << 16) | int64_t(rc), wsum, &tot);
    const int off = int(tot >> 32);
    const int rx = int(x & 0xffff), cx = int((x >> 16) & 0xffff);
    if (tid < n_qb) {
        rcnt[tid] = off + rx;                      // start of row tid's list
        q2k_ptr[int64_t(bh) * n_qb + tid + 1] = off + rx + rc;
    }
    if (tid < n_kb) {
        ccnt[tid] = off + cx;
        k2q_ptr[int64_t(bh) * n_kb + tid + 1] = off + cx + cc;
    }
    if (bh == 0 && tid == 0) {
        q2k_ptr[0] = 0;
        k2q_ptr[0] = 0;
    }
    __syncthreads();

    // column lists: ballot + prefix popcount place each kept block
    for (int r = wid; r < n_qb; r += NW) {
        int base = rcnt[r];
        for (int c0 = 0; c0 < n_kb; c0 += 64) {
            const int kb = c0 + lane;
            const bool on = kb < n_kb && pres[r * n_kb + kb] != 0;
            const uint64_t m = __ballot(on);
            if (on) q2k_col[base + __popcll(m & below)] = kb;
            base += __popcll(m);
        }
    }
    for (int k = wid; k < n_kb; k += NW) {
        int base = ccnt[k];
        for (int q0 = 0; q0 < n_qb; q0 += 64) {
            const int qb = q0 + lane;
            const bool on = qb < n_qb && pres[qb * n_kb + k] != 0;
            const uint64_t m = __ballot(on);
            if (on) k2q_col[base + __popcll(m & below)] = qb;
            base += __popcll(m);
        }
    }
}

// Token bits: every slot cleared, then one workgroup per (qb, hk, b) sets the
// bits of its rows' selected keys in both layouts (row-major and key-major)
// with relaxed 32-bit atomic ORs (rows of one block hit the same words).
__global__ __launch_bounds__(256) void k_tok_clear(uint32_t* __restrict__ bits, int64_t n4) {
    const int64_t stride = int64_t(gridDim.x) * 256;
    for (int64_t u = int64_t(blockIdx.x) * 256 + threadIdx.x; u < n4; u += stride)
        reinterpret_cast<u32x4_t*>(bits)[u] = u32x4_t{0u, 0u, 0u, 0u};
}

__global__ __launch_bounds__(256) void k_tok_set(const int32_t* __restrict__ idx, const int32_t* __restrict__ cu_q,
                                                 const int32_t* __restrict__ cu_k, int32_t Sq, int32_t Sk,
                                                 int32_t nhk, int32_t topk, int32_t n_qb, int32_t n_kb,
                                                 uint32_t* __restrict__ bits) {
    const int qb = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    int64_t first = int64_t(b) * Sq;
    if (cu_q != nullptr) {
        first = cu_q[b];
        Sq = min(max(cu_q[b + 1] - cu_q[b], 0), Sq);
        Sk = min(max(cu_k[b + 1] - cu_k[b], 0), Sk);
    }
    const int r0 = qb * kBlock;
    const int rows = max(0, min(kBlock, Sq - r0));
    const int64_t row_stride = int64_t(nhk) * topk;
    const int32_t* base = idx + (first + r0) * row_stride + int64_t(hk) * topk;
    uint32_t* slots = bits + ((int64_t(b) * nhk + hk) * n_qb + qb) * int64_t(n_kb) * 1024;
    const int total = rows * topk;
    for (int u = threadIdx.x; u < total; u += 256) {
        const int r = u / topk;
        const int j = base[int64_t(r) * row_stride + (u - r * topk)];
        if (static_cast<unsigned>(j) >= static_cast<unsigned>(Sk)) continue;   // padding
        uint32_t* slot = slots + int64_t(j / kBlock) * 1024;
        const int jj = j % kBlock;
        __hip_atomic_fetch_or(slot + 4 * r + jj / 32, 1u << (jj & 31), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_or(slot + 512 + 4 * jj + r / 32, 1u << (r & 31), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace

hipError_t launch_index_token_bits(const int32_t* idx, const int32_t* cu_q, const int32_t* cu_k, int32_t B,
                                   int32_t Sq, int32_t Sk, int32_t nhk, int32_t topk, int32_t n_qb,
                                   int32_t n_kb, uint32_t* bits, hipStream_t s) {
    const int64_t n4 = int64_t(B) * nhk * n_qb * n_kb * 256;
    if (n4 == 0) return hipSuccess;
    const int64_t nb = (n4 + 255) / 256;
    hipLaunchKernelGGL(k_tok_clear, dim3(unsigned(nb < 16384 ? nb : 16384)), dim3(256), 0, s, bits, n4);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_tok_set, dim3(n_qb, nhk, B), dim3(256), 0, s, idx, cu_q, cu_k, Sq, Sk, nhk, topk, n_qb,
                       n_kb, bits);
    return hipGetLastError();
}

hipError_t launch_index_presence(const int32_t* idx, const int32_t* cu_q, const int32_t* cu_k, int32_t B,
                                 int32_t Sq, int32_t Sk, int32_t nhk, int32_t topk, int32_t bq, int32_t bk,
                                 int32_t n_qb, int32_t n_kb, uint8_t* presence, int32_t* qcnt,
                                 hipStream_t s) {
    if (B == 0 || nhk == 0 || n_qb == 0) return hipSuccess;
    const int bk_shift = (bk & (bk - 1)) == 0 ? __builtin_ctz(unsigned(bk)) : -1;
    const int vec4 = (topk % 4 == 0) && ((reinterpret_cast<uintptr_t>(idx) & 15u) == 0);
    const size_t lds = size_t((n_kb + 31) / 32) * sizeof(uint32_t);
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_index_presence),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return e;
    }
    dim3 grid(n_qb, nhk, B);
    hipLaunchKernelGGL(k_index_presence, grid, dim3(kPresThreads), lds, s, idx, cu_q, cu_k, Sq, Sk, nhk, topk,
                       bq, bk, bk_shift, n_qb, n_kb, vec4, presence, qcnt);
    return hipGetLastError();
}

hipError_t launch_presence_to_csr(const uint8_t* presence, int32_t BH, int32_t n_qb,
                                  int32_t n_kb, bool have_row_counts, int32_t* qcnt,
                                  int32_t* kcnt, int32_t* q2k_ptr, int32_t* q2k_col,
                                  int32_t* k2q_ptr, int32_t* k2q_col, hipStream_t s) {
    const int32_t rows = BH * n_qb;
    const int32_t cols = BH * n_kb;
    const int64_t slice = int64_t(n_qb) * n_kb;
    // the single launch while each workgroup's offset count stays small: the
    // slices before it hold at most kCsrTotalBytes, and all workgroups
    // together re-read at most kCsrPrefixBytes of presence
    if (BH > 0 && slice > 0 && n_qb <= kCsrSideMax && n_kb <= kCsrSideMax && slice <= kCsrSliceBytes &&
        int64_t(BH) * slice <= kCsrTotalBytes && int64_t(BH) * (BH - 1) / 2 * slice <= kCsrPrefixBytes) {
        hipLaunchKernelGGL(k_csr_small, dim3(BH), dim3(kCsrThreads), 0, s, presence, n_qb, n_kb, q2k_ptr, q2k_col,
                           k2q_ptr, k2q_col);
        return hipGetLastError();
    }
    const int32_t row_blocks = rows > 0 && !have_row_counts ? (rows + 3) / 4 : 0;
    const int32_t tiles = (n_kb + 63) / 64;
    const int32_t col_blocks = cols > 0 ? BH * tiles : 0;
    if (row_blocks + col_blocks > 0)
        hipLaunchKernelGGL(k_counts, dim3(row_blocks + col_blocks), dim3(256), 0, s, presence, rows,
                           row_blocks, n_qb, n_kb, tiles, qcnt, kcnt);
    hipLaunchKernelGGL(k_scan2, dim3(2), dim3(kScanThreads), 0, s, qcnt, rows, q2k_ptr, kcnt, cols,
                       k2q_ptr);
    const int32_t q_blocks = rows > 0 && n_kb > 0 ? (rows + 3) / 4 : 0;
    const int32_t k_blocks = cols > 0 && n_qb > 0 ? (cols + 3) / 4 : 0;
    if (q_blocks + k_blocks > 0)
        hipLaunchKernelGGL(k_fill, dim3(q_blocks + k_blocks), dim3(256), 0, s, presence, rows, cols,
                           q_blocks, n_qb, n_kb, q2k_ptr, q2k_col, k2q_ptr, k2q_col);
    return hipGetLastError();
}

}  // namespace isattn
