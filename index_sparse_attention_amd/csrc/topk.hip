// Top-k selection of index rows from scores: the DSA indexer's selection step
// that produces the (total_q, NHK, topk) index tensor (xtuner PR #2096, Main
// Changes item 1: radix selection over fp32 keys restricted to each row's
// [start, end) range, indices ordered by score, -1 where a row has fewer
// valid positions than topk).
//
// One workgroup per row, 512 threads:
//   1. scores become order-preserving unsigned keys (negative floats
//      bit-inverted, positive ones with the sign bit set, -0 taken as +0);
//   2. radix select, 8 bits per pass from the top: a 256-bin LDS histogram of
//      the digit over the keys that share the prefix found so far picks the
//      digit of the topk-th largest key; after 4 passes the threshold key T
//      and how many keys equal to T are still needed are known;
//   3. one collection pass takes every key > T and, in position order, the
//      first keys equal to T (ties resolve to the smaller position);
//   4. a bitonic sort orders the selection by (key descending, position
//      ascending) and the row is written, padded with -1.  The sort keeps
//      E = CAP / 512 entries per thread in registers: exchanges between a
//      thread's own entries happen in registers, exchanges within a wave by
//      lane shuffles, and only partners in other waves go through LDS.
// Rows with no more valid positions than topk skip the radix passes.  The
// row is re-read from global memory by every pass (L2-resident after the
// first); scores are only read, never modified.
#include "device_common.hpp"
#include "kernels.hpp"

namespace isattn {
namespace {

constexpr int kTopkThreads = 512;
constexpr int kTopkUnroll = 8;    // positions per thread whose loads are in flight together

__device__ __forceinline__ uint32_t order_key(float x) {
    const uint32_t u = x == 0.f ? 0u : __float_as_uint(x);   // -0 and +0 are one score
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix over the workgroup of one flag per thread (thread order);
// *total receives the count.  Uses 64-lane ballots and an LDS word per wave.
__device__ __forceinline__ int block_rank(bool flag, int* wcnt, int* total) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const uint64_t m = __ballot(flag);
    if (lane == 0) wcnt[w] = __popcll(m);
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < kTopkThreads / 64; ++i) {
        const int c = wcnt[i];
        before += i < w ? c : 0;
        all += c;
    }
    __syncthreads();
    *total = all;
    return before + __popcll(m & ((uint64_t(1) << lane) - 1));
}

// one compare-exchange result: the entry this side keeps
__device__ __forceinline__ uint64_t bitonic_keep(uint64_t mine, uint64_t other, bool lower, bool desc) {
    const bool take_max = lower == desc;
    return take_max ? (mine > other ? mine : other) : (mine < other ? mine : other);
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
    const uint32_t lo = uint32_t(__shfl_xor(int(uint32_t(v)), m, 64));
    const uint32_t hi = uint32_t(__shfl_xor(int(uint32_t(v >> 32)), m, 64));
    return (uint64_t(hi) << 32) | lo;
}

// Sort the first `size` (a power of two, at most 512 E) entries of sel
// descending; returns with thread t holding entries t E .. t E + E - 1 of the
// sorted order in v (entries past `size` stay in place: the network never
// pairs them with the first `size`).
template <int E>
__device__ __forceinline__ void bitonic_sort(uint64_t* sel, uint64_t (&v)[E], int size) {
    const int t = threadIdx.x;
    const int lane = t & 63;
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = sel[t * E + e];
    for (int k = 2; k <= size; k <<= 1) {
        // partners in other threads (j >= E), largest distance first
        for (int j = k >> 1; j >= E; j >>= 1) {
            if (j < 64 * E) {                               // partner in another lane of this wave
                const int m = j / E;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int i = t * E + e;
                    v[e] = bitonic_keep(v[e], shfl_xor64(v[e], m), (lane & m) == 0, (i & k) == 0);
                }
            } else {                                        // partner in another wave: through LDS
                __syncthreads();
#pragma unroll
                for (int e = 0; e < E; ++e) sel[t * E + e] = v[e];
                __syncthreads();
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int i = t * E + e;
                    v[e] = bitonic_keep(v[e], sel[i ^ j], (i & j) == 0, (i & k) == 0);
                }
            }
        }
        // partners in this thread's registers (j < E): compile-time indices
#pragma unroll
        for (int j = E / 2; j > 0; j >>= 1) {
            if (j < k) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    if ((e & j) == 0) {
                        const bool desc = ((t * E + e) & k) == 0;
                        const uint64_t a = v[e], b = v[e | j];
                        v[e] = bitonic_keep(a, b, true, desc);
                        v[e | j] = bitonic_keep(b, a, false, desc);
                    }
                }
            }
        }
    }
}

template <int E>
__global__ __launch_bounds__(kTopkThreads) void k_topk(const float* __restrict__ scores, int64_t ld, int32_t n,
                                                       const int32_t* __restrict__ starts,
                                                       const int32_t* __restrict__ ends, int32_t topk,
                                                       int32_t* __restrict__ out) {
    constexpr int CAP = kTopkThreads * E;
    extern __shared__ uint64_t sel[];                 // CAP (key << 32 | ~position) entries
    __shared__ int hist[256];
    __shared__ int wcnt[kTopkThreads / 64];
    __shared__ int s_digit, s_above;
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const float* x = scores + row * ld;
    int lo = starts != nullptr ? starts[row] : 0;
    int hi = ends != nullptr ? ends[row] : n;
    lo = max(lo, 0);
    hi = min(hi, n);
    const int valid = max(hi - lo, 0);
    const int take = min(valid, topk);

    uint32_t thr = 0;                                  // keys > thr all taken
    int need_eq = 0;                                   // how many keys == thr to take
    bool radix = valid > topk;
    if (radix) {
        uint32_t prefix = 0, pmask = 0;
        int rem = topk;
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0;
            __syncthreads();
            for (int base = lo; base < hi; base += kTopkUnroll * kTopkThreads) {
                float v[kTopkUnroll];
#pragma unroll
                for (int u = 0; u < kTopkUnroll; ++u) {
                    const int j = base + u * kTopkThreads + tid;
                    v[u] = j < hi ? x[j] : 0.f;
                }
#pragma unroll
                for (int u = 0; u < kTopkUnroll; ++u) {
                    const uint32_t key = order_key(v[u]);
                    if (base + u * kTopkThreads + tid < hi && (key & pmask) == prefix)
                        atomicAdd(&hist[(key >> shift) & 255], 1);
                }
            }
            __syncthreads();
            if (tid < 64) {
                // bins from the top: find the digit where the running count reaches rem
                int c[4], s = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    c[q] = hist[255 - (4 * tid + q)];
                    s += c[q];
                }
                int incl = s;                          // inclusive scan over lanes (bins 255 .. 0)
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int t = __shfl_up(incl, o, 64);
                    if ((tid & 63) >= o) incl += t;
                }
                int run = incl - s;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (run < rem && run + c[q] >= rem) {
                        s_digit = 255 - (4 * tid + q);
                        s_above = run;
                    }
                    run += c[q];
                }
            }
            __syncthreads();
            rem -= s_above;
            prefix |= uint32_t(s_digit) << shift;
            pmask |= 255u << shift;
            __syncthreads();
        }
        thr = prefix;
        need_eq = rem;
    }

    // collection in position order, chunks of kTopkThreads positions
    int filled = 0, eq_seen = 0;
    for (int base0 = lo; base0 < hi; base0 += kTopkUnroll * kTopkThreads) {
        float v[kTopkUnroll];
#pragma unroll
        for (int u = 0; u < kTopkUnroll; ++u) {
            const int j = base0 + u * kTopkThreads + tid;
            v[u] = j < hi ? x[j] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kTopkUnroll; ++u) {
            const int base = base0 + u * kTopkThreads;
            if (base >= hi) break;                     // uniform: every thread sees the same base
            const int j = base + tid;
            const bool in = j < hi;
            const uint32_t key = in ? order_key(v[u]) : 0u;
            const bool gt = in && (!radix || key > thr);
            const bool eq = in && radix && key == thr;
            int n_eq = 0;
            const int r_eq = block_rank(eq, wcnt, &n_eq);
            const bool take_eq = eq && eq_seen + r_eq < need_eq;
            int n_take = 0;
            const int slot = block_rank(gt || take_eq, wcnt, &n_take);
            if (gt || take_eq) sel[filled + slot] = (uint64_t(key) << 32) | uint32_t(~uint32_t(j));
            filled += n_take;
            eq_seen += n_eq;
        }
    }
    // pad to the sort size with entries that sort last (a real entry is
    // never 0: its low word is a bit-inverted position below 2^31)
    for (int i = take + tid; i < CAP; i += kTopkThreads) sel[i] = 0;
    __syncthreads();
    int size = 1;
    while (size < take) size <<= 1;
    uint64_t v[E];
    bitonic_sort<E>(sel, v, size);
    int32_t* o = out + row * int64_t(topk);
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = tid * E + e;
        if (i < topk) o[i] = i < take ? int32_t(~uint32_t(v[e])) : -1;
    }
}

template <int E>
hipError_t launch_topk_e(const float* scores, int64_t ld, int32_t rows, int32_t n, const int32_t* starts,
                         const int32_t* ends, int32_t topk, int32_t* out, hipStream_t s) {
    const size_t lds = size_t(kTopkThreads) * E * sizeof(uint64_t);
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_topk<E>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_topk<E>, dim3(unsigned(rows)), dim3(kTopkThreads), lds, s, scores, ld, n, starts, ends,
                       topk, out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const float* scores, int64_t ld, int32_t rows, int32_t n, const int32_t* starts,
                       const int32_t* ends, int32_t topk, int32_t* out, hipStream_t s) {
    if (rows == 0 || topk == 0) return hipSuccess;
    // sort size: 512 x E entries, E the smallest power of two with 512 E >= topk
    if (topk <= 512) return launch_topk_e<1>(scores, ld, rows, n, starts, ends, topk, out, s);
    if (topk <= 1024) return launch_topk_e<2>(scores, ld, rows, n, starts, ends, topk, out, s);
    if (topk <= 2048) return launch_topk_e<4>(scores, ld, rows, n, starts, ends, topk, out, s);
    if (topk <= 4096) return launch_topk_e<8>(scores, ld, rows, n, starts, ends, topk, out, s);
    return launch_topk_e<16>(scores, ld, rows, n, starts, ends, topk, out, s);
}

}  // namespace isattn
