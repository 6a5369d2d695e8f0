// Device helpers for gfx950 (CDNA4): bf16 MFMA wrappers, packing, loads.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <utility>

namespace isattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// D = A(32x16) * B(16x32) + C, fp32 accumulate.  Lane l: A row l%32 and B
// column l%32, eight k-slots 8*(l/32)..+7; C/D register i holds row
// 8*(i/4) + 4*(l/32) + i%4 of column l%32.
__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D = A(16x32) * B(32x16) + C.  Lane l: A row l%16 and B column l%16, k-slots
// 8*(l/16)..+7; C/D register i holds row 4*(l/16) + i of column l%16.
__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp32 pair -> packed bf16 pair, round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2_t x = {lo, hi};
    bf16x2_t y = __builtin_convertvector(x, bf16x2_t);
    return __builtin_bit_cast(uint32_t, y);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t w) { return __builtin_bit_cast(bf16x8_t, w); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Hardware fp32 atomic add (global_atomic_add_f32, no return value).
__device__ __forceinline__ void atomic_add_f32(float* p, float v) { unsafeAtomicAdd(p, v); }

__device__ __forceinline__ u32x4_t lds_read128(const uint16_t* p) {
    return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ u32x2_t lds_read64(const uint16_t* p) {
    return *reinterpret_cast<const u32x2_t*>(p);
}

__device__ __forceinline__ u32x4_t gload128(const uint16_t* p) {
    return *reinterpret_cast<const u32x4_t*>(p);
}
// 16-byte global row chunk as an MFMA operand (resident operands are read once
// per workgroup straight from HBM).
__device__ __forceinline__ bf16x8_t gload_operand(const uint16_t* p) { return as_bf16x8(gload128(p)); }

}  // namespace isattn

namespace isattn {

// Swap bits 2 and 3 of a row index.  Staging tile row r at LDS row
// swap23(r) makes the 32x32 MFMA accumulator registers 8c..8c+7 of lane
// half h hold logical rows 16c + 8h + 0..7 -- eight consecutive rows, so the
// accumulator can feed the next MFMA as an operand whose partner operand is
// read as contiguous runs.
__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// (i % 4) of the 8-byte runs addressed by lanes 4s + i/4, s = 0..3.  Pointing
// lane L of a group at row (r0 + L/4), column (c0 + 4*(L%4)) of a row-major
// bf16 tile returns, in lane i, rows r0..r0+3 of column c0 + i: four
// consecutive k of one MFMA B-operand column.
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint16_t* p) {
    typedef short i16x4_t __attribute__((ext_vector_type(4)));
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)(p));
    return __builtin_bit_cast(u32x2_t, v);
}

}  // namespace isattn

namespace isattn {

// Cooperative copy of ROWS rows x D bf16 of a [seq, D] slice (row stride in
// elements) into LDS with row pitch PITCH.  All of a thread's 16-byte global
// loads are issued before any LDS store, so their latencies overlap; load()
// and store() can be split around other work to prefetch the next tile.
// Rows at or past `limit` read as zeros.  With PERM, tile row r lands at LDS
// row swap23(r).
__device__ __forceinline__ int chunk_swz(int r, int D);   // below: the chunk swizzle of a tile row

template <int D, int PITCH, int ROWS, int NT, bool PERM>
struct TileStager {
    static constexpr int CH = D / 8;               // 16-byte chunks per row
    static constexpr int N = ROWS * CH / NT;       // chunks per thread
    static_assert((ROWS * CH) % NT == 0, "tile must split evenly over the threads");
    u32x4_t v[N];

    __device__ __forceinline__ void load(const uint16_t* src, int64_t row_stride, int row0, int limit,
                                         int tid) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int u = tid + i * NT;
            const int r = u / CH;
            const int c = u - r * CH;
            const int gr = row0 + r;
            v[i] = u32x4_t{0u, 0u, 0u, 0u};
            if (gr < limit) v[i] = gload128(src + gr * row_stride + 8 * c);
        }
    }
    __device__ __forceinline__ void store(uint16_t* dst, int tid) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int u = tid + i * NT;
            const int r = u / CH;
            const int c = u - r * CH;
            const int lr = PERM ? swap23(r) : r;
            *reinterpret_cast<u32x4_t*>(dst + lr * PITCH + 8 * c) = v[i];
        }
    }
    // Row-major copy into a swizzled tile without padding (PITCH == D): tile
    // row r at LDS row swap23(r) when PERM, chunk c at c ^ chunk_swz(row, D).
    __device__ __forceinline__ void store_swz(uint16_t* dst, int tid) const {
        static_assert(PITCH == D, "swizzled tiles have no padding");
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int u = tid + i * NT;
            const int r = u / CH;
            const int c = u - r * CH;
            const int lr = PERM ? swap23(r) : r;
            *reinterpret_cast<u32x4_t*>(dst + lr * D + 8 * (c ^ chunk_swz(lr, D))) = v[i];
        }
    }
    // Transposed copy: element (r, d) to dstT[d * PT + r].
    template <int PT>
    __device__ __forceinline__ void store_t(uint16_t* dstT, int tid) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int u = tid + i * NT;
            const int r = u / CH;
            const int c = u - r * CH;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                dstT[(8 * c + 2 * j) * PT + r] = uint16_t(v[i][j] & 0xffffu);
                dstT[(8 * c + 2 * j + 1) * PT + r] = uint16_t(v[i][j] >> 16);
            }
        }
    }
};

}  // namespace isattn

namespace isattn {

// ---- swizzled LDS tiles filled by direct global->LDS loads -----------------
// A tile of ROWS x D bf16 is stored unpadded (row r at element r * D); its
// 16-byte chunk c sits at chunk position c ^ chunk_swz(r, D).  gfx950 LDS has
// 64 banks of 4 bytes: a ds_read_b128 is served 16 lanes per pass and a
// ds_read_b64(_tr_b16) 32 lanes per pass, each pass conflict-free when its
// lanes cover distinct banks.  The XOR makes both patterns used here
// conflict-free: 16 consecutive rows reading one chunk each (b128 operand
// reads), and 4 consecutive rows x 4 consecutive chunks starting at a row
// multiple of 4 (transposing reads).  With 16 or more chunks per row the rows
// start on the same bank and the XOR spans 4 bits; with 8 or 24 chunks per row
// odd rows start half a bank line later and a 3-bit XOR (which keeps a chunk
// inside its aligned group of 8) suffices.
__device__ __forceinline__ int chunk_swz(int r, int D) {
    return (D / 8) % 16 == 0 ? ((r & 3) << 2) | ((r >> 2) & 3) : (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

template <int D>
__device__ __forceinline__ int swz_off(int r, int elem) {
    return r * D + ((((elem >> 3) ^ chunk_swz(r, D)) << 3) | (elem & 7));
}

// Async copy of tile rows [row0, row0 + ROWS) of a [seq, D] slice into a
// swizzled LDS tile, tile row t landing at LDS row swap23(t).  Each wave issues
// 1 KiB direct-to-LDS loads (global_load_lds_dwordx4: lane L's 16 bytes go to
// the instruction's LDS base + 16 * L).  Rows at or past `limit` are clamped
// to limit - 1 (in-bounds data that the caller masks out); limit must be > 0.
// Returns nothing; completion is tracked by vmcnt.
template <int D, int ROWS, int NW>
__device__ __forceinline__ void load_tile_async(uint16_t* tile, const uint16_t* src, int64_t row_stride,
                                                int row0, int limit, int wave, int lane) {
    constexpr int NI = ROWS * D * 2 / 1024;        // 1 KiB instructions per tile
    static_assert((ROWS * D * 2) % 1024 == 0 && NI % NW == 0, "tile must split into whole wave loads");
#pragma unroll
    for (int k = 0; k < NI / NW; ++k) {
        const int j = wave + k * NW;
        const int e = 512 * j + 8 * lane;          // element offset this lane fills
        const int r = e / D;
        const int p = (e - r * D) >> 3;
        const int c = p ^ chunk_swz(r, D);
        const int gr = min(row0 + swap23(r), limit - 1);
        __builtin_amdgcn_global_load_lds(src + gr * row_stride + 8 * c,
                                         (__attribute__((address_space(3))) void*)(tile + 512 * j), 16, 0, 0);
    }
}

// ---- operand reads at per-lane LDS addresses ------------------------------
// A kernel that walks a ring of LDS stages keeps, per lane, the address of
// each of its operand reads as an LDS pointer (stage base included) and
// advances it once per step; the compile-time part of an address (row group,
// k-chunk) lands in the instruction's offset field.
typedef __attribute__((address_space(3))) char lds_char;
__device__ __forceinline__ const lds_char* lds_ptr(const void* p) {
    return (const lds_char*)((__attribute__((address_space(3))) const void*)(p));
}
__device__ __forceinline__ u32x4_t lds_ld128(const lds_char* p) {
    return *(const __attribute__((address_space(3))) u32x4_t*)(p);
}
__device__ __forceinline__ f32x4_t lds_ldf4(const lds_char* p) {
    return *(const __attribute__((address_space(3))) f32x4_t*)(p);
}
__device__ __forceinline__ void lds_st128(const lds_char* p, u32x4_t v) {
    *(__attribute__((address_space(3))) u32x4_t*)(const_cast<lds_char*>(p)) = v;
}
__device__ __forceinline__ u32x2_t lds_ld_tr16(const lds_char* p) {
    typedef short i16x4_t __attribute__((ext_vector_type(4)));
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(p));
    return __builtin_bit_cast(u32x2_t, v);
}
// Per-lane byte offsets inside a swizzled, swap23-staged tile of D-element rows:
//   row_read_off: the A-operand read of chunk pair c of LDS row lane%32
//     (elements 16c + 8*(lane/32) .. +7), as row_operand_swz reads it;
//   tr_read_off: the lo (hi = 0) or hi (hi = 1) transposing read of the
//     B operand of column group dt, as b_operand_tr_swz reads it at row32 = 0,
//     cc = 0.
// The swizzle repeats every 16 rows, so rows 16k further on add 32 * k * D
// bytes: a compile-time offset.
template <int D>
__device__ __forceinline__ uint32_t row_read_off(int lane, int c) {
    return 2u * uint32_t(swz_off<D>(lane & 31, 16 * c + 8 * (lane >> 5)));
}
template <int D>
__device__ __forceinline__ uint32_t tr_read_off(int lane, int dt, int hi) {
    const int L = lane & 15;
    const int g = lane >> 4;
    const int row = 4 * (g >> 1) + (L >> 2) + 8 * hi;
    const int col = 32 * dt + 16 * (g & 1) + 4 * (L & 3);
    return 2u * uint32_t(swz_off<D>(row, col));
}

// Direct global->LDS copies issued as inline assembly: lane L reads the bytes
// at base + off (base a wave-uniform pointer, off a per-lane byte offset) and
// they land at LDS byte address lds + 16 * L (dwordx4) or lds + 4 * L (dword).
// The compiler does not track these loads, so it never delays LDS reads of
// other buffers behind them; the caller makes a tile visible with
// wait_vmcnt<0>() and a workgroup barrier before reading it.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return uint32_t(uintptr_t((__attribute__((address_space(3))) const void*)(p)));
}
// A wave-uniform value that the compiler may hold in a VGPR, moved to SGPRs
// (the base address and LDS address operands below must be scalar).
__device__ __forceinline__ const void* scalar_ptr(const void* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
    return reinterpret_cast<const void*>((uint64_t(hi) << 32) | lo);
}
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(scalar_ptr(base))
                 : "memory");
}
// The same with the non-temporal hint, for data read exactly once (keeps it
// from displacing reused tiles in L2).
__device__ __forceinline__ void dma16_nt(const void* base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(scalar_ptr(base))
                 : "memory");
}
// dma16 to LDS address lds + IMM, the sum formed in m0 next to the load: a
// run of loads into one tile then keeps only lds live in a scalar register
template <int IMM>
__device__ __forceinline__ void dma16_imm(const void* base, uint32_t off, uint32_t lds) {
    asm volatile("s_add_u32 m0, %0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(scalar_ptr(base)), "i"(IMM)
                 : "memory", "scc");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(off), "s"(scalar_ptr(base))
                 : "memory");
}

// Work item of a workgroup, chosen so each XCD walks a contiguous range of
// the item list.  Workgroups are dispatched to the 8 XCDs round-robin
// (workgroup i to XCD i % 8); giving XCD x the items [x * per, (x + 1) * per)
// in order makes the workgroups an XCD runs at one time neighbours in the
// list, which share their operand tiles in that XCD's L2.  The grid has
// 8 * per workgroups; -1 marks the padding ones past the last item.
constexpr int kXcds = 8;
constexpr int kCusPerXcd = 32;
__host__ __device__ inline int xcd_items_per(int n_items) { return (n_items + kXcds - 1) / kXcds; }
__device__ __forceinline__ int xcd_item(int id, int n_items) {
    const int w = (id % kXcds) * xcd_items_per(n_items) + id / kXcds;
    return w < n_items ? w : -1;
}

// s_waitcnt with only the vector-memory counter constrained (<= n outstanding).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// B operand of a 32x32x16 MFMA from a swizzled, swap23-staged tile: logical
// rows 16*cc + 8*h + 0..7 of the 32-row group at `row32`, column col0 + lane%32.
template <int D>
__device__ __forceinline__ bf16x8_t b_operand_tr_swz(const uint16_t* tile, int row32, int cc, int col0,
                                                     int lane) {
    const int L = lane & 15;
    const int g = lane >> 4;
    const int h = g >> 1;
    const int row = row32 + 16 * cc + 4 * h + (L >> 2);
    const int col = col0 + 16 * (g & 1) + 4 * (L & 3);
    const u32x2_t lo = lds_read_tr16(tile + swz_off<D>(row, col));
    const u32x2_t hi = lds_read_tr16(tile + swz_off<D>(row + 8, col));
    const u32x4_t v = {lo[0], lo[1], hi[0], hi[1]};
    return as_bf16x8(v);
}

// A operand (or B operand of the non-transposed kind) of a 32x32x16 MFMA:
// 8 consecutive elements of LDS row `row` starting at a multiple of 8.
template <int D>
__device__ __forceinline__ bf16x8_t row_operand_swz(const uint16_t* tile, int row, int col) {
    return as_bf16x8(lds_read128(tile + swz_off<D>(row, col)));
}

}  // namespace isattn
