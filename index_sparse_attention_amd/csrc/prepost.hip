// Preprocess and postprocess of the attention backward.
//
// Preprocess of LoopK and LoopQ: the delta rows (delta[b, h, i] = sum_d
// dO[b,i,h,d] * O[b,i,h,d], fp32 sum of exact bf16 products, padded to
// whole 128-row blocks with 0; delta_rows in pre_rows.hpp) plus zeroing of
// the fp32 accumulators the main loop reduces into (dK/dV for LoopK, dQ for
// LoopQ).  The zeroing is a plain fill kernel, not a memset node, so the
// whole call can be graph-captured.  (SPLIT_DS runs the same delta rows, with
// lse2, inside its set-up launch; SPLIT computes delta in its dQ pass.)
//
// Postprocess: fp32 accumulator -> bf16 output (round to nearest even), times
// softmax_scale for dK and dQ.  MagiAttention PR #334, Core changes item 3:
// the LoopK path always takes this fp32-accumulate-then-convert-and-scale
// step for dK/dV.
//
// Both kernels are HBM-bound streaming passes: 16-byte loads/stores, one row
// segment per lane group, rows in memory order.
#include "device_common.hpp"
#include "kernels.hpp"
#include "pre_rows.hpp"

namespace isattn {
namespace {

constexpr int kThreads = 256;

template <int DV>
__global__ __launch_bounds__(kThreads) void k_preprocess(BwdArgs a, int32_t nblk_delta, int64_t n4_0,
                                                         int64_t n4_1) {
    if (int32_t(blockIdx.x) < nblk_delta) {
        delta_rows<DV, kThreads>(a, blockIdx.x);
    } else {
        const int64_t n4 = n4_0 + n4_1;
        const int64_t stride = int64_t(gridDim.x - nblk_delta) * kThreads;
        for (int64_t u = int64_t(blockIdx.x - nblk_delta) * kThreads + threadIdx.x; u < n4; u += stride) {
            float4* p = u < n4_0 ? reinterpret_cast<float4*>(a.acc0) + u
                                 : reinterpret_cast<float4*>(a.acc1) + (u - n4_0);
            *p = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
}

template <int D>
__global__ __launch_bounds__(kThreads) void k_postprocess(const float* __restrict__ acc,
                                                          uint16_t* __restrict__ out, int64_t sb,
                                                          int64_t ss, int64_t sh, int32_t S, int32_t H,
                                                          int64_t rows, float mul) {
    constexpr int L = D / 8;
    const int64_t u = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    const int64_t row = u / L;
    const int sub = int(u % L);
    if (row >= rows) return;
    const int64_t s = row % S;          // accumulator rows are head-major (b, h, s)
    const int64_t t = row / S;
    const int64_t h = t % H;
    const int64_t b = t / H;
    const float4* src = reinterpret_cast<const float4*>(acc + row * D + 8 * sub);
    const float4 x = src[0];
    const float4 y = src[1];
    u32x4_t w;
    w[0] = pack_bf16x2(x.x * mul, x.y * mul);
    w[1] = pack_bf16x2(x.z * mul, x.w * mul);
    w[2] = pack_bf16x2(y.x * mul, y.y * mul);
    w[3] = pack_bf16x2(y.z * mul, y.w * mul);
    *reinterpret_cast<u32x4_t*>(out + b * sb + s * ss + h * sh + 8 * sub) = w;
}

template <int D>
hipError_t post_one(const float* acc, uint16_t* out, int64_t sb, int64_t ss, int64_t sh, int32_t B,
                    int32_t S, int32_t H, float mul, hipStream_t st) {
    const int64_t rows = int64_t(B) * S * H;
    const int64_t threads = rows * (D / 8);
    if (threads == 0) return hipSuccess;
    const int64_t blocks = (threads + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(k_postprocess<D>, dim3(unsigned(blocks)), dim3(kThreads), 0, st, acc, out, sb, ss,
                       sh, S, H, rows, mul);
    return hipGetLastError();
}

hipError_t post_dispatch(int D, const float* acc, uint16_t* out, int64_t sb, int64_t ss, int64_t sh,
                         int32_t B, int32_t S, int32_t H, float mul, hipStream_t st) {
    switch (D) {
        case 64: return post_one<64>(acc, out, sb, ss, sh, B, S, H, mul, st);
        case 128: return post_one<128>(acc, out, sb, ss, sh, B, S, H, mul, st);
        case 192: return post_one<192>(acc, out, sb, ss, sh, B, S, H, mul, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_preprocess(const BwdArgs& a, int algo, hipStream_t s) {
    (void)algo;
    const int64_t rows = int64_t(a.B) * a.Hq * a.stat_ld;
    const int rpb = a.Dv == 64 ? delta_rows_per_block<64, kThreads>() : delta_rows_per_block<128, kThreads>();
    const int32_t nblk_delta = int32_t((rows + rpb - 1) / rpb);
    const int64_t n4_0 = a.acc0_elems / 4;
    const int64_t n4_1 = a.acc1_elems / 4;
    const int64_t nz64 = (n4_0 + n4_1 + kThreads - 1) / kThreads;
    const int32_t nz = int32_t(nz64 < 8192 ? nz64 : 8192);
    const int32_t grid = nblk_delta + nz;
    if (grid == 0) return hipSuccess;
    switch (a.Dv) {
        case 64:
            hipLaunchKernelGGL(k_preprocess<64>, dim3(grid), dim3(kThreads), 0, s, a, nblk_delta, n4_0, n4_1);
            break;
        case 128:
            hipLaunchKernelGGL(k_preprocess<128>, dim3(grid), dim3(kThreads), 0, s, a, nblk_delta, n4_0, n4_1);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_postprocess(const BwdArgs& a, int algo, hipStream_t s) {
    if (algo == 2 || algo == 3) return hipSuccess;   // SPLIT and SPLIT_DS store bf16 outputs directly
    if (algo == 0) {
        hipError_t e = post_dispatch(a.Dqk, a.acc0, a.dk, a.dk_sb, a.dk_ss, a.dk_sh, a.B, a.Sk, a.Hk,
                                     a.scale, s);
        if (e != hipSuccess) return e;
        return post_dispatch(a.Dv, a.acc1, a.dv, a.dv_sb, a.dv_ss, a.dv_sh, a.B, a.Sk, a.Hk, 1.0f, s);
    }
    return post_dispatch(a.Dqk, a.acc0, a.dq, a.dq_sb, a.dq_ss, a.dq_sh, a.B, a.Sq, a.Hq, a.scale, s);
}

}  // namespace isattn
