// extern "C" entry points of libisattn.so (declared in include/isattn.h).
// Validation is in validate.cpp (HIP-free); this file carves workspaces and
// enqueues the kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <mutex>
#include <new>
#include <vector>

#include "../../include/isattn.h"
#include "kernels.hpp"
#include "validate.hpp"

// Scratch of isattn_attn_bwd_noalloc: the workspace of its SPLIT call, a
// static device array of ISATTN_NOALLOC_SCRATCH_BYTES that every GPU the
// library runs on holds from the first such call until the process ends.
// Host code never uses its name as an address: each device's copy is looked
// up once with hipGetSymbolAddress (scratch_address below) and that pointer
// is what the kernels receive.
static __device__ __align__(256) unsigned char scratch[ISATTN_NOALLOC_SCRATCH_BYTES];

struct isattn_timer {
    int32_t capacity = 0;
    int32_t recorded = 0;      // calls recorded since the last reset (may exceed capacity)
    std::vector<hipEvent_t> ev;  // kTimerEvents per slot
};

namespace {

using namespace isattn;

constexpr int kTimerEvents = 5;   // boundaries of the 4 stages

inline char* ws_at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

isattn_status_t record(isattn_timer_t* t, int slot, int k, hipStream_t s) {
    if (t == nullptr) return ISATTN_OK;
    return hipEventRecord(t->ev[size_t(slot) * kTimerEvents + k], s) == hipSuccess ? ISATTN_OK : ISATTN_ERR_HIP;
}

// Address of the current device's copy of `scratch`, looked up on the
// device's first call (with that device current) and kept per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

isattn_status_t scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ISATTN_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return ISATTN_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return ISATTN_OK;
}

isattn_status_t attn_bwd_impl(const isattn_shape_t* shape, const isattn_tensor_t* q,
                              const isattn_tensor_t* k, const isattn_tensor_t* v,
                              const isattn_tensor_t* o, const isattn_tensor_t* dO, const float* lse,
                              const isattn_mask_t* mask, int32_t causal, float softmax_scale,
                              const isattn_tensor_t* dq, const isattn_tensor_t* dk,
                              const isattn_tensor_t* dv, int32_t algo, void* workspace,
                              size_t workspace_bytes, void* stream, isattn_timer_t* timer,
                              const isattn_varlen_t* varlen = nullptr, bool allow_parts = true) {
    BwdArgs a{};
    BwdPlan plan{};
    isattn_status_t st = validate_bwd(shape, q, k, v, o, dO, lse, mask, causal, softmax_scale, dq, dk,
                                      dv, algo, workspace, workspace_bytes, &a, &plan, varlen, allow_parts);
    if (st != ISATTN_OK) return st;
    if (a.B == 0) return ISATTN_OK;
    a.delta = reinterpret_cast<float*>(ws_at(workspace, plan.off_delta));
    const bool split = algo == ISATTN_ALGO_SPLIT || algo == ISATTN_ALGO_SPLIT_DS;
    a.lse2 = split ? reinterpret_cast<float*>(ws_at(workspace, plan.off_lse2)) : nullptr;
    a.order = split ? reinterpret_cast<int32_t*>(ws_at(workspace, plan.off_order)) : nullptr;
    a.ds = algo == ISATTN_ALGO_SPLIT_DS ? reinterpret_cast<uint16_t*>(ws_at(workspace, plan.off_ds)) : nullptr;
    if (algo == ISATTN_ALGO_SPLIT_DS && a.mask_kind == ISATTN_MASK_BLOCK_CSR) {
        a.ds_map = reinterpret_cast<int32_t*>(ws_at(workspace, plan.off_dsmap));
        a.ds_flag = a.ds_map + plan.ds_map_len;
    }
    a.kv_parts_T = plan.kv_parts_T;
    a.kv_units_bound = plan.kv_units_bound;
    a.units = plan.kv_parts_T > 0 ? reinterpret_cast<int32_t*>(ws_at(workspace, plan.off_units)) : nullptr;
    a.item_info = plan.kv_parts_T > 0 ? reinterpret_cast<int32_t*>(ws_at(workspace, plan.off_info)) : nullptr;
    a.partial = plan.kv_parts_T > 0 ? reinterpret_cast<float*>(ws_at(workspace, plan.off_partial)) : nullptr;
    a.acc0 = reinterpret_cast<float*>(ws_at(workspace, plan.off_acc0));
    a.acc1 = reinterpret_cast<float*>(ws_at(workspace, plan.off_acc1));
    hipStream_t s = static_cast<hipStream_t>(stream);
    int slot = 0;
    if (timer != nullptr) slot = timer->recorded % timer->capacity;

    if ((st = record(timer, slot, 0, s)) != ISATTN_OK) return st;
    // LoopK / LoopQ: delta rows and zeroed accumulators.  SPLIT and SPLIT_DS:
    // one set-up launch (work order; for SPLIT_DS also the delta and lse2
    // rows and, with a block CSR, the dS position map).  SPLIT computes delta
    // and lse2 in its dQ pass, which runs first.
    if (!split && launch_preprocess(a, algo, s) != hipSuccess) return ISATTN_ERR_HIP;
    if (split && launch_split_setup(a, algo == ISATTN_ALGO_SPLIT_DS, s) != hipSuccess) return ISATTN_ERR_HIP;
    if ((st = record(timer, slot, 1, s)) != ISATTN_OK) return st;
    hipError_t e;
    if (algo == ISATTN_ALGO_LOOPK) e = launch_loopk(a, s);
    else if (algo == ISATTN_ALGO_LOOPQ) e = launch_loopq(a, s);
    else if (algo == ISATTN_ALGO_SPLIT) e = launch_split_dq(a, s);
    else e = launch_split_dkdv(a, s);                // SPLIT_DS: dK/dV pass first, storing dS
    if (e != hipSuccess) return ISATTN_ERR_HIP;
    if ((st = record(timer, slot, 2, s)) != ISATTN_OK) return st;
    if (algo == ISATTN_ALGO_SPLIT) e = launch_split_dkdv(a, s);
    else if (algo == ISATTN_ALGO_SPLIT_DS) e = launch_split_ds_dq(a, s);
    if (e != hipSuccess) return ISATTN_ERR_HIP;
    if ((st = record(timer, slot, 3, s)) != ISATTN_OK) return st;
    if (launch_postprocess(a, algo, s) != hipSuccess) return ISATTN_ERR_HIP;
    if ((st = record(timer, slot, 4, s)) != ISATTN_OK) return st;
    if (timer != nullptr) timer->recorded++;
    return ISATTN_OK;
}

}  // namespace

extern "C" {

size_t isattn_attn_bwd_workspace_bytes(const isattn_shape_t* shape, int32_t algo) {
    if (shape == nullptr) return 0;
    BwdPlan p{};
    if (!plan_bwd_workspace(*shape, algo, &p)) return 0;
    return p.total;
}

size_t isattn_attn_bwd_workspace_bytes_mask(const isattn_shape_t* shape, int32_t algo, const isattn_mask_t* mask,
                                            int32_t causal, int32_t varlen) {
    if (shape == nullptr) return 0;
    MaskInfo mi;
    mi.kind = ISATTN_MASK_DENSE;
    if (mask != nullptr && mask->kind == ISATTN_MASK_BLOCK_CSR) {
        mi.kind = ISATTN_MASK_BLOCK_CSR;
        mi.heads = mask->heads;
        mi.nnz = mask->nnz;
    } else if (mask != nullptr && mask->kind != ISATTN_MASK_DENSE) {
        return 0;
    }
    if (mi.kind == ISATTN_MASK_BLOCK_CSR && (mi.heads < 1 || shape->heads_q % mi.heads != 0)) return 0;
    mi.causal = causal != 0;
    mi.varlen = varlen != 0;
    BwdPlan p{};
    if (!plan_bwd_workspace(*shape, algo, &p, mi)) return 0;
    return p.total;
}

isattn_status_t isattn_attn_bwd(const isattn_shape_t* shape, const isattn_tensor_t* q,
                                const isattn_tensor_t* k, const isattn_tensor_t* v,
                                const isattn_tensor_t* o, const isattn_tensor_t* dO, const float* lse,
                                const isattn_mask_t* mask_desc, int32_t causal, float softmax_scale,
                                const isattn_tensor_t* dq, const isattn_tensor_t* dk,
                                const isattn_tensor_t* dv, int32_t algo, void* workspace,
                                size_t workspace_bytes, void* stream) {
    return attn_bwd_impl(shape, q, k, v, o, dO, lse, mask_desc, causal, softmax_scale, dq, dk, dv, algo,
                         workspace, workspace_bytes, stream, nullptr);
}

isattn_status_t isattn_attn_bwd_noalloc(const isattn_shape_t* shape, const isattn_tensor_t* q,
                                        const isattn_tensor_t* k, const isattn_tensor_t* v,
                                        const isattn_tensor_t* o, const isattn_tensor_t* dO, const float* lse,
                                        const isattn_mask_t* mask_desc, int32_t causal, float softmax_scale,
                                        const isattn_tensor_t* dq, const isattn_tensor_t* dk,
                                        const isattn_tensor_t* dv, void* stream) {
    // the size check needs no device: SPLIT's workspace without part mode
    if (shape != nullptr) {
        BwdPlan p{};
        if (plan_bwd_workspace(*shape, ISATTN_ALGO_SPLIT, &p, MaskInfo{}, false) &&
            p.total > size_t(ISATTN_NOALLOC_SCRATCH_BYTES))
            return ISATTN_ERR_SCRATCH;
    }
    void* ws = nullptr;
    isattn_status_t st = scratch_address(&ws);
    if (st != ISATTN_OK) return st;
    st = attn_bwd_impl(shape, q, k, v, o, dO, lse, mask_desc, causal, softmax_scale, dq, dk, dv, ISATTN_ALGO_SPLIT,
                       ws, ISATTN_NOALLOC_SCRATCH_BYTES, stream, nullptr, nullptr, false);
    return st == ISATTN_ERR_WORKSPACE ? ISATTN_ERR_SCRATCH : st;
}

isattn_status_t isattn_attn_bwd_varlen(const isattn_shape_t* shape, const isattn_varlen_t* varlen,
                                       const isattn_tensor_t* q, const isattn_tensor_t* k,
                                       const isattn_tensor_t* v, const isattn_tensor_t* o,
                                       const isattn_tensor_t* dO, const float* lse,
                                       const isattn_mask_t* mask_desc, int32_t causal,
                                       float softmax_scale, const isattn_tensor_t* dq,
                                       const isattn_tensor_t* dk, const isattn_tensor_t* dv,
                                       int32_t algo, void* workspace, size_t workspace_bytes,
                                       void* stream) {
    if (varlen == nullptr) return ISATTN_ERR_NULL;
    return attn_bwd_impl(shape, q, k, v, o, dO, lse, mask_desc, causal, softmax_scale, dq, dk, dv, algo,
                         workspace, workspace_bytes, stream, nullptr, varlen);
}

static isattn_status_t attn_fwd_impl(const isattn_shape_t* shape, const isattn_tensor_t* q,
                                     const isattn_tensor_t* k, const isattn_tensor_t* v,
                                     const isattn_mask_t* mask_desc, int32_t causal, float softmax_scale,
                                     const isattn_tensor_t* o, float* lse, void* stream,
                                     const isattn_varlen_t* varlen) {
    FwdArgs a{};
    const isattn_status_t st =
        validate_fwd(shape, q, k, v, mask_desc, causal, softmax_scale, o, lse, &a, varlen);
    if (st != ISATTN_OK) return st;
    if (a.B == 0) return ISATTN_OK;
    return launch_attn_fwd(a, static_cast<hipStream_t>(stream)) == hipSuccess ? ISATTN_OK : ISATTN_ERR_HIP;
}

isattn_status_t isattn_attn_fwd(const isattn_shape_t* shape, const isattn_tensor_t* q,
                                const isattn_tensor_t* k, const isattn_tensor_t* v,
                                const isattn_mask_t* mask_desc, int32_t causal, float softmax_scale,
                                const isattn_tensor_t* o, float* lse, void* stream) {
    return attn_fwd_impl(shape, q, k, v, mask_desc, causal, softmax_scale, o, lse, stream, nullptr);
}

isattn_status_t isattn_attn_fwd_varlen(const isattn_shape_t* shape, const isattn_varlen_t* varlen,
                                       const isattn_tensor_t* q, const isattn_tensor_t* k,
                                       const isattn_tensor_t* v, const isattn_mask_t* mask_desc,
                                       int32_t causal, float softmax_scale,
                                       const isattn_tensor_t* o, float* lse, void* stream) {
    if (varlen == nullptr) return ISATTN_ERR_NULL;
    return attn_fwd_impl(shape, q, k, v, mask_desc, causal, softmax_scale, o, lse, stream, varlen);
}

isattn_status_t isattn_attn_bwd_timed(const isattn_shape_t* shape, const isattn_tensor_t* q,
                                      const isattn_tensor_t* k, const isattn_tensor_t* v,
                                      const isattn_tensor_t* o, const isattn_tensor_t* dO,
                                      const float* lse, const isattn_mask_t* mask_desc, int32_t causal,
                                      float softmax_scale, const isattn_tensor_t* dq,
                                      const isattn_tensor_t* dk, const isattn_tensor_t* dv,
                                      int32_t algo, void* workspace, size_t workspace_bytes,
                                      void* stream, isattn_timer_t* timer) {
    return attn_bwd_impl(shape, q, k, v, o, dO, lse, mask_desc, causal, softmax_scale, dq, dk, dv, algo,
                         workspace, workspace_bytes, stream, timer);
}

size_t isattn_index_to_block_sparse_workspace_bytes(int32_t batch, int32_t seqlen_q, int32_t seqlen_k,
                                                    int32_t nhk, int32_t block_q, int32_t block_k) {
    if (block_q < 1 || block_k < 1 || seqlen_q < 0 || seqlen_k < 0) return 0;
    CsrPlan p{};
    if (!plan_csr_workspace(batch, nhk, cdiv(seqlen_q, block_q), cdiv(seqlen_k, block_k), true, &p))
        return 0;
    return p.total;
}

static isattn_status_t index_to_block_sparse_impl(const int32_t* indices, int32_t batch,
                                                  const int32_t* cu_q, const int32_t* cu_k, int32_t seqlen_q,
                                                  int32_t seqlen_k, int32_t nhk, int32_t topk,
                                                  int32_t block_q, int32_t block_k, int32_t* q2k_row_ptr,
                                                  int32_t* q2k_col, int32_t* k2q_row_ptr, int32_t* k2q_col,
                                                  int64_t col_capacity, void* workspace,
                                                  size_t workspace_bytes, void* stream) {
    CsrPlan p{};
    isattn_status_t st = validate_index(indices, batch, seqlen_q, seqlen_k, nhk, topk, block_q, block_k,
                                        q2k_row_ptr, q2k_col, k2q_row_ptr, k2q_col, col_capacity,
                                        workspace, workspace_bytes, &p);
    if (st != ISATTN_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int32_t n_qb = cdiv(seqlen_q, block_q);
    const int32_t n_kb = cdiv(seqlen_k, block_k);
    uint8_t* presence = reinterpret_cast<uint8_t*>(ws_at(workspace, p.off_presence));
    int32_t* qcnt = reinterpret_cast<int32_t*>(ws_at(workspace, p.off_qcnt));
    int32_t* kcnt = reinterpret_cast<int32_t*>(ws_at(workspace, p.off_kcnt));
    if (launch_index_presence(indices, cu_q, cu_k, batch, seqlen_q, seqlen_k, nhk, topk, block_q, block_k,
                              n_qb, n_kb, presence, qcnt, s) != hipSuccess)
        return ISATTN_ERR_HIP;
    if (launch_presence_to_csr(presence, batch * nhk, n_qb, n_kb, true, qcnt, kcnt, q2k_row_ptr, q2k_col,
                               k2q_row_ptr, k2q_col, s) != hipSuccess)
        return ISATTN_ERR_HIP;
    return ISATTN_OK;
}

isattn_status_t isattn_index_to_block_sparse(const int32_t* indices, int32_t batch, int32_t seqlen_q,
                                             int32_t seqlen_k, int32_t nhk, int32_t topk,
                                             int32_t block_q, int32_t block_k, int32_t* q2k_row_ptr,
                                             int32_t* q2k_col, int32_t* k2q_row_ptr, int32_t* k2q_col,
                                             int64_t col_capacity, void* workspace,
                                             size_t workspace_bytes, void* stream) {
    return index_to_block_sparse_impl(indices, batch, nullptr, nullptr, seqlen_q, seqlen_k, nhk, topk, block_q,
                                      block_k, q2k_row_ptr, q2k_col, k2q_row_ptr, k2q_col, col_capacity,
                                      workspace, workspace_bytes, stream);
}

isattn_status_t isattn_index_to_block_sparse_varlen(const int32_t* indices, int32_t batch,
                                                    const int32_t* cu_seqlens_q,
                                                    const int32_t* cu_seqlens_k, int32_t max_seqlen_q,
                                                    int32_t max_seqlen_k, int32_t nhk, int32_t topk,
                                                    int32_t block_q, int32_t block_k,
                                                    int32_t* q2k_row_ptr, int32_t* q2k_col,
                                                    int32_t* k2q_row_ptr, int32_t* k2q_col,
                                                    int64_t col_capacity, void* workspace,
                                                    size_t workspace_bytes, void* stream) {
    if (batch > 0 && (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr)) return ISATTN_ERR_NULL;
    return index_to_block_sparse_impl(indices, batch, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                                      nhk, topk, block_q, block_k, q2k_row_ptr, q2k_col, k2q_row_ptr,
                                      k2q_col, col_capacity, workspace, workspace_bytes, stream);
}

isattn_status_t isattn_topk_select(const float* scores, int64_t ld, int32_t rows, int32_t n,
                                   const int32_t* starts, const int32_t* ends, int32_t topk,
                                   int32_t* out, void* stream) {
    if (rows < 0 || n < 0 || topk < 0 || ld < n) return ISATTN_ERR_SHAPE;
    if (topk > 8192) return ISATTN_ERR_UNSUPPORTED;
    if ((starts == nullptr) != (ends == nullptr)) return ISATTN_ERR_NULL;
    if (rows == 0 || topk == 0) return ISATTN_OK;
    if (out == nullptr || (n > 0 && scores == nullptr)) return ISATTN_ERR_NULL;
    return launch_topk(scores, ld, rows, n, starts, ends, topk, out, static_cast<hipStream_t>(stream)) == hipSuccess
               ? ISATTN_OK
               : ISATTN_ERR_HIP;
}

isattn_status_t isattn_index_to_token_bits(const int32_t* indices, int32_t batch, int32_t seqlen_q,
                                           int32_t seqlen_k, int32_t nhk, int32_t topk,
                                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                           uint32_t* bits, int64_t bits_words, void* stream) {
    if (batch < 0 || seqlen_q < 0 || seqlen_k < 0 || nhk < 0 || topk < 0) return ISATTN_ERR_SHAPE;
    if (seqlen_q >= (1 << 30) || seqlen_k >= (1 << 30)) return ISATTN_ERR_SHAPE;
    if ((cu_seqlens_q == nullptr) != (cu_seqlens_k == nullptr)) return ISATTN_ERR_NULL;
    const int32_t n_qb = cdiv(seqlen_q, kBlock), n_kb = cdiv(seqlen_k, kBlock);
    const int64_t need = int64_t(batch) * nhk * n_qb * n_kb * 1024;
    if (need == 0) return ISATTN_OK;
    if (nhk > 65535 || batch > 65535) return ISATTN_ERR_SHAPE;   // grid (n_qb, nhk, batch)
    if (bits == nullptr || (seqlen_q > 0 && topk > 0 && indices == nullptr)) return ISATTN_ERR_NULL;
    if (bits_words < need) return ISATTN_ERR_CAPACITY;
    if ((reinterpret_cast<uintptr_t>(bits) & 15u) != 0) return ISATTN_ERR_STRIDE_ALIGN;
    return launch_index_token_bits(indices, cu_seqlens_q, cu_seqlens_k, batch, seqlen_q, seqlen_k, nhk, topk,
                                   n_qb, n_kb, bits, static_cast<hipStream_t>(stream)) == hipSuccess
               ? ISATTN_OK
               : ISATTN_ERR_HIP;
}

size_t isattn_block_mask_to_csr_workspace_bytes(int32_t batch, int32_t heads, int32_t n_qb,
                                                int32_t n_kb) {
    CsrPlan p{};
    if (!plan_csr_workspace(batch, heads, n_qb, n_kb, false, &p)) return 0;
    return p.total;
}

isattn_status_t isattn_block_mask_to_csr(const uint8_t* presence, int32_t batch, int32_t heads,
                                         int32_t n_qb, int32_t n_kb, int32_t* q2k_row_ptr,
                                         int32_t* q2k_col, int32_t* k2q_row_ptr, int32_t* k2q_col,
                                         int64_t col_capacity, void* workspace, size_t workspace_bytes,
                                         void* stream) {
    CsrPlan p{};
    isattn_status_t st = validate_blockmask(presence, batch, heads, n_qb, n_kb, q2k_row_ptr, q2k_col,
                                            k2q_row_ptr, k2q_col, col_capacity, workspace,
                                            workspace_bytes, &p);
    if (st != ISATTN_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int32_t* qcnt = reinterpret_cast<int32_t*>(ws_at(workspace, p.off_qcnt));
    int32_t* kcnt = reinterpret_cast<int32_t*>(ws_at(workspace, p.off_kcnt));
    if (launch_presence_to_csr(presence, batch * heads, n_qb, n_kb, false, qcnt, kcnt, q2k_row_ptr,
                               q2k_col, k2q_row_ptr, k2q_col, s) != hipSuccess)
        return ISATTN_ERR_HIP;
    return ISATTN_OK;
}

const char* isattn_status_string(isattn_status_t status) {
    switch (status) {
        case ISATTN_OK: return "ok";
        case ISATTN_ERR_NULL: return "required pointer is NULL";
        case ISATTN_ERR_SHAPE: return "invalid or inconsistent sizes";
        case ISATTN_ERR_STRIDE_ALIGN: return "unsupported stride or alignment";
        case ISATTN_ERR_UNSUPPORTED: return "outside the supported set";
        case ISATTN_ERR_MASK: return "malformed mask descriptor";
        case ISATTN_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
        case ISATTN_ERR_CAPACITY: return "CSR column or dS tile capacity too small";
        case ISATTN_ERR_HIP: return "HIP runtime error";
        case ISATTN_ERR_SCRATCH: return "problem needs more than the static no-allocation scratch";
    }
    return "unknown status";
}

const char* isattn_version(void) { return "0.2.0"; }

isattn_status_t isattn_timer_create(int32_t capacity, isattn_timer_t** out) {
    if (out == nullptr) return ISATTN_ERR_NULL;
    *out = nullptr;
    if (capacity < 1) return ISATTN_ERR_SHAPE;
    isattn_timer_t* t = new (std::nothrow) isattn_timer_t();
    if (t == nullptr) return ISATTN_ERR_HIP;
    t->capacity = capacity;
    t->ev.assign(size_t(capacity) * kTimerEvents, nullptr);
    for (auto& e : t->ev) {
        if (hipEventCreate(&e) != hipSuccess) {
            e = nullptr;
            isattn_timer_destroy(t);
            return ISATTN_ERR_HIP;
        }
    }
    *out = t;
    return ISATTN_OK;
}

isattn_status_t isattn_timer_destroy(isattn_timer_t* timer) {
    if (timer == nullptr) return ISATTN_OK;
    for (auto& e : timer->ev)
        if (e != nullptr) (void)hipEventDestroy(e);
    delete timer;
    return ISATTN_OK;
}

isattn_status_t isattn_timer_reset(isattn_timer_t* timer) {
    if (timer == nullptr) return ISATTN_ERR_NULL;
    timer->recorded = 0;
    return ISATTN_OK;
}

isattn_status_t isattn_timer_read(isattn_timer_t* timer, int32_t* n_calls, float* stage_ms) {
    if (timer == nullptr || n_calls == nullptr || stage_ms == nullptr) return ISATTN_ERR_NULL;
    const int32_t n = timer->recorded < timer->capacity ? timer->recorded : timer->capacity;
    for (int k = 0; k < kTimerEvents - 1; ++k) stage_ms[k] = 0.f;
    *n_calls = n;
    for (int32_t i = 0; i < n; ++i) {
        hipEvent_t* ev = &timer->ev[size_t(i) * kTimerEvents];
        if (hipEventSynchronize(ev[kTimerEvents - 1]) != hipSuccess) return ISATTN_ERR_HIP;
        for (int k = 0; k < kTimerEvents - 1; ++k) {
            float ms = 0.f;
            if (hipEventElapsedTime(&ms, ev[k], ev[k + 1]) != hipSuccess) return ISATTN_ERR_HIP;
            stage_ms[k] += ms;
        }
    }
    return ISATTN_OK;
}

}  // extern "C"
