// Host-side argument checking and workspace planning for the C ABI.
// HIP-free on purpose: every rule here can be exercised on a machine without
// a GPU, and a failed check means nothing was enqueued.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/isattn.h"
#include "bwd_args.hpp"

namespace isattn {

constexpr size_t kWsAlign = 256;

// The SPLIT dK/dV pass addresses the rows of one (batch, head) slice of Q and
// dO by 32-bit byte offsets from the slice's first row: n_qb * 128 rows times
// the sequence stride must stay below 2^31 bytes.

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int32_t cdiv(int32_t a, int32_t b) { return (a + b - 1) / b; }

struct BwdPlan {
    int32_t n_qb, n_kb, G, Hm, stat_ld;
    size_t off_delta, off_lse2, off_order, off_units, off_info, off_partial, off_acc0, off_acc1, off_dsmap, off_ds,
        total;
    int32_t kv_parts_T, kv_units_bound;
    int64_t acc0_elems, acc1_elems;
    // SPLIT_DS: dS tiles the mask needs (the part from off_ds on), tiles per
    // (b, h) of a dense mask, length of the Q->K -> K->Q position map
    int64_t ds_tiles, ds_T, ds_map_len;
};

// What the workspace plan knows of the mask.  kind < 0: nothing (every
// block of every head, a position map for heads_q mask heads).
struct MaskInfo {
    int32_t kind = -1;      // ISATTN_MASK_DENSE, ISATTN_MASK_BLOCK_CSR, or -1
    int32_t heads = 0;      // mask heads of a block CSR
    int64_t nnz = -1;       // blocks of a block CSR, < 0 if unknown
    bool causal = false;
    bool varlen = false;
};

// Workspace layout for isattn_attn_bwd; false if the shape or algo is unusable.
// allow_parts = false keeps SPLIT's dK/dV pass at one workgroup per item
// (no fp32 partial slots), whatever the item count.
bool plan_bwd_workspace(const isattn_shape_t& s, int32_t algo, BwdPlan* plan, const MaskInfo& mask = MaskInfo{},
                        bool allow_parts = true);

// Full argument check.  On success fills `args` (all but the workspace
// pointers, which the caller carves from `plan`) and `plan`.
isattn_status_t validate_bwd(const isattn_shape_t* shape, const isattn_tensor_t* q,
                             const isattn_tensor_t* k, const isattn_tensor_t* v,
                             const isattn_tensor_t* o, const isattn_tensor_t* dO,
                             const float* lse, const isattn_mask_t* mask, int32_t causal,
                             float softmax_scale, const isattn_tensor_t* dq,
                             const isattn_tensor_t* dk, const isattn_tensor_t* dv, int32_t algo,
                             const void* workspace, size_t workspace_bytes, BwdArgs* args,
                             BwdPlan* plan, const isattn_varlen_t* varlen = nullptr, bool allow_parts = true);

// Argument check of the forward; on success fills `args`.
isattn_status_t validate_fwd(const isattn_shape_t* shape, const isattn_tensor_t* q,
                             const isattn_tensor_t* k, const isattn_tensor_t* v,
                             const isattn_mask_t* mask, int32_t causal, float softmax_scale,
                             const isattn_tensor_t* o, const float* lse, FwdArgs* args,
                             const isattn_varlen_t* varlen = nullptr);

struct CsrPlan {
    int32_t rows_q, rows_k;       // B*H*n_qb, B*H*n_kb
    size_t off_presence, off_qcnt, off_kcnt, total;
};

// Workspace layout of the converter; presence part omitted when the caller
// supplies the presence matrix (block-mask path).
bool plan_csr_workspace(int64_t batch, int64_t heads, int64_t n_qb, int64_t n_kb,
                        bool with_presence, CsrPlan* plan);

isattn_status_t validate_index(const int32_t* indices, int32_t batch, int32_t seqlen_q,
                               int32_t seqlen_k, int32_t nhk, int32_t topk, int32_t block_q,
                               int32_t block_k, const int32_t* q2k_row_ptr, const int32_t* q2k_col,
                               const int32_t* k2q_row_ptr, const int32_t* k2q_col,
                               int64_t col_capacity, const void* workspace,
                               size_t workspace_bytes, CsrPlan* plan);

isattn_status_t validate_blockmask(const uint8_t* presence, int32_t batch, int32_t heads,
                                   int32_t n_qb, int32_t n_kb, const int32_t* q2k_row_ptr,
                                   const int32_t* q2k_col, const int32_t* k2q_row_ptr,
                                   const int32_t* k2q_col, int64_t col_capacity,
                                   const void* workspace, size_t workspace_bytes, CsrPlan* plan);

// Largest key-block count the converter's on-chip bitmap holds.
constexpr int32_t kMaxKeyBlocks = 1 << 19;

}  // namespace isattn
