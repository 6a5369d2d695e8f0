// Host-side launchers of the HIP kernels (one translation unit each).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bwd_args.hpp"

namespace isattn {

// LoopK / LoopQ: delta = rowsum(dO * O) and zeroing of the fp32 accumulators of `algo`.
hipError_t launch_preprocess(const BwdArgs& a, int algo, hipStream_t s);
// fp32 accumulators -> bf16 outputs (x softmax_scale for dK / dQ).
hipError_t launch_postprocess(const BwdArgs& a, int algo, hipStream_t s);
// Main loops.
hipError_t launch_loopk(const BwdArgs& a, hipStream_t s);
hipError_t launch_loopq(const BwdArgs& a, hipStream_t s);
// Atomic-free two-pass backward: dK/dV pass (key-outer), dQ pass (query-outer).
// Attention forward: O and LSE.
hipError_t launch_attn_fwd(const FwdArgs& a, hipStream_t s);
// Set-up of the two-pass backward, before either pass: the work order of
// both (into a.order); for SPLIT_DS with a block CSR the K->Q position of
// every Q->K entry (a.ds_map) and the overflow flag; with `delta` the delta
// rows (negated, as the dK/dV pass reads them) and the lse2 rows.  One launch.
hipError_t launch_split_setup(const BwdArgs& a, bool delta, hipStream_t s);
hipError_t launch_split_dkdv(const BwdArgs& a, hipStream_t s);
hipError_t launch_split_dq(const BwdArgs& a, hipStream_t s);
// SPLIT_DS second pass: dQ from the dS tiles the dK/dV pass stored.
hipError_t launch_split_ds_dq(const BwdArgs& a, hipStream_t s);

// Token indices -> presence rows [B, nhk, n_qb, n_kb] (+ per-row counts).
// Top-k positions per score row within [starts[r], ends[r]) (full rows when
// null), ordered by score (ties: smaller position first), -1 padded.
hipError_t launch_topk(const float* scores, int64_t ld, int32_t rows, int32_t n, const int32_t* starts,
                       const int32_t* ends, int32_t topk, int32_t* out, hipStream_t s);
// Token-exact bits of the index rows (slots of 1024 words per block, see the
// token_bits layout of the C ABI); cu_q / cu_k as below.
hipError_t launch_index_token_bits(const int32_t* idx, const int32_t* cu_q, const int32_t* cu_k, int32_t B,
                                   int32_t Sq, int32_t Sk, int32_t nhk, int32_t topk, int32_t n_qb,
                                   int32_t n_kb, uint32_t* bits, hipStream_t s);
// Packed sequences: cu_q / cu_k (else null) give each sequence's rows and
// length; Sq, Sk are then the longest lengths.
hipError_t launch_index_presence(const int32_t* idx, const int32_t* cu_q, const int32_t* cu_k, int32_t B,
                                 int32_t Sq, int32_t Sk, int32_t nhk, int32_t topk, int32_t bq, int32_t bk,
                                 int32_t n_qb, int32_t n_kb, uint8_t* presence, int32_t* qcnt,
                                 hipStream_t s);
// Presence -> Q->K and K->Q CSR.  Row counts are computed here unless
// `have_row_counts` (the index path produces them with the presence rows).
hipError_t launch_presence_to_csr(const uint8_t* presence, int32_t BH, int32_t n_qb,
                                  int32_t n_kb, bool have_row_counts, int32_t* qcnt,
                                  int32_t* kcnt, int32_t* q2k_ptr, int32_t* q2k_col,
                                  int32_t* k2q_ptr, int32_t* k2q_col, hipStream_t s);

}  // namespace isattn
