/*
 * isattn -- sparse attention backward for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libisattn.so.  Every pointer argument that names tensor data is a
 * device pointer (HIP global memory) unless stated otherwise; every entry
 * point only enqueues work on the given HIP stream and never synchronises the
 * host.  The library allocates no device memory and holds no state: the
 * caller owns inputs, outputs, CSR arrays and workspaces.  All argument
 * checks run before the first launch -- on any error nothing is enqueued and a
 * status code is returned.  No C++ exception crosses this interface.
 *
 * Sources (web pages, by title and section):
 *  [P1] MagiAttention PR #334 "BWD LoopK with warp-specialized pipeline +
 *       IndexSparse/BlockSparse support": Summary, Core changes 1-3.
 *  [P3] xtuner PR #2096 "Add optional TileLang Top-K selector": Main Changes 1.
 *  [P4] MagiAttention PR #331 "support 192/128 and 256/256 ffa_fa4": Summary,
 *       CSR Tile Mapping.
 */
#ifndef ISATTN_H
#define ISATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum isattn_status {
    ISATTN_OK = 0,
    ISATTN_ERR_NULL = 1,          /* a required pointer is NULL                          */
    ISATTN_ERR_SHAPE = 2,         /* a size is negative or sizes are inconsistent       */
    ISATTN_ERR_STRIDE_ALIGN = 3,  /* a tensor view's stride or alignment is unsupported */
    ISATTN_ERR_UNSUPPORTED = 4,   /* outside the supported set (head dims, block, algo) */
    ISATTN_ERR_MASK = 5,          /* malformed mask descriptor                          */
    ISATTN_ERR_WORKSPACE = 6,     /* workspace missing, too small or misaligned         */
    ISATTN_ERR_CAPACITY = 7,      /* CSR column or dS tile capacity below what is needed */
    ISATTN_ERR_HIP = 8,           /* a HIP runtime call or kernel launch failed         */
    ISATTN_ERR_SCRATCH = 9        /* needs more than the static scratch of _noalloc     */
} isattn_status_t;

/* Problem sizes.  Token-major layout (row = token), as the (total_q, NHK, topk)
 * index tensor of [P1] Core changes 2 implies.  heads_q % heads_k == 0; query
 * head h reads KV head h / (heads_q / heads_k). */
typedef struct isattn_shape {
    int32_t batch, seqlen_q, seqlen_k, heads_q, heads_k, dim_qk, dim_v;
} isattn_shape_t;

/* A 4-D bf16 device tensor [batch, seq, heads, dim] with the last dimension
 * contiguous.  Strides are in elements.  ptr and every stride * 2 bytes must
 * be multiples of 16 bytes. */
typedef struct isattn_tensor {
    void*   ptr;
    int64_t stride_b, stride_s, stride_h;
} isattn_tensor_t;

enum { ISATTN_MASK_DENSE = 0, ISATTN_MASK_BLOCK_CSR = 1 };

/* Mask descriptor.  kind == ISATTN_MASK_DENSE: every pair is kept (before the
 * causal term).  kind == ISATTN_MASK_BLOCK_CSR: a pair (i, j) of query head h
 * is kept iff key block j / block_k is listed in the Q->K CSR row of
 * (batch b, mask head h * heads / heads_q, query block i / block_q) -- the
 * per-M-block N-block lists of [P1] Core changes 2; k2q_* holds the same
 * pairs transposed (per key block, its query blocks: the K2Q metadata of [P4]
 * CSR Tile Mapping).  Rows are flattened as ((b * heads + hm) * n_blocks +
 * block); columns ascend within a row; row_ptr[0] == 0.  LoopK reads only
 * q2k_*, LoopQ only k2q_*, SPLIT and SPLIT_DS both (and need the two forms
 * to hold the same pairs); a pair not read may be NULL.  Inside a kept block
 * every pair is attended, unless token_bits is given: then pair (i, j) of a
 * kept block is attended iff its bit is set (token-exact index sparsity: each
 * query keeps exactly its selected keys; isattn_index_to_token_bits builds
 * it).  token_bits: uint32 device, one slot of 1024 words per (b, hm, qb, kb)
 * at ((b * heads + hm) * n_qb + qb) * n_kb + kb (every block, kept or not):
 * words [0, 512) row-major -- bit j % 32 of word 4 r + j / 32 is row r, key j
 * of the block -- and words [512, 1024) the same bits key-major -- bit r % 32
 * of word 512 + 4 j + r / 32.  SPLIT, SPLIT_DS and the forward only.
 * block_q = block_k = 128; heads is 1, heads_k or heads_q.
 * nnz: host-side count of the CSR's blocks (q2k_row_ptr[last]) when the
 * caller knows it, else any negative value.  Only SPLIT_DS reads it, to size
 * its dS store by the kept blocks; a count below the true one makes results
 * undefined (dS stores past the workspace are dropped, never written out of
 * bounds). */
typedef struct isattn_mask {
    int32_t kind;
    int32_t block_q, block_k;
    int32_t heads;
    const int32_t* q2k_row_ptr;   /* [batch*heads*n_qb + 1] device */
    const int32_t* q2k_col;       /* [nnz] device                   */
    const int32_t* k2q_row_ptr;   /* [batch*heads*n_kb + 1] device */
    const int32_t* k2q_col;       /* [nnz] device                   */
    const uint32_t* token_bits;   /* NULL, or [batch*heads*n_qb*n_kb][1024] device */
    int64_t nnz;                  /* host: blocks in the CSR, or < 0 if unknown */
} isattn_mask_t;

/* Loop orders of [P1] Summary.  LOOPK: outer loop over 128-row query tiles,
 * inner loop streams the kept K/V tiles; dQ stays on chip and is stored once,
 * dK/dV are reduced as fp32 atomics into the workspace and converted by a
 * postprocess.  LOOPQ: outer loop over 128-key tiles, inner loop over the
 * query tiles of every head of the GQA group; dK/dV stay on chip and are
 * stored directly, dQ is reduced as fp32 atomics and converted afterwards.
 * SPLIT: both loop orders, each restricted to the outputs it keeps on chip --
 * a LOOPK pass for dQ, which runs first and also computes delta and
 * lse * log2(e) of every query row, then a LOOPQ pass for dK/dV --
 * recomputing P and dS in each; no atomics, no fp32 accumulators and no
 * separate preprocess (1.4x the MFMA work at Dqk = Dv).
 * SPLIT_DS: the LOOPQ pass for dK/dV runs first (after a preprocess for
 * delta) and also stores every dS tile it forms (bf16) in the workspace; a
 * LOOPK pass then accumulates dQ = dS K from them, streaming 32 KiB of dS per
 * kept block instead of recomputing S and dP.  Same results as SPLIT up to
 * rounding order.  Its workspace holds one 32 KiB dS tile per kept block
 * of each query head: (heads_q / mask heads) * nnz tiles for a block CSR,
 * batch * heads_q * (visible 128 x 128 blocks of one head) for a dense or
 * causal mask, batch * heads_q * ceil(Sq/128) * ceil(Sk/128) for a dense
 * mask over packed sequences; a block CSR whose nnz the caller does not give
 * is sized for every block of every mask head. */
enum { ISATTN_ALGO_LOOPK = 0, ISATTN_ALGO_LOOPQ = 1, ISATTN_ALGO_SPLIT = 2, ISATTN_ALGO_SPLIT_DS = 3 };

/* Bytes of device workspace isattn_attn_bwd needs for this shape and algo
 * (fp32 delta [B,Hq,Sq] plus head-major fp32 accumulators: dK,dV [B,Hk,Sk,D]
 * for LOOPK, dQ [B,Hq,Sq,Dqk] for LOOPQ; for SPLIT fp32 delta and
 * lse * log2(e), each [B,Hq,ceil(Sq/128)*128], the int32 work order of its
 * two passes, and -- when there are fewer than 512 (b, KV head, 128-key
 * block) items -- the schedule and fp32 partial dK|dV of the items cut into
 * parts; for SPLIT_DS the same plus, for block CSR masks, the int32 K->Q
 * position of every Q->K entry and then the bf16 dS tiles of 128 x 128;
 * each part 256-byte aligned).  This form assumes nothing about the mask:
 * its SPLIT_DS size holds a dS tile for every (b, h, query block, key
 * block).  Returns 0 for a NULL shape or unknown algo. */
size_t isattn_attn_bwd_workspace_bytes(const isattn_shape_t* shape, int32_t algo);

/* The same for a given mask (NULL = dense), causal flag and layout (varlen
 * nonzero: packed sequences, the shape holding the longest lengths): SPLIT_DS
 * gets exactly the dS tiles of the kept blocks (see ISATTN_ALGO_SPLIT_DS),
 * reading mask->nnz for a block CSR.  isattn_attn_bwd derives the dS
 * capacity from workspace_bytes and returns ISATTN_ERR_CAPACITY, before any
 * launch, when it holds fewer tiles than the mask needs (an nnz below 0
 * needs the every-block size).  The other algorithms' sizes do not depend on
 * the mask. */
size_t isattn_attn_bwd_workspace_bytes_mask(const isattn_shape_t* shape, int32_t algo,
                                            const isattn_mask_t* mask, int32_t causal,
                                            int32_t varlen);

/* Attention backward ([P1] Summary and Core changes 1-3): recompute
 * P = exp(softmax_scale * Q K^T - LSE) on the kept pairs, then
 *   D  = rowsum(dO * O),  dS = P * (dO V^T - D),
 *   dV = P^T dO,  dK = softmax_scale * dS^T Q,  dQ = softmax_scale * dS K
 * (dK/dV summed over the query heads of a GQA group).
 *
 * q [B,Sq,Hq,Dqk], k [B,Sk,Hk,Dqk], v [B,Sk,Hk,Dv], o and dO [B,Sq,Hq,Dv]:
 *   bf16 inputs.  lse: fp32 [B,Hq,Sq] contiguous, natural-log log-sum-exp of
 *   the scaled scores over the kept keys (+inf for a row with none).
 * mask_desc: see isattn_mask_t; NULL means dense.
 * causal: nonzero adds the bottom-right causal term j <= i + Sk - Sq.
 * dq, dk, dv: bf16 outputs with q/k/v's shapes; overwritten, not accumulated.
 * algo: ISATTN_ALGO_LOOPK, ISATTN_ALGO_LOOPQ, ISATTN_ALGO_SPLIT or
 *   ISATTN_ALGO_SPLIT_DS.
 * workspace: device buffer of at least isattn_attn_bwd_workspace_bytes bytes,
 *   256-byte aligned; its contents on entry do not matter.
 * stream: hipStream_t (NULL = default stream).
 * Supported: (dim_qk, dim_v) in {(64,64), (128,128), (192,128)}.  SPLIT and
 *   SPLIT_DS address rows within one head with 32-bit byte offsets: they return
 *   ISATTN_ERR_STRIDE_ALIGN unless ceil(S/128)*128 * stride_s * 2 < 2^31 for
 *   q and dO (S = Sq) and for k and v (S = Sk). */
isattn_status_t isattn_attn_bwd(const isattn_shape_t* shape,
                                const isattn_tensor_t* q, const isattn_tensor_t* k,
                                const isattn_tensor_t* v, const isattn_tensor_t* o,
                                const isattn_tensor_t* dO, const float* lse,
                                const isattn_mask_t* mask_desc, int32_t causal,
                                float softmax_scale,
                                const isattn_tensor_t* dq, const isattn_tensor_t* dk,
                                const isattn_tensor_t* dv,
                                int32_t algo, void* workspace, size_t workspace_bytes,
                                void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * isattn_attn_bwd with algo ISATTN_ALGO_SPLIT and no workspace argument.  Its
 * workspace is a static device array of ISATTN_NOALLOC_SCRATCH_BYTES (64
 * MiB) inside the library; each GPU holds its own copy from its first call
 * until the process ends, and nothing is allocated or freed per call (no
 * hipMalloc, no hipFree).  The dK/dV pass runs one workgroup per (b, KV head,
 * key block) item (no part mode, so no fp32 partials), which bounds the
 * scratch to delta and lse * log2(e), fp32 [B,Hq,ceil(Sq/128)*128] each, and
 * the int32 work order: B*Hq*ceil(Sq/128)*128*8 + 4*(B*Hk*ceil(Sk/128) +
 * B*Hq*ceil(Sq/128)) bytes, 256-byte aligned parts.  A problem needing more
 * returns ISATTN_ERR_SCRATCH before anything is enqueued.  Every call on a
 * GPU uses that GPU's one scratch array, whose contents (left over from the
 * previous call) need no clearing; calls that overlap in time on one GPU --
 * on different streams or from different threads without ordering -- race
 * on it and give undefined results.  Other arguments, errors and results as
 * isattn_attn_bwd with ISATTN_ALGO_SPLIT. */
#define ISATTN_NOALLOC_SCRATCH_BYTES (64u << 20)
isattn_status_t isattn_attn_bwd_noalloc(const isattn_shape_t* shape,
                                        const isattn_tensor_t* q, const isattn_tensor_t* k,
                                        const isattn_tensor_t* v, const isattn_tensor_t* o,
                                        const isattn_tensor_t* dO, const float* lse,
                                        const isattn_mask_t* mask_desc, int32_t causal,
                                        float softmax_scale,
                                        const isattn_tensor_t* dq, const isattn_tensor_t* dk,
                                        const isattn_tensor_t* dv, void* stream);

/* Attention forward on the same mask descriptor: the outputs the backward
 * consumes ([P1] Summary: the backward recomputes P from the forward's LSE;
 * online rescaling as in the attention notes of the nvfp4-megamoe-kernel log):
 *   S = softmax_scale * Q K^T on the kept pairs,
 *   LSE = ln sum_j exp(S_ij)  (natural log, fp32; +inf for a row with none),
 *   O = sum_j exp(S_ij - LSE_i) V_j  (bf16, 0 for a row with no kept key).
 * q [B,Sq,Hq,Dqk], k [B,Sk,Hk,Dqk], v [B,Sk,Hk,Dv]: bf16 inputs; o
 * [B,Sq,Hq,Dv] bf16 output; lse fp32 [B,Hq,Sq] contiguous output.  Both are
 * overwritten.  mask_desc: NULL (dense) or a block CSR whose q2k lists are
 * read (k2q may be NULL); causal as for isattn_attn_bwd.  No workspace.
 * Errors as for isattn_attn_bwd; K/V rows are addressed with 32-bit byte
 * offsets within a head (ceil(Sk/128)*128 * stride_s * 2 < 2^31 for k and v,
 * else ISATTN_ERR_STRIDE_ALIGN).  stream: hipStream_t (NULL = default). */
isattn_status_t isattn_attn_fwd(const isattn_shape_t* shape,
                                const isattn_tensor_t* q, const isattn_tensor_t* k,
                                const isattn_tensor_t* v, const isattn_mask_t* mask_desc,
                                int32_t causal, float softmax_scale,
                                const isattn_tensor_t* o, float* lse, void* stream);

/* Bytes of device workspace isattn_index_to_block_sparse needs (presence
 * matrix plus row/column counts, 256-byte aligned parts). */
size_t isattn_index_to_block_sparse_workspace_bytes(int32_t batch, int32_t seqlen_q,
                                                    int32_t seqlen_k, int32_t nhk,
                                                    int32_t block_q, int32_t block_k);

/* Token top-k indices -> block sparsity ([P1] Core changes 2; [P4] CSR Tile
 * Mapping; index format of [P3] Main Changes 1).
 * indices: int32 device [batch*seqlen_q, nhk, topk], contiguous; row r is
 *   query r % seqlen_q of sequence r / seqlen_q; a value is a key position in
 *   that sequence.  -1 and any value outside [0, seqlen_k) select nothing;
 *   duplicates select once; entry order is irrelevant.
 * Builds presence[b, hk, qb, kb] = 1 iff a row of query block qb selects a key
 * of key block kb, then writes both CSR forms (rows flattened over (b, hk),
 * columns ascending, row_ptr[0] = 0):
 *   q2k_row_ptr [batch*nhk*n_qb + 1], q2k_col [nnz];
 *   k2q_row_ptr [batch*nhk*n_kb + 1], k2q_col [nnz].
 * nnz is left on the device as row_ptr[last] (no host synchronisation).
 * col_capacity (elements of each col array) must be at least
 * batch*nhk*n_qb*n_kb.  block_q, block_k >= 1 (128 for isattn_attn_bwd). */
isattn_status_t isattn_index_to_block_sparse(const int32_t* indices, int32_t batch,
                                             int32_t seqlen_q, int32_t seqlen_k, int32_t nhk,
                                             int32_t topk, int32_t block_q, int32_t block_k,
                                             int32_t* q2k_row_ptr, int32_t* q2k_col,
                                             int32_t* k2q_row_ptr, int32_t* k2q_col,
                                             int64_t col_capacity, void* workspace,
                                             size_t workspace_bytes, void* stream);

/* ---- Packed variable-length sequences ----------------------------------
 * (the packed sequences of [P2]'s variable-length backward and of [P3]
 * Background; [P1] Limitations leaves LoopK fixed-length only.)
 * Sequence b of a batch of `batch` sequences is tokens [cu_seqlens_q[b],
 * cu_seqlens_q[b+1]) of the query-side tensors (q, o, dO, dq) and
 * [cu_seqlens_k[b], cu_seqlens_k[b+1]) of the key side (k, v, dk, dv); both
 * arrays are int32 device [batch + 1], nondecreasing, starting at 0.  Tensor
 * views address token t as ptr + t * stride_s + h * stride_h (stride_b is
 * unused).  shape->seqlen_q / seqlen_k are the longest lengths: every
 * sequence must fit them (a longer one is cut to them).  Attention, causal
 * alignment (bottom-right, per sequence) and 128-row / 128-key blocks are
 * those of each sequence on its own; mask rows and presence use the longest
 * block counts, blocks past a sequence's end are ignored.  lse is fp32
 * [batch, heads_q, seqlen_q] (entries past a sequence's length unused). */
typedef struct isattn_varlen {
    const int32_t* cu_seqlens_q;
    const int32_t* cu_seqlens_k;
} isattn_varlen_t;

/* isattn_attn_bwd over packed sequences.  algo: ISATTN_ALGO_SPLIT or
 * ISATTN_ALGO_SPLIT_DS (others: ISATTN_ERR_UNSUPPORTED); workspace as
 * isattn_attn_bwd_workspace_bytes(shape, algo) with the longest lengths.
 * NULL cu_seqlens with batch > 0: ISATTN_ERR_NULL. */
isattn_status_t isattn_attn_bwd_varlen(const isattn_shape_t* shape, const isattn_varlen_t* varlen,
                                       const isattn_tensor_t* q, const isattn_tensor_t* k,
                                       const isattn_tensor_t* v, const isattn_tensor_t* o,
                                       const isattn_tensor_t* dO, const float* lse,
                                       const isattn_mask_t* mask_desc, int32_t causal,
                                       float softmax_scale, const isattn_tensor_t* dq,
                                       const isattn_tensor_t* dk, const isattn_tensor_t* dv,
                                       int32_t algo, void* workspace, size_t workspace_bytes,
                                       void* stream);

/* isattn_attn_fwd over packed sequences (same conventions). */
isattn_status_t isattn_attn_fwd_varlen(const isattn_shape_t* shape, const isattn_varlen_t* varlen,
                                       const isattn_tensor_t* q, const isattn_tensor_t* k,
                                       const isattn_tensor_t* v, const isattn_mask_t* mask_desc,
                                       int32_t causal, float softmax_scale,
                                       const isattn_tensor_t* o, float* lse, void* stream);

/* isattn_index_to_block_sparse over packed sequences: indices int32 device
 * [cu_seqlens_q[batch], nhk, topk]; row r of sequence b (cu_seqlens_q[b] <=
 * r < cu_seqlens_q[b+1]) is its query r - cu_seqlens_q[b] and its values are
 * key positions in that sequence (outside [0, its key length): padding).
 * Block counts, outputs, capacity and workspace are those of
 * isattn_index_to_block_sparse with seqlen_q = max_seqlen_q and seqlen_k =
 * max_seqlen_k. */
isattn_status_t isattn_index_to_block_sparse_varlen(const int32_t* indices, int32_t batch,
                                                    const int32_t* cu_seqlens_q,
                                                    const int32_t* cu_seqlens_k, int32_t max_seqlen_q,
                                                    int32_t max_seqlen_k, int32_t nhk, int32_t topk,
                                                    int32_t block_q, int32_t block_k,
                                                    int32_t* q2k_row_ptr, int32_t* q2k_col,
                                                    int32_t* k2q_row_ptr, int32_t* k2q_col,
                                                    int64_t col_capacity, void* workspace,
                                                    size_t workspace_bytes, void* stream);

/* Top-k selection (the indexer step before the converter; xtuner PR #2096,
 * Main Changes item 1).  scores: fp32 device [rows, ld] (row r at scores +
 * r * ld, ld >= n); starts / ends: int32 device [rows] -- row r selects
 * among positions [starts[r], ends[r]) clipped to [0, n) -- or both NULL for
 * whole rows.  out: int32 device [rows, topk]: the selected positions ordered
 * by score, highest first (equal scores: smaller position first), then -1
 * where the row has fewer valid positions than topk.  0 <= topk <= 8192.
 * Scores must not be NaN. */
isattn_status_t isattn_topk_select(const float* scores, int64_t ld, int32_t rows, int32_t n,
                                   const int32_t* starts, const int32_t* ends, int32_t topk,
                                   int32_t* out, void* stream);

/* Token-exact bits of an index tensor (the per-block bitmaps of
 * isattn_mask_t.token_bits, heads = nhk, 128 x 128 blocks): indices as for
 * isattn_index_to_block_sparse, or packed sequences when cu_seqlens_q and
 * cu_seqlens_k are given (then seqlen_q / seqlen_k are the longest lengths);
 * bit (i, j) is set iff query i's row selects key j.  bits: uint32 device of
 * at least bits_words = batch*nhk*ceil(seqlen_q/128)*ceil(seqlen_k/128)*1024
 * words, fully overwritten. */
isattn_status_t isattn_index_to_token_bits(const int32_t* indices, int32_t batch, int32_t seqlen_q,
                                           int32_t seqlen_k, int32_t nhk, int32_t topk,
                                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                           uint32_t* bits, int64_t bits_words, void* stream);

/* Bytes of device workspace isattn_block_mask_to_csr needs. */
size_t isattn_block_mask_to_csr_workspace_bytes(int32_t batch, int32_t heads, int32_t n_qb,
                                                int32_t n_kb);

/* Block presence matrix -> Q->K and K->Q CSR (the normalisation step of [P1]
 * Core changes 2 and the transposed lists of [P4]).  presence: uint8 device
 * [batch, heads, n_qb, n_kb], nonzero = kept.  Outputs and col_capacity as for
 * isattn_index_to_block_sparse (capacity >= batch*heads*n_qb*n_kb). */
isattn_status_t isattn_block_mask_to_csr(const uint8_t* presence, int32_t batch, int32_t heads,
                                         int32_t n_qb, int32_t n_kb,
                                         int32_t* q2k_row_ptr, int32_t* q2k_col,
                                         int32_t* k2q_row_ptr, int32_t* k2q_col,
                                         int64_t col_capacity, void* workspace,
                                         size_t workspace_bytes, void* stream);

/* Static string for a status code (never NULL). */
const char* isattn_status_string(isattn_status_t status);

/* Library version as "major.minor.patch" (static string). */
const char* isattn_version(void);

/* ---- Stage timing (measurement support) -----------------------------------
 * A timer records HIP events on the call's stream around the launches of
 * isattn_attn_bwd_timed: stage [0] preprocess (for SPLIT only its work-order
 * kernel), [1] first main kernel (LOOPK / LOOPQ main loop, the SPLIT dQ pass
 * or the SPLIT_DS dK/dV pass), [2] second main kernel (the SPLIT dK/dV pass
 * or the SPLIT_DS dQ pass; empty otherwise), [3] postprocess (empty for
 * SPLIT and SPLIT_DS).
 * isattn_timer_read synchronises on the recorded events and returns the number
 * of timed calls and the summed milliseconds per stage (stage_ms[4]).  A timer
 * holds `capacity` calls; further calls wrap and overwrite. */
typedef struct isattn_timer isattn_timer_t;

isattn_status_t isattn_timer_create(int32_t capacity, isattn_timer_t** out);
isattn_status_t isattn_timer_destroy(isattn_timer_t* timer);
isattn_status_t isattn_timer_reset(isattn_timer_t* timer);
isattn_status_t isattn_timer_read(isattn_timer_t* timer, int32_t* n_calls, float* stage_ms);

/* isattn_attn_bwd with stage events recorded into `timer` (may be NULL). */
isattn_status_t isattn_attn_bwd_timed(const isattn_shape_t* shape,
                                      const isattn_tensor_t* q, const isattn_tensor_t* k,
                                      const isattn_tensor_t* v, const isattn_tensor_t* o,
                                      const isattn_tensor_t* dO, const float* lse,
                                      const isattn_mask_t* mask_desc, int32_t causal,
                                      float softmax_scale,
                                      const isattn_tensor_t* dq, const isattn_tensor_t* dk,
                                      const isattn_tensor_t* dv,
                                      int32_t algo, void* workspace, size_t workspace_bytes,
                                      void* stream, isattn_timer_t* timer);

#ifdef __cplusplus
}
#endif

#endif /* ISATTN_H */
