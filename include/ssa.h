/*
 * ssa.h - C ABI of the streaming sparse attention (SSA) kernel library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (LongCat ZigZag Attention; digest on www.163.com, section 01,
 * part (1): the SSA paragraph after the calibration equations; part (2): the
 * deployed configuration): each query token attends only to a few "sink"
 * blocks and a few "local" blocks; the selected, blocked keys and values are
 * fixed by the number of sink blocks s, the number of local blocks l and the
 * block size b. The deployed setting is b = 128, s = 1, l = 7, a 1,024-token
 * window; the same page's section 02 (efficiency figure paragraph) compares a
 * streaming sparse decode kernel with a full-attention decode kernel.
 *
 * Exact rule implemented (readings of the page, which lost the equation):
 * blocks are b consecutive positions aligned at 0; for a query at position i
 * in block qb = i / b, key j is attended iff
 *     j <= i   and   ( j / b < s   or   j / b > qb - l )
 * i.e. the first s blocks plus the l blocks ending at the query's own block,
 * causal, each key once. The result is softmax(scale * q . k_j) weighted sum
 * of v_j over the attended keys; lse is the natural-log log-sum-exp of the
 * scaled scores.
 *
 * Conventions shared by every entry point:
 *  - Every pointer argument is a DEVICE pointer owned by the caller (q, k, v,
 *    caches, outputs, page tables, lengths, workspace). The library allocates
 *    nothing, keeps no pointer after it returns and holds no mutable global
 *    state; calls on different streams are independent.
 *  - Calls are asynchronous on `stream`. Inputs, outputs and workspace must
 *    stay valid until the stream passes the call.
 *  - The softmax scale must be finite and > 0 (1/sqrt(d_qk) is the usual one).
 *  - Arguments are checked on the host before anything is launched:
 *    SSA_ERR_INVALID_ARG for a bad size, stride, pattern, scale or pointer;
 *    SSA_ERR_UNSUPPORTED for a (dtype, d_qk, d_v, group) combination that has
 *    no compiled kernel; SSA_ERR_WORKSPACE when the workspace is too small.
 *    Nothing is launched when a check fails. SSA_ERR_HIP reports a failed
 *    kernel launch.
 *  - Strides are in ELEMENTS, the head-dim axis has unit stride, and every
 *    row must start on a 16-byte boundary (pointers and strides aligned).
 *  - Accumulation is fp32. bf16 outputs are rounded to nearest-even.
 *  - Device-resident integers (page ids, context lengths) are trusted: they
 *    are not range-checked on the host. A context length above the page
 *    table's capacity (max_pages x page_size) is taken as that capacity; a
 *    page id outside the cache is not detected.
 */
#ifndef BLOCK_SPARSE_STREAMING_SSA_H
#define BLOCK_SPARSE_STREAMING_SSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums are int-sized in C and C++ alike. In C++ they get int as their
 * fixed underlying type, so any int a C caller passes is a value of the type
 * (an unknown dtype is then rejected, not undefined behaviour). */
#ifdef __cplusplus
#define SSA_ENUM_BASE : int
#else
#define SSA_ENUM_BASE
#endif

typedef enum ssa_status SSA_ENUM_BASE {
    SSA_OK = 0,
    SSA_ERR_INVALID_ARG = 1,
    SSA_ERR_UNSUPPORTED = 2,
    SSA_ERR_WORKSPACE = 3,
    SSA_ERR_HIP = 4
} ssa_status;

/* Element type of q, k, v, caches and outputs (lse is always fp32). */
typedef enum ssa_dtype SSA_ENUM_BASE { SSA_F32 = 0, SSA_BF16 = 1 } ssa_dtype;

/* The SSA pattern: block size b >= 1, sink blocks s >= 0, local blocks l >= 1
 * (the local blocks include the query's own block, so l >= 1 keeps every row
 * non-empty). */
typedef struct ssa_pattern {
    int32_t block;
    int32_t sink;
    int32_t local;
} ssa_pattern;

/*
 * ssa_prefill - causal streaming sparse attention over whole sequences
 * (the SSA operator of the digest's section 01 part (1), applied to every
 * query row of a sequence, as in prefill).
 *
 *   q   [batch, seq_len, heads_q,  d_qk]  strides q_strides  (batch, token, head)
 *   k   [batch, seq_len, heads_kv, d_qk]  strides k_strides
 *   v   [batch, seq_len, heads_kv, d_v ]  strides v_strides
 *   o   [batch, seq_len, heads_q,  d_v ]  strides o_strides, written
 *   lse [batch, heads_q, seq_len] fp32 contiguous, written; may be NULL
 * Query head h reads kv head h / (heads_q / heads_kv); heads_q % heads_kv
 * must be 0. batch == 0 or seq_len == 0 is a no-op returning SSA_OK.
 * Compiled (dtype, d_qk, d_v): bf16 (64,64), (128,128), (192,128);
 * fp32 (64,64), (128,128).
 */
ssa_status ssa_prefill(ssa_dtype dtype, const void *q, const void *k, const void *v, void *o,
                       float *lse, int32_t batch, int32_t seq_len, int32_t heads_q,
                       int32_t heads_kv, int32_t d_qk, int32_t d_v, const int64_t q_strides[3],
                       const int64_t k_strides[3], const int64_t v_strides[3],
                       const int64_t o_strides[3], ssa_pattern pattern, float scale,
                       hipStream_t stream);

/*
 * ssa_prefill_dual - SSA attention and full causal attention of the same
 * q, k, v in one pass, plus their mix. The digest's calibration step (section
 * 01, part (1): the calibration paragraph before the SSA paragraph) gives each
 * attention module a learnable weight alpha in [0, 1] that mixes its full and
 * sparse outputs; the equation was lost from the page, and the mix is read as
 *     o_mix = alpha * o_full + (1 - alpha) * o_ssa.
 * Calibration needs both outputs of every layer; SSA keys are a subset of the
 * causal keys, so the kernel visits them first, writes the SSA result, and
 * goes on over the remaining causal keys for the full result.
 *
 *   q, k, v        as in ssa_prefill.
 *   o_ssa, lse_ssa what ssa_prefill writes (lse_ssa may be NULL).
 *   o_full         full causal attention, softmax(scale q k^T) v over j <= i,
 *                  [batch, seq_len, heads_q, d_v]; required.
 *   lse_full       its lse [batch, heads_q, seq_len] fp32; may be NULL.
 *   o_mix          alpha * o_full + (1 - alpha) * o_ssa, or NULL for none.
 *                  It is formed from the fp32 full result and the rounded
 *                  o_ssa already written.
 *   o_strides      shared by o_ssa, o_full and o_mix, which must be distinct
 *                  buffers that overlap neither each other nor the inputs.
 *   alpha          in [0, 1] (checked even when o_mix is NULL).
 * Cost is that of full causal attention (the SSA keys are not visited twice).
 * batch == 0 or seq_len == 0 is a no-op. Compiled: bf16 with (d_qk, d_v) =
 * (64,64), (128,128), (192,128); fp32 returns SSA_ERR_UNSUPPORTED.
 */
ssa_status ssa_prefill_dual(ssa_dtype dtype, const void *q, const void *k, const void *v,
                            void *o_ssa, float *lse_ssa, void *o_full, float *lse_full, void *o_mix,
                            float alpha, int32_t batch, int32_t seq_len, int32_t heads_q,
                            int32_t heads_kv, int32_t d_qk, int32_t d_v,
                            const int64_t q_strides[3], const int64_t k_strides[3],
                            const int64_t v_strides[3], const int64_t o_strides[3],
                            ssa_pattern pattern, float scale, hipStream_t stream);

/*
 * ssa_prefill_backward - gradients of ssa_prefill (same operator, same
 * pattern). The digest trains the sparsified layers further after replacing
 * them with SSA (section 01, part (1): the training paragraph after the SSA
 * output; part (2): mid-training and post-training), which needs dq, dk, dv.
 * With P_ij = exp(scale q_i.k_j - lse_i) over the attended pairs and
 * D_i = sum_d dout_id o_id:
 *     dq_i = scale sum_j P_ij (dout_i.v_j - D_i) k_j
 *     dk_j = scale sum_i P_ij (dout_i.v_j - D_i) q_i
 *     dv_j = sum_i P_ij dout_i
 * summed over every query head of a kv head's group for dk and dv.
 *
 *   q, k, v    the forward's inputs, layouts as in ssa_prefill.
 *   o, lse     the forward's output [batch, seq_len, heads_q, d_v] (strides
 *              o_strides) and its lse [batch, heads_q, seq_len] (fp32,
 *              contiguous, natural log), as written by ssa_prefill; lse is
 *              required here.
 *   dout       upstream gradient, shape of o, strides do_strides.
 *   dq, dk, dv written, shapes of q, k, v with their own strides; every
 *              element is overwritten (no accumulation into old contents).
 *              They must not overlap any input.
 *   workspace  device scratch of at least ssa_prefill_backward_workspace_size
 *              bytes; no initial contents are required; calls sharing one
 *              workspace must not overlap.
 * Accumulation is fp32; P and the score gradients are rounded to bf16 as
 * MFMA operands. Results are deterministic (no atomics). batch == 0 or
 * seq_len == 0 is a no-op. Compiled: bf16 with (d_qk, d_v) = (64,64),
 * (128,128), (192,128); anything else returns SSA_ERR_UNSUPPORTED.
 */
ssa_status ssa_prefill_backward(ssa_dtype dtype, const void *q, const void *k, const void *v,
                                const void *o, const float *lse, const void *dout, void *dq,
                                void *dk, void *dv, int32_t batch, int32_t seq_len,
                                int32_t heads_q, int32_t heads_kv, int32_t d_qk, int32_t d_v,
                                const int64_t q_strides[3], const int64_t k_strides[3],
                                const int64_t v_strides[3], const int64_t o_strides[3],
                                const int64_t do_strides[3], const int64_t dq_strides[3],
                                const int64_t dk_strides[3], const int64_t dv_strides[3],
                                void *workspace, size_t workspace_bytes, ssa_pattern pattern,
                                float scale, hipStream_t stream);

/*
 * Workspace bytes for ssa_prefill_backward with the same shape arguments;
 * 0 for arguments it would reject and for an empty problem. It holds two
 * floats per (batch, query head, row) and, when the pattern has sink blocks,
 * fp32 partial sums of the sink keys' dk and dv per chunk of query rows.
 */
size_t ssa_prefill_backward_workspace_size(ssa_dtype dtype, int32_t batch, int32_t seq_len,
                                           int32_t heads_q, int32_t heads_kv, int32_t d_qk,
                                           int32_t d_v, ssa_pattern pattern);

/*
 * ssa_decode - one new query token per sequence against a paged KV cache,
 * attending to the SSA window (digest section 02: the streaming sparse
 * attention kernel in the decode phase).
 *
 *   q          [batch, heads_q, d_qk] contiguous.
 *   k_cache    page-major cache; element (page, slot, kv head, dim) sits at
 *              page*k_strides[0] + slot*k_strides[1] + head*k_strides[2] + dim.
 *   v_cache    likewise with v_strides and d_v dims. v_cache may equal k_cache
 *              with equal strides: then the value is the first d_v entries of
 *              the key row (a latent cache, as in absorbed MLA).
 *   page_table [batch, max_pages] int32 physical page ids, row-major.
 *   max_pages  the page table's row length; it follows page_table, the array
 *              it describes.
 *   ctx_lens   [batch] int32 context lengths L, the new token included: its
 *              key and value are already in the cache and the query sits at
 *              position L - 1. Token t of a sequence is in page
 *              page_table[t / page_size] at slot t % page_size.
 *              L <= 0 writes a zero output and lse = -inf; L must not exceed
 *              max_pages * page_size.
 *   o          [batch, heads_q, d_v] contiguous, written; lse [batch, heads_q]
 *              fp32 or NULL.
 *   workspace  device scratch of at least ssa_decode_workspace_size(...)
 *              bytes (same shape arguments, full = 0); no initial contents
 *              are required. Calls sharing one workspace must not overlap.
 *              A non-latent call whose attended tokens fit one split (a
 *              window of at most 128 tokens; for full_attn_decode a table of
 *              at most 256) writes o and lse from the split kernel and
 *              leaves the workspace untouched; it is still checked.
 * Compiled: bf16 or fp32 with d_qk = d_v in {64, 128, 256} and
 * heads_q / heads_kv in {1, 2, 4, 8}, except group 8 at d = 256
 * (SSA_ERR_UNSUPPORTED); bf16 latent shape d_qk = 576, d_v = 512 with
 * heads_q / heads_kv a multiple of 16.
 */
ssa_status ssa_decode(ssa_dtype dtype, const void *q, const void *k_cache, const void *v_cache,
                      const int64_t k_strides[3], const int64_t v_strides[3],
                      const int32_t *page_table, int32_t max_pages, const int32_t *ctx_lens,
                      int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t d_qk,
                      int32_t d_v, int32_t page_size, void *o, float *lse, void *workspace,
                      size_t workspace_bytes, ssa_pattern pattern, float scale,
                      hipStream_t stream);

/*
 * ssa_decode_noalloc - ssa_decode for callers that cannot allocate: code
 * under HIP graph capture, tight serving loops, harnesses that forbid device
 * allocation. Same arguments, layouts, checks and results as ssa_decode,
 * without the workspace: the call runs in a fixed scratch array of 32 MiB
 * (33,554,432 bytes) compiled into the library, one copy per GPU, held until
 * the process ends. The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine); on its first use on
 * a device it looks up that device's copy of the array (hipGetSymbolAddress,
 * with the device current), and after that it makes no HIP call other than
 * the launches.
 *
 * A call whose ssa_decode_workspace_size(...) exceeds the scratch returns
 * SSA_ERR_WORKSPACE and launches nothing (the 128K-context latent batch of
 * 32 sequences needs 16.8 MB; 65 sequences x 16 heads at d = 128, 4.3 MB).
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents (no call needs initial contents): calls that overlap on one
 * GPU (other streams, other threads) race and give wrong results. The
 * device is the one `stream` belongs to. SSA_ERR_HIP if the scratch cannot
 * be found on it.
 */
ssa_status ssa_decode_noalloc(ssa_dtype dtype, const void *q, const void *k_cache, const void *v_cache,
                              const int64_t k_strides[3], const int64_t v_strides[3],
                              const int32_t *page_table, int32_t max_pages, const int32_t *ctx_lens,
                              int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t d_qk,
                              int32_t d_v, int32_t page_size, void *o, float *lse, ssa_pattern pattern,
                              float scale, hipStream_t stream);

/*
 * full_attn_decode - the dense comparator of the digest's section 02
 * efficiency figure: the same call as ssa_decode, attending to every token
 * 0..L-1 of the context. Same layouts, ownership, errors and compiled shapes.
 */
ssa_status full_attn_decode(ssa_dtype dtype, const void *q, const void *k_cache,
                            const void *v_cache, const int64_t k_strides[3],
                            const int64_t v_strides[3], const int32_t *page_table,
                            int32_t max_pages, const int32_t *ctx_lens, int32_t batch,
                            int32_t heads_q, int32_t heads_kv, int32_t d_qk, int32_t d_v,
                            int32_t page_size, void *o, float *lse, void *workspace,
                            size_t workspace_bytes, float scale, hipStream_t stream);

/*
 * Workspace bytes for ssa_decode (full = 0; pattern used) or full_attn_decode
 * (full = 1; pattern ignored). Returns 0 for arguments the decode calls would
 * reject. It takes the decode call's shape arguments (dtype, head counts and
 * dims, page size and table width), since the split plan depends on all of
 * them. The workspace holds one partial output (bf16 for the latent shape,
 * fp32 otherwise) and one log-sum-exp per (sequence, query head, split of
 * the attended tokens).
 */
size_t ssa_decode_workspace_size(ssa_dtype dtype, int32_t batch, int32_t heads_q,
                                 int32_t heads_kv, int32_t d_qk, int32_t d_v,
                                 int32_t page_size, int32_t max_pages, ssa_pattern pattern,
                                 int full);

/*
 * ssa_extend - several new query tokens per sequence against the paged KV
 * cache, each attending to its own SSA window: a prefill chunk appended to a
 * cached prefix (chunked prefill), or the few tokens of a multi-token decode
 * step (speculative or multi-token-prediction drafts; the SSA paragraph of
 * the digest's section 01 part (1) defines the window per query position,
 * and section 02 measures the decode and prefill phases it serves).
 *
 * Sequence b has q_len_b = cu_q[b+1] - cu_q[b] new tokens at positions
 * ctx_lens[b] - q_len_b .. ctx_lens[b] - 1; their keys and values are
 * already in the cache (append, then attend). Row r of the chunk (packed row
 * cu_q[b] + r) attends exactly as a decode step at context length
 * ctx_lens[b] - q_len_b + r + 1 would, so causality inside the chunk holds.
 *
 *   q          [total_q, heads_q, d_qk] contiguous, rows packed by sequence.
 *   k_cache, v_cache, k_strides, v_strides, page_table, max_pages,
 *   page_size  as in ssa_decode.
 *   ctx_lens   [batch] int32 context lengths, the new tokens included.
 *   cu_q       [batch + 1] int32 prefix sums of the chunk lengths: cu_q[0] = 0,
 *              non-decreasing, cu_q[batch] = total_q, and q_len_b <= ctx_lens[b]
 *              (device data: trusted, not checked on the host).
 *   max_q_len  an upper bound of every q_len_b (host value, >= 1 when
 *              total_q > 0); rows beyond it are not computed.
 *   o          [total_q, heads_q, d_v] contiguous, written; lse [total_q,
 *              heads_q] fp32 or NULL.
 *   workspace  device scratch of at least ssa_extend_workspace_size(...)
 *              bytes (0 is possible); calls sharing it must not overlap.
 * Kernels: bf16 with (d_qk, d_v) in {(64,64), (128,128), (192,128)} takes a
 * paged tile kernel (128 rows of one sequence per work-group) when max_q_len
 * > 1 or no decode kernel fits; otherwise, and for the other shapes
 * ssa_decode compiles (fp32, d = 256, the latent shape), each row runs as a
 * decode step, with at most 65,535 rows per call. The tile kernel needs slot
 * strides below 2^24 elements. batch == 0 or total_q == 0 is a no-op.
 */
ssa_status ssa_extend(ssa_dtype dtype, const void *q, const void *k_cache, const void *v_cache,
                      const int64_t k_strides[3], const int64_t v_strides[3],
                      const int32_t *page_table, int32_t max_pages, const int32_t *ctx_lens,
                      const int32_t *cu_q, int32_t batch, int32_t total_q, int32_t max_q_len,
                      int32_t heads_q, int32_t heads_kv, int32_t d_qk, int32_t d_v,
                      int32_t page_size, void *o, float *lse, void *workspace,
                      size_t workspace_bytes, ssa_pattern pattern, float scale,
                      hipStream_t stream);

/*
 * Workspace bytes for ssa_extend with the same shape arguments; 0 when the
 * call needs none (the tile kernel), is empty, or would be rejected.
 */
size_t ssa_extend_workspace_size(ssa_dtype dtype, int32_t batch, int32_t total_q, int32_t max_q_len,
                                 int32_t heads_q, int32_t heads_kv, int32_t d_qk, int32_t d_v,
                                 int32_t page_size, int32_t max_pages, ssa_pattern pattern);

/*
 * hybrid_decode - one-token decode over the SSA window of `pattern` plus a
 * list of tokens chosen elsewhere, the two merged by log-sum-exp. It follows
 * the streaming-aware indexing of "LongCat Sparse Attention" (agihunt.info,
 * the streaming-aware indexing paragraph): of a 2,048-token budget, 16 sink
 * tokens and a 1,024-token sliding window are fixed and contiguous, and
 * 1,024 tokens come from an indexer; a hybrid kernel attends the fixed and
 * the sparse part separately and merges them with online softmax. Here the
 * fixed part is the SSA window (block 1, sink 16, local 1024 reproduces it
 * token for token) and the list is an input: the indexer is not part of this
 * library.
 *
 *   q, caches, strides, page_table, max_pages, ctx_lens, page_size, o, lse,
 *   scale      as in ssa_decode.
 *   topk       [batch, topk_k] int32 token positions, device memory. An entry
 *              inside the window, at or past the context length, or negative
 *              (padding) is skipped; entries must be distinct (a repeated
 *              token would count twice). Trusted device data.
 *   workspace  at least hybrid_decode_workspace_size(...) bytes.
 * The window and the listed tokens are cut into splits of one size; one
 * merge combines all of a row's splits. Compiled: every shape ssa_decode
 * compiles (bf16 or fp32 with d_qk = d_v in {64, 128, 256} and heads_q /
 * heads_kv in {1, 2, 4, 8}, except group 8 at d = 256; the bf16 latent
 * shape). The list is shared by a sequence's query heads. topk_k must be
 * >= 1.
 */
ssa_status hybrid_decode(ssa_dtype dtype, const void *q, const void *k_cache, const void *v_cache,
                         const int64_t k_strides[3], const int64_t v_strides[3],
                         const int32_t *page_table, int32_t max_pages, const int32_t *ctx_lens,
                         const int32_t *topk, int32_t topk_k, int32_t batch, int32_t heads_q,
                         int32_t heads_kv, int32_t d_qk, int32_t d_v, int32_t page_size, void *o,
                         float *lse, void *workspace, size_t workspace_bytes, ssa_pattern pattern,
                         float scale, hipStream_t stream);

/* Workspace bytes for hybrid_decode with the same shape arguments; 0 for
 * arguments it would reject. */
size_t hybrid_decode_workspace_size(ssa_dtype dtype, int32_t batch, int32_t heads_q, int32_t heads_kv,
                                    int32_t d_qk, int32_t d_v, int32_t page_size, int32_t max_pages,
                                    int32_t topk_k, ssa_pattern pattern);

/* Static, human-readable name of a status code. */
const char *ssa_status_string(ssa_status status);

#ifdef __cplusplus
}
#endif

#endif /* BLOCK_SPARSE_STREAMING_SSA_H */
