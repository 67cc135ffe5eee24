// Internal interface between the C-ABI layer (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssa {

struct PrefillArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;              // [B, Hq, N] or null
    int64_t qs[3], ks[3], vs[3], os[3];  // (batch, token, head) element strides
    int32_t B, N, Hq, Hkv, group;        // group = Hq / Hkv
    int32_t block, sink, local;
    float scale_log2;        // softmax scale * log2(e)
    int32_t num_qtiles;      // ceil(N / 128)
    int32_t total_wgs;       // num_qtiles * Hq * B
    // Dual mode (SSA and full causal attention in one pass): o / lse above
    // receive the SSA result; these the full one and, if o_mix is set,
    // alpha * o_full + (1 - alpha) * o (same strides as o).
    void *o_full;
    float *lse_full;         // [B, Hq, N] or null
    void *o_mix;             // or null
    float alpha;
    // Paged mode (new tokens of each sequence against a paged cache): q / o
    // are packed rows [total_q, Hq, d] (qs[0] = os[0] = 0), k / v are the
    // caches with (page, slot, head) strides, and sequence b's rows
    // cu_q[b] .. cu_q[b+1]-1 sit at the last positions of its ctx_lens[b]
    // tokens. num_qtiles is then the tiles of the longest chunk; lse is
    // [total_q, Hq].
    const int32_t *page_table;  // [B, max_pages]
    const int32_t *ctx_lens;    // [B]
    const int32_t *cu_q;        // [B + 1]
    int32_t max_pages, page_size;
};

enum PrefillMode { kModePlain = 0, kModeDual = 1, kModePaged = 2 };

bool prefill_supported(bool bf16, int d_qk, int d_v);
hipError_t launch_prefill(bool bf16, int d_qk, int d_v, const PrefillArgs &a, hipStream_t stream);
bool prefill_dual_supported(bool bf16, int d_qk, int d_v);
hipError_t launch_prefill_dual(bool bf16, int d_qk, int d_v, const PrefillArgs &a, hipStream_t stream);
bool prefill_paged_supported(bool bf16, int d_qk, int d_v);
hipError_t launch_prefill_paged(bool bf16, int d_qk, int d_v, const PrefillArgs &a, hipStream_t stream);

// Backward of the prefill operator. Workspace: per (batch, query head, group
// of 64 rows) the rows' lse * log2(e) then their D = sum_d dO*O (128 floats),
// and, for key tiles that hold sink keys, fp32 partial sums of dk (scaled)
// and dv per chunk of query rows.
struct BackwardArgs {
    const void *q, *k, *v, *o, *dout;
    const float *lse;                    // [B, Hq, N], natural log, from the forward
    void *dq, *dk, *dv;
    int64_t qs[3], ks[3], vs[3], os[3], dos[3], dqs[3], dks[3], dvs[3];  // (batch, token, head)
    int32_t B, N, Hq, Hkv, group;
    int32_t block, sink, local;
    float scale, scale_log2;
    float *rowstat;                      // [B, Hq, n_pad / 64, 2, 64]
    float *sink_part;                    // [n_chunks, B, Hkv, sink_rows, d_qk + d_v]
    int32_t n_pad;                       // N rounded up to a multiple of 128
    int32_t num_qtiles;                  // ceil(N / 128): query tiles, also key tiles
    int32_t sink_tiles;                  // key tiles holding a sink key
    int32_t sink_rows;                   // sink_tiles * 128, clamped to N
    int32_t chunk_rows, n_chunks;        // query rows per sink chunk (multiple of 128)
    int32_t dq_wgs, dkv_wgs, fin_wgs;    // grid sizes of the three launches
};

bool backward_supported(bool bf16, int d_qk, int d_v);
hipError_t launch_backward(bool bf16, int d_qk, int d_v, const BackwardArgs &a, hipStream_t stream);

enum DecodeKind { kDecodeValu = 0, kDecodeLatent = 1 };

// The latent kernel keeps the page ids of one split in LDS. A split of T
// positions covers at most two token runs, so at most (T - 2) / page_size + 4
// pages; the planner keeps that within this bound.
constexpr int kDecodeLatentMaxPages = 256;
// It also keeps the row offsets of a split of listed tokens (hybrid decode)
// in LDS: at most this many positions per split.
constexpr int kDecodeLatentMaxListSplit = 1024;

// How a decode call is cut into work-groups. Computed on the host from shapes
// only (context lengths live on the device), so the workspace size is known
// before the call.
struct DecodePlan {
    int kind;          // DecodeKind
    int split_tokens;  // attended tokens per split (multiple of the chunk size)
    int max_splits;    // splits per (sequence, head) the workspace holds
    int head_chunks;   // latent kernel: work-groups per kv head (64 heads each)
    int direct;        // VALU kernel with one split and no list: the split kernel
                       // writes o and lse itself and no merge runs
};

struct DecodeArgs {
    const void *q, *kc, *vc;
    int64_t ks[3], vs[3];          // (page, slot, head) element strides
    const int32_t *page_table;
    const int32_t *ctx_lens;
    int32_t max_pages, page_size;
    int32_t B, Hq, Hkv, group;
    int32_t block, sink, local, full;
    float scale_log2;
    void *o;
    float *lse;                     // [B, Hq] or null
    float *ws_o;                    // [B, Hq, max_splits, d_v]; bf16 for the latent kernel
    float *ws_lse;                  // [B, Hq, max_splits], log2 domain
    DecodePlan plan;
    // Several query rows per sequence: B counts query rows, and row r reads
    // page-table row row_seq[r] with context length row_ctx[r] (its position
    // + 1). Null for one row per sequence (row r = sequence r, ctx_lens[r]).
    const int32_t *row_seq;
    const int32_t *row_ctx;
    int32_t n_seqs;                 // sequences (page-table rows) when row_seq is set
    // Hybrid decode: besides the SSA window, each sequence attends the listed
    // tokens topk[b * topk_k + i] that lie outside the window (others, and
    // negative padding, are skipped). Their splits follow the window's.
    const int32_t *topk;
    int32_t topk_k;                 // 0: no list
};

bool decode_valu_supported(bool bf16, int d_qk, int d_v, int group);
bool decode_latent_supported(bool bf16, int d_qk, int d_v, int group);
hipError_t launch_decode(bool bf16, int d_qk, int d_v, const DecodeArgs &a, hipStream_t stream);

// Row map of packed query rows: row r of sequence b (cu_q[b] <= r < cu_q[b+1])
// gets row_seq[r] = b and row_ctx[r] = ctx_lens[b] - (cu_q[b+1] - 1 - r).
// Rows past cu_q[b] + max_q_len are not written; no write leaves [0, total_q).
hipError_t launch_extend_rows(const int32_t *cu_q, const int32_t *ctx_lens, int32_t batch,
                              int32_t max_q_len, int32_t total_q, int32_t *row_seq, int32_t *row_ctx,
                              hipStream_t stream);

}  // namespace ssa
