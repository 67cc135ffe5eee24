// C ABI of the SSA library: argument checks, work planning and dispatch.
// Every check runs on the host before any HIP call, so a rejected call
// launches nothing and touches no device state.
#include <cmath>
#include <cstdint>
#include <limits>
#include <mutex>

#include "ssa.h"
#include "kernels.h"

namespace {

using ssa::DecodeArgs;
using ssa::DecodePlan;
using ssa::PrefillArgs;

constexpr int64_t kInt32Max = std::numeric_limits<int32_t>::max();
// Target number of work-groups for a full-attention decode: two per CU on
// 256 CUs, i.e. long splits (8,192 tokens per split for 32 sequences at
// 128K). Each work-group pays a fixed set-up and partial write-out, and
// fewer, longer splits also leave the merge fewer partials; measured on the
// 128K latent workload, 512 beat 1,024 by 7% and 2,048 by 11-14%, and 256
// was level with 512.
constexpr int64_t kFullDecodeTargetWgs = 512;
// Upper bound of a full-attention split. Without it a call with many
// (sequence, head) rows (>= 512) would give every row a single split, and one
// work-group would walk a whole long context while the others sit idle.
constexpr int64_t kFullDecodeMaxSplit = 8192;
// Attended tokens per split for the windowed (SSA) decode.
constexpr int64_t kSsaSplitTokens = 128;

bool pattern_ok(const ssa_pattern &p) { return p.block >= 1 && p.sink >= 0 && p.local >= 1; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Strides must be non-negative and keep every row on a 16-byte boundary.
bool strides_ok(const int64_t *s, int n, int elem_bytes) {
    if (!s) return false;
    const int64_t unit = 16 / elem_bytes;
    for (int i = 0; i < n; ++i)
        if (s[i] < 0 || s[i] % unit) return false;
    return true;
}

int elem_bytes(ssa_dtype t) { return t == SSA_BF16 ? 2 : 4; }

bool dtype_ok(ssa_dtype t) { return t == SSA_F32 || t == SSA_BF16; }

// The latent split kernel holds a whole CU (its ring of latent rows fills the
// LDS): once a call has this many work-groups, wider splits cost no
// parallelism and cut the bf16 partials each split writes and the merge
// reads (64 heads x 512 x 2 B per split, about the size of 57 latent rows).
constexpr int64_t kLatentTargetWgs = 256;

// Work plan of a decode call; false if no compiled kernel fits the shape.
// list_tokens: listed tokens per row (hybrid decode), which take splits of
// the same width after the window's.
bool make_plan(ssa_dtype dtype, int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t d_qk,
               int32_t d_v, int32_t page_size, int32_t max_pages, const ssa_pattern &pat, bool full,
               DecodePlan *plan, int32_t list_tokens = 0) {
    const bool bf16 = dtype == SSA_BF16;
    const int group = heads_q / heads_kv;
    int chunk;
    plan->direct = 0;
    if (ssa::decode_latent_supported(bf16, d_qk, d_v, group)) {
        plan->kind = ssa::kDecodeLatent;
        plan->head_chunks = (group + 63) / 64;
        chunk = 32;
    } else if (ssa::decode_valu_supported(bf16, d_qk, d_v, group)) {
        plan->kind = ssa::kDecodeValu;
        plan->head_chunks = 1;
        chunk = 64;
    } else {
        return false;
    }
    const int64_t max_ctx = (int64_t)max_pages * page_size;
    int64_t split;
    int64_t max_tokens;
    if (full) {
        max_tokens = max_ctx;
        const int64_t wgs_per_split = (int64_t)batch * heads_kv * plan->head_chunks;
        split = (max_tokens * wgs_per_split + kFullDecodeTargetWgs - 1) / kFullDecodeTargetWgs;
        split = split < kFullDecodeMaxSplit ? split : kFullDecodeMaxSplit;
        split = split < 256 ? 256 : split;
    } else {
        const int64_t window = ((int64_t)pat.sink + pat.local) * pat.block;
        max_tokens = window < max_ctx ? window : max_ctx;
        split = kSsaSplitTokens;
        if (plan->kind == ssa::kDecodeLatent) {
            const int64_t rows = (int64_t)batch * heads_kv * plan->head_chunks;
            auto wgs = [&](int64_t w) { return rows * ((max_tokens + w - 1) / w + (list_tokens + w - 1) / w); };
            while (split < 1024 && wgs(2 * split) >= kLatentTargetWgs) split *= 2;
        }
    }
    split = (split + chunk - 1) / chunk * chunk;
    if (plan->kind == ssa::kDecodeLatent) {
        // Keep (split - 2) / page_size + 4 page ids within the kernel's table.
        const int64_t cap = ((int64_t)(ssa::kDecodeLatentMaxPages - 4) * page_size + 1) / chunk * chunk;
        if (cap < chunk) return false;
        split = split < cap ? split : cap;
    }
    if (split > kInt32Max) return false;
    const int64_t splits = (max_tokens + split - 1) / split;
    if (splits < 1 || splits > 65535) return false;
    plan->split_tokens = (int)split;
    plan->max_splits = (int)splits;
    // One split per row (a window, or a full context, within one split): the
    // VALU kernel writes the result itself and the merge launch is skipped.
    // (Whole windows of up to 1,024 tokens per work-group, to make every
    // call single-split, measured 7-12% slower on the 65 x 16 row ragged
    // workload than 128-token splits plus the merge.)
    plan->direct = plan->kind == ssa::kDecodeValu && splits == 1 && list_tokens == 0;
    return true;
}

// Hybrid decode: the listed tokens take splits of the same size after the
// window's (both split kernels read a token list).
bool add_list_splits(DecodePlan *plan, int32_t topk_k) {
    const int64_t n = plan->max_splits + ((int64_t)topk_k + plan->split_tokens - 1) / plan->split_tokens;
    if (n > 65535) return false;
    plan->max_splits = (int)n;
    plan->direct = 0;
    return true;
}

struct WorkspaceLayout {
    size_t o_bytes, lse_offset, total;
};

WorkspaceLayout workspace_layout(int32_t batch, int32_t heads_q, int32_t d_v, const DecodePlan &plan) {
    WorkspaceLayout w;
    const size_t slots = (size_t)batch * heads_q * plan.max_splits;
    // The latent kernel keeps its partial outputs in bf16, the others in fp32.
    w.o_bytes = slots * d_v * (plan.kind == ssa::kDecodeLatent ? 2 : sizeof(float));
    w.lse_offset = (w.o_bytes + 255) / 256 * 256;
    w.total = w.lse_offset + slots * sizeof(float);
    return w;
}

// Scratch of ssa_decode_noalloc: a fixed device array, one copy on each GPU
// the library runs on, held until the process ends. Host code never passes
// the array's name to a kernel (on the host it is only a stand-in for the
// device symbol): it takes the device address that hipGetSymbolAddress
// returns, found once per device with that device current.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];

// Device address of the scratch on the device `stream` runs on; null on a
// HIP failure.
void *device_scratch(hipStream_t stream) {
    int dev = -1;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return nullptr;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
        void *p = nullptr;
        const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (err != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

// Checks, plans and launches a decode-family call. With noalloc the
// workspace arguments are ignored and the call runs in the device scratch
// above (after every argument check, and only if it fits there).
ssa_status decode_common(ssa_dtype dtype, const void *q, const void *k_cache, const void *v_cache,
                         const int64_t k_strides[3], const int64_t v_strides[3],
                         const int32_t *page_table, int32_t max_pages, const int32_t *ctx_lens,
                         int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t d_qk, int32_t d_v,
                         int32_t page_size, void *o, float *lse, void *workspace,
                         size_t workspace_bytes, ssa_pattern pattern, float scale, bool full,
                         hipStream_t stream, const int32_t *topk = nullptr, int32_t topk_k = 0,
                         bool noalloc = false) {
    if (!dtype_ok(dtype)) return SSA_ERR_INVALID_ARG;
    if (topk_k < 0 || (topk_k > 0 && !topk && batch > 0)) return SSA_ERR_INVALID_ARG;
    if (batch < 0 || heads_q < 1 || heads_kv < 1 || heads_q % heads_kv || d_qk < 1 || d_v < 1 ||
        page_size < 1 || max_pages < 1)
        return SSA_ERR_INVALID_ARG;
    if (!full && !pattern_ok(pattern)) return SSA_ERR_INVALID_ARG;
    if (!(std::isfinite(scale) && scale > 0.f)) return SSA_ERR_INVALID_ARG;
    const int eb = elem_bytes(dtype);
    if (!strides_ok(k_strides, 3, eb) || !strides_ok(v_strides, 3, eb)) return SSA_ERR_INVALID_ARG;
    if (batch == 0) return SSA_OK;
    if (!q || !k_cache || !v_cache || !page_table || !ctx_lens || !o) return SSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
        return SSA_ERR_INVALID_ARG;
    if ((d_qk * eb) % 16 || (d_v * eb) % 16) return SSA_ERR_INVALID_ARG;

    DecodePlan plan;
    if (!make_plan(dtype, batch, heads_q, heads_kv, d_qk, d_v, page_size, max_pages, pattern, full, &plan,
                   topk_k))
        return SSA_ERR_UNSUPPORTED;
    if (topk_k > 0 && !add_list_splits(&plan, topk_k)) return SSA_ERR_UNSUPPORTED;
    if (topk_k > 0 && plan.kind == ssa::kDecodeLatent && plan.split_tokens > ssa::kDecodeLatentMaxListSplit)
        return SSA_ERR_UNSUPPORTED;  // the planner keeps latent splits within 1,024 tokens
    if (plan.kind == ssa::kDecodeLatent) {
        // The latent kernel reads the value as the first d_v entries of the key row.
        if (v_cache != k_cache || v_strides[0] != k_strides[0] || v_strides[1] != k_strides[1] ||
            v_strides[2] != k_strides[2])
            return SSA_ERR_UNSUPPORTED;
    }
    if ((int64_t)batch * heads_q > kInt32Max || (int64_t)heads_kv * plan.head_chunks > 65535 ||
        batch > 65535 || heads_q > 65535 ||
        (int64_t)plan.max_splits * heads_kv * plan.head_chunks * batch > kInt32Max)  // linear work-group ids
        return SSA_ERR_UNSUPPORTED;
    const WorkspaceLayout wl = workspace_layout(batch, heads_q, d_v, plan);
    if (noalloc) {
        if (wl.total > kNoAllocScratchBytes) return SSA_ERR_WORKSPACE;
        workspace = device_scratch(stream);
        if (!workspace) return SSA_ERR_HIP;
    } else if (!workspace || !aligned16(workspace) || workspace_bytes < wl.total) {
        return SSA_ERR_WORKSPACE;
    }

    DecodeArgs a{};
    a.q = q;
    a.kc = k_cache;
    a.vc = v_cache;
    for (int i = 0; i < 3; ++i) {
        a.ks[i] = k_strides[i];
        a.vs[i] = v_strides[i];
    }
    a.page_table = page_table;
    a.ctx_lens = ctx_lens;
    a.max_pages = max_pages;
    a.page_size = page_size;
    a.B = batch;
    a.Hq = heads_q;
    a.Hkv = heads_kv;
    a.group = heads_q / heads_kv;
    a.block = full ? 1 : pattern.block;
    a.sink = full ? 0 : pattern.sink;
    a.local = full ? 1 : pattern.local;
    a.full = full ? 1 : 0;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.o = o;
    a.lse = lse;
    a.ws_o = static_cast<float *>(workspace);
    a.ws_lse = reinterpret_cast<float *>(static_cast<char *>(workspace) + wl.lse_offset);
    a.plan = plan;
    a.topk = topk_k > 0 ? topk : nullptr;
    a.topk_k = topk_k;
    return ssa::launch_decode(dtype == SSA_BF16, d_qk, d_v, a, stream) == hipSuccess ? SSA_OK : SSA_ERR_HIP;
}

// Work plan of a backward call (shapes only).
struct BackwardPlan {
    int64_t n_pad, num_qtiles, sink_tiles, sink_rows, chunk_rows, n_chunks;
    int64_t dq_wgs, dkv_wgs, fin_wgs;
    size_t rowstat_bytes, part_offset, total;
};

// Rows of a key tile that holds sink keys are cut into chunks of about four
// times the rows a key past the sink is attended by (l*b), so that a chunk's
// work is a small multiple of an ordinary key tile's.
BackwardPlan backward_plan(int32_t batch, int32_t seq_len, int32_t heads_q, int32_t heads_kv,
                           int32_t d_qk, int32_t d_v, const ssa_pattern &p) {
    BackwardPlan b;
    b.n_pad = ((int64_t)seq_len + 127) / 128 * 128;
    b.num_qtiles = b.n_pad / 128;
    const int64_t sb = (int64_t)p.sink * p.block;
    const int64_t sink_keys = sb < seq_len ? sb : seq_len;
    b.sink_tiles = (sink_keys + 127) / 128;
    b.sink_rows = b.sink_tiles * 128 < seq_len ? b.sink_tiles * 128 : seq_len;
    int64_t span = (int64_t)p.local * p.block;
    span = span < b.n_pad ? span : b.n_pad;
    span = (span + 127) / 128 * 128;
    int64_t chunk = 4 * (span < 128 ? 128 : span);
    b.chunk_rows = chunk < b.n_pad ? chunk : b.n_pad;
    b.n_chunks = b.sink_tiles > 0 ? (seq_len + b.chunk_rows - 1) / b.chunk_rows : 0;
    b.dq_wgs = b.num_qtiles * heads_q * batch;
    b.dkv_wgs = (b.sink_tiles * b.n_chunks + (b.num_qtiles - b.sink_tiles)) * heads_kv * batch;
    const int64_t fin_items = (int64_t)batch * heads_kv * b.sink_rows * ((d_qk + d_v) / 4);
    b.fin_wgs = (fin_items + 255) / 256;
    b.rowstat_bytes = (size_t)batch * heads_q * b.n_pad * 2 * sizeof(float);
    b.part_offset = (b.rowstat_bytes + 255) / 256 * 256;
    b.total = b.part_offset +
              (size_t)b.n_chunks * batch * heads_kv * b.sink_rows * (d_qk + d_v) * sizeof(float);
    return b;
}

bool backward_shape_ok(ssa_dtype dtype, int32_t batch, int32_t seq_len, int32_t heads_q,
                       int32_t heads_kv, int32_t d_qk, int32_t d_v, const ssa_pattern &p) {
    return dtype_ok(dtype) && batch >= 0 && seq_len >= 0 && heads_q >= 1 && heads_kv >= 1 &&
           heads_q % heads_kv == 0 && d_qk >= 1 && d_v >= 1 && pattern_ok(p);
}

// Checks shared by the prefill entry points and the argument block they
// launch with. Returns SSA_OK with *empty set for a no-op call.
ssa_status prefill_common(ssa_dtype dtype, const void *q, const void *k, const void *v, void *o,
                          int32_t batch, int32_t seq_len, int32_t heads_q, int32_t heads_kv,
                          int32_t d_qk, int32_t d_v, const int64_t q_strides[3],
                          const int64_t k_strides[3], const int64_t v_strides[3],
                          const int64_t o_strides[3], const ssa_pattern &pattern, float scale,
                          PrefillArgs *a, bool *empty) {
    *empty = false;
    if (!dtype_ok(dtype)) return SSA_ERR_INVALID_ARG;
    if (batch < 0 || seq_len < 0 || heads_q < 1 || heads_kv < 1 || heads_q % heads_kv || d_qk < 1 ||
        d_v < 1)
        return SSA_ERR_INVALID_ARG;
    if (!pattern_ok(pattern) || !(std::isfinite(scale) && scale > 0.f)) return SSA_ERR_INVALID_ARG;
    const int eb = elem_bytes(dtype);
    if (!strides_ok(q_strides, 3, eb) || !strides_ok(k_strides, 3, eb) || !strides_ok(v_strides, 3, eb) ||
        !strides_ok(o_strides, 3, eb))
        return SSA_ERR_INVALID_ARG;
    if (batch == 0 || seq_len == 0) {
        *empty = true;
        return SSA_OK;
    }
    if (!q || !k || !v || !o) return SSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return SSA_ERR_INVALID_ARG;
    if (!ssa::prefill_supported(dtype == SSA_BF16, d_qk, d_v)) return SSA_ERR_UNSUPPORTED;
    // Kernels index positions in int32 and address a 64-key sub-tile with
    // 32-bit byte offsets from its first row.
    if (seq_len > kInt32Max - 256 || k_strides[1] >= (int64_t(1) << 24) ||
        v_strides[1] >= (int64_t(1) << 24))
        return SSA_ERR_UNSUPPORTED;

    const int64_t qtiles = ((int64_t)seq_len + 127) / 128;
    const int64_t total = qtiles * heads_q * batch;
    // a 1-D grid holds fewer than 2^32 work-items: 256 per work-group
    if (total >= (int64_t(1) << 24)) return SSA_ERR_UNSUPPORTED;

    *a = PrefillArgs{};
    a->q = q;
    a->k = k;
    a->v = v;
    a->o = o;
    for (int i = 0; i < 3; ++i) {
        a->qs[i] = q_strides[i];
        a->ks[i] = k_strides[i];
        a->vs[i] = v_strides[i];
        a->os[i] = o_strides[i];
    }
    a->B = batch;
    a->N = seq_len;
    a->Hq = heads_q;
    a->Hkv = heads_kv;
    a->group = heads_q / heads_kv;
    a->block = pattern.block;
    a->sink = pattern.sink;
    a->local = pattern.local;
    a->scale_log2 = scale * 1.4426950408889634f;
    a->num_qtiles = (int32_t)qtiles;
    a->total_wgs = (int32_t)total;
    return SSA_OK;
}


// Chunks up to this many rows per sequence go to the decode kernels (one
// work-group per split of a row's window) when they support the shape; longer
// ones to the paged tile kernel, which reads a window once per 128 rows.
// Measured (16 heads, d = 128, 16-64 sequences at 32K): the two tie at one
// row, and the tile kernel is 1.2x faster at two rows and 3.4x at eight.
constexpr int32_t kExtendDecodeMaxRows = 1;

struct ExtendPlan {
    bool tiles;             // paged tile kernel, else decode kernels over query rows
    DecodePlan dplan;       // decode path
    size_t rows_bytes;      // decode path: row map (row_seq, row_ctx) at the workspace start
    WorkspaceLayout wl;     // decode path: partials after the row map
    size_t total;
};

bool extend_plan(ssa_dtype dtype, int32_t total_q, int32_t max_q_len, int32_t heads_q,
                 int32_t heads_kv, int32_t d_qk, int32_t d_v, int32_t page_size, int32_t max_pages,
                 const ssa_pattern &pattern, ExtendPlan *p) {
    const bool tiles_ok = ssa::prefill_paged_supported(dtype == SSA_BF16, d_qk, d_v);
    DecodePlan dp;
    const bool dec_ok = make_plan(dtype, total_q, heads_q, heads_kv, d_qk, d_v, page_size, max_pages,
                                  pattern, false, &dp);
    if (!tiles_ok && !dec_ok) return false;
    *p = ExtendPlan{};
    p->tiles = tiles_ok && (!dec_ok || max_q_len > kExtendDecodeMaxRows);
    if (p->tiles) return true;
    p->dplan = dp;
    p->rows_bytes = ((size_t)total_q * 2 * sizeof(int32_t) + 255) / 256 * 256;
    p->wl = workspace_layout(total_q, heads_q, d_v, dp);
    p->total = p->rows_bytes + p->wl.total;
    return true;
}

bool extend_shape_ok(ssa_dtype dtype, int32_t batch, int32_t total_q, int32_t max_q_len,
                     int32_t heads_q, int32_t heads_kv, int32_t d_qk, int32_t d_v, int32_t page_size,
                     int32_t max_pages, const ssa_pattern &pattern) {
    return dtype_ok(dtype) && batch >= 0 && total_q >= 0 && max_q_len >= 0 && heads_q >= 1 &&
           heads_kv >= 1 && heads_q % heads_kv == 0 && d_qk >= 1 && d_v >= 1 && page_size >= 1 &&
           max_pages >= 1 && pattern_ok(pattern) && (total_q == 0 || max_q_len >= 1);
}

}  // namespace

extern "C" {

ssa_status ssa_prefill(ssa_dtype dtype, const void *q, const void *k, const void *v, void *o,
                       float *lse, int32_t batch, int32_t seq_len, int32_t heads_q,
                       int32_t heads_kv, int32_t d_qk, int32_t d_v, const int64_t q_strides[3],
                       const int64_t k_strides[3], const int64_t v_strides[3],
                       const int64_t o_strides[3], ssa_pattern pattern, float scale,
                       hipStream_t stream) {
    PrefillArgs a;
    bool empty;
    const ssa_status st = prefill_common(dtype, q, k, v, o, batch, seq_len, heads_q, heads_kv, d_qk,
                                         d_v, q_strides, k_strides, v_strides, o_strides, pattern,
                                         scale, &a, &empty);
    if (st != SSA_OK || empty) return st;
    a.lse = lse;
    return ssa::launch_prefill(dtype == SSA_BF16, d_qk, d_v, a, stream) == hipSuccess ? SSA_OK
                                                                                     : SSA_ERR_HIP;
}

ssa_status ssa_prefill_dual(ssa_dtype dtype, const void *q, const void *k, const void *v,
                            void *o_ssa, float *lse_ssa, void *o_full, float *lse_full, void *o_mix,
                            float alpha, int32_t batch, int32_t seq_len, int32_t heads_q,
                            int32_t heads_kv, int32_t d_qk, int32_t d_v,
                            const int64_t q_strides[3], const int64_t k_strides[3],
                            const int64_t v_strides[3], const int64_t o_strides[3],
                            ssa_pattern pattern, float scale, hipStream_t stream) {
    if (!(alpha >= 0.f && alpha <= 1.f)) return SSA_ERR_INVALID_ARG;  // also rejects NaN
    PrefillArgs a;
    bool empty;
    const ssa_status st = prefill_common(dtype, q, k, v, o_ssa, batch, seq_len, heads_q, heads_kv,
                                         d_qk, d_v, q_strides, k_strides, v_strides, o_strides,
                                         pattern, scale, &a, &empty);
    if (st != SSA_OK || empty) return st;
    if (!o_full || !aligned16(o_full) || (o_mix && !aligned16(o_mix))) return SSA_ERR_INVALID_ARG;
    if (o_full == o_ssa || o_mix == o_ssa || o_mix == o_full) return SSA_ERR_INVALID_ARG;
    if (!ssa::prefill_dual_supported(dtype == SSA_BF16, d_qk, d_v)) return SSA_ERR_UNSUPPORTED;
    a.lse = lse_ssa;
    a.o_full = o_full;
    a.lse_full = lse_full;
    a.o_mix = o_mix;
    a.alpha = alpha;
    return ssa::launch_prefill_dual(dtype == SSA_BF16, d_qk, d_v, a, stream) == hipSuccess
               ? SSA_OK
               : SSA_ERR_HIP;
}

ssa_status ssa_prefill_backward(ssa_dtype dtype, const void *q, const void *k, const void *v,
                                const void *o, const float *lse, const void *dout, void *dq,
                                void *dk, void *dv, int32_t batch, int32_t seq_len,
                                int32_t heads_q, int32_t heads_kv, int32_t d_qk, int32_t d_v,
                                const int64_t q_strides[3], const int64_t k_strides[3],
                                const int64_t v_strides[3], const int64_t o_strides[3],
                                const int64_t do_strides[3], const int64_t dq_strides[3],
                                const int64_t dk_strides[3], const int64_t dv_strides[3],
                                void *workspace, size_t workspace_bytes, ssa_pattern pattern,
                                float scale, hipStream_t stream) {
    if (!backward_shape_ok(dtype, batch, seq_len, heads_q, heads_kv, d_qk, d_v, pattern))
        return SSA_ERR_INVALID_ARG;
    if (!(std::isfinite(scale) && scale > 0.f)) return SSA_ERR_INVALID_ARG;
    const int eb = elem_bytes(dtype);
    const int64_t *all_strides[8] = {q_strides, k_strides, v_strides, o_strides,
                                     do_strides, dq_strides, dk_strides, dv_strides};
    for (const int64_t *st : all_strides)
        if (!strides_ok(st, 3, eb)) return SSA_ERR_INVALID_ARG;
    if (batch == 0 || seq_len == 0) return SSA_OK;
    const void *ptrs[10] = {q, k, v, o, lse, dout, dq, dk, dv, workspace};
    for (int n = 0; n < 9; ++n)
        if (!ptrs[n] || !aligned16(ptrs[n])) return SSA_ERR_INVALID_ARG;
    if (!ssa::backward_supported(dtype == SSA_BF16, d_qk, d_v)) return SSA_ERR_UNSUPPORTED;
    // Kernels index positions in int32 and address a 64-row tile with 32-bit
    // byte offsets from its first row.
    if (seq_len > kInt32Max - 256 || k_strides[1] >= (int64_t(1) << 24) ||
        v_strides[1] >= (int64_t(1) << 24) || q_strides[1] >= (int64_t(1) << 24) ||
        do_strides[1] >= (int64_t(1) << 24))
        return SSA_ERR_UNSUPPORTED;
    const BackwardPlan pl = backward_plan(batch, seq_len, heads_q, heads_kv, d_qk, d_v, pattern);
    if (pl.dq_wgs >= (int64_t(1) << 24) || pl.dkv_wgs >= (int64_t(1) << 24) ||
        pl.fin_wgs >= (int64_t(1) << 24) || pl.n_chunks * batch * heads_kv > kInt32Max)
        return SSA_ERR_UNSUPPORTED;
    if (!workspace || !aligned16(workspace) || workspace_bytes < pl.total) return SSA_ERR_WORKSPACE;

    ssa::BackwardArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dout = dout;
    a.lse = lse;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    for (int i = 0; i < 3; ++i) {
        a.qs[i] = q_strides[i];
        a.ks[i] = k_strides[i];
        a.vs[i] = v_strides[i];
        a.os[i] = o_strides[i];
        a.dos[i] = do_strides[i];
        a.dqs[i] = dq_strides[i];
        a.dks[i] = dk_strides[i];
        a.dvs[i] = dv_strides[i];
    }
    a.B = batch;
    a.N = seq_len;
    a.Hq = heads_q;
    a.Hkv = heads_kv;
    a.group = heads_q / heads_kv;
    a.block = pattern.block;
    a.sink = pattern.sink;
    a.local = pattern.local;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.rowstat = static_cast<float *>(workspace);
    a.sink_part = reinterpret_cast<float *>(static_cast<char *>(workspace) + pl.part_offset);
    a.n_pad = (int32_t)pl.n_pad;
    a.num_qtiles = (int32_t)pl.num_qtiles;
    a.sink_tiles = (int32_t)pl.sink_tiles;
    a.sink_rows = (int32_t)pl.sink_rows;
    a.chunk_rows = (int32_t)pl.chunk_rows;
    a.n_chunks = (int32_t)pl.n_chunks;
    a.dq_wgs = (int32_t)pl.dq_wgs;
    a.dkv_wgs = (int32_t)pl.dkv_wgs;
    a.fin_wgs = (int32_t)pl.fin_wgs;
    return ssa::launch_backward(dtype == SSA_BF16, d_qk, d_v, a, stream) == hipSuccess ? SSA_OK
                                                                                       : SSA_ERR_HIP;
}

size_t ssa_prefill_backward_workspace_size(ssa_dtype dtype, int32_t batch, int32_t seq_len,
                                           int32_t heads_q, int32_t heads_kv, int32_t d_qk,
                                           int32_t d_v, ssa_pattern pattern) {
    if (!backward_shape_ok(dtype, batch, seq_len, heads_q, heads_kv, d_qk, d_v, pattern)) return 0;
    if (!ssa::backward_supported(dtype == SSA_BF16, d_qk, d_v)) return 0;
    if (batch == 0 || seq_len == 0) return 0;
    return backward_plan(batch, seq_len, heads_q, heads_kv, d_qk, d_v, pattern).total;
}

ssa_status ssa_decode(ssa_dtype dtype, const void *q, const void *k_cache, const void *v_cache,
                      const int64_t k_strides[3], const int64_t v_strides[3],
                      const int32_t *page_table, int32_t max_pages, const int32_t *ctx_lens,
                      int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t d_qk, int32_t d_v,
                      int32_t page_size, void *o, float *lse, void *workspace,
                      size_t workspace_bytes, ssa_pattern pattern, float scale, hipStream_t stream) {
    return decode_common(dtype, q, k_cache, v_cache, k_strides, v_strides, page_table, max_pages,
                         ctx_lens, batch, heads_q, heads_kv, d_qk, d_v, page_size, o, lse, workspace,
                         workspace_bytes, pattern, scale, false, stream);
}

ssa_status ssa_decode_noalloc(ssa_dtype dtype, const void *q, const void *k_cache, const void *v_cache,
                              const int64_t k_strides[3], const int64_t v_strides[3],
                              const int32_t *page_table, int32_t max_pages, const int32_t *ctx_lens,
                              int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t d_qk,
                              int32_t d_v, int32_t page_size, void *o, float *lse, ssa_pattern pattern,
                              float scale, hipStream_t stream) {
    return decode_common(dtype, q, k_cache, v_cache, k_strides, v_strides, page_table, max_pages,
                         ctx_lens, batch, heads_q, heads_kv, d_qk, d_v, page_size, o, lse, nullptr, 0,
                         pattern, scale, false, stream, nullptr, 0, true);
}

ssa_status full_attn_decode(ssa_dtype dtype, const void *q, const void *k_cache, const void *v_cache,
                            const int64_t k_strides[3], const int64_t v_strides[3],
                            const int32_t *page_table, int32_t max_pages, const int32_t *ctx_lens,
                            int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t d_qk,
                            int32_t d_v, int32_t page_size, void *o, float *lse, void *workspace,
                            size_t workspace_bytes, float scale, hipStream_t stream) {
    const ssa_pattern unused = {1, 0, 1};
    return decode_common(dtype, q, k_cache, v_cache, k_strides, v_strides, page_table, max_pages,
                         ctx_lens, batch, heads_q, heads_kv, d_qk, d_v, page_size, o, lse, workspace,
                         workspace_bytes, unused, scale, true, stream);
}

size_t ssa_decode_workspace_size(ssa_dtype dtype, int32_t batch, int32_t heads_q, int32_t heads_kv,
                                 int32_t d_qk, int32_t d_v, int32_t page_size, int32_t max_pages,
                                 ssa_pattern pattern, int full) {
    if (!dtype_ok(dtype) || batch < 1 || heads_q < 1 || heads_kv < 1 || heads_q % heads_kv ||
        page_size < 1 || max_pages < 1 || d_qk < 1 || d_v < 1)
        return 0;
    if (!full && !pattern_ok(pattern)) return 0;
    DecodePlan plan;
    if (!make_plan(dtype, batch, heads_q, heads_kv, d_qk, d_v, page_size, max_pages, pattern, full != 0,
                   &plan))
        return 0;
    return workspace_layout(batch, heads_q, d_v, plan).total;
}

ssa_status ssa_extend(ssa_dtype dtype, const void *q, const void *k_cache, const void *v_cache,
                      const int64_t k_strides[3], const int64_t v_strides[3],
                      const int32_t *page_table, int32_t max_pages, const int32_t *ctx_lens,
                      const int32_t *cu_q, int32_t batch, int32_t total_q, int32_t max_q_len,
                      int32_t heads_q, int32_t heads_kv, int32_t d_qk, int32_t d_v,
                      int32_t page_size, void *o, float *lse, void *workspace,
                      size_t workspace_bytes, ssa_pattern pattern, float scale,
                      hipStream_t stream) {
    if (!extend_shape_ok(dtype, batch, total_q, max_q_len, heads_q, heads_kv, d_qk, d_v, page_size,
                         max_pages, pattern))
        return SSA_ERR_INVALID_ARG;
    if (!(std::isfinite(scale) && scale > 0.f)) return SSA_ERR_INVALID_ARG;
    const int eb = elem_bytes(dtype);
    if (!strides_ok(k_strides, 3, eb) || !strides_ok(v_strides, 3, eb)) return SSA_ERR_INVALID_ARG;
    if (batch == 0 || total_q == 0) return SSA_OK;
    if (!q || !k_cache || !v_cache || !page_table || !ctx_lens || !cu_q || !o) return SSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
        return SSA_ERR_INVALID_ARG;
    if ((d_qk * eb) % 16 || (d_v * eb) % 16) return SSA_ERR_INVALID_ARG;

    ExtendPlan plan;
    if (!extend_plan(dtype, total_q, max_q_len, heads_q, heads_kv, d_qk, d_v, page_size, max_pages,
                     pattern, &plan))
        return SSA_ERR_UNSUPPORTED;

    if (plan.tiles) {
        // Lane offsets inside a 64-row sub-tile are 32-bit.
        if (k_strides[1] >= (int64_t(1) << 24) || v_strides[1] >= (int64_t(1) << 24))
            return SSA_ERR_UNSUPPORTED;
        const int64_t qtiles = ((int64_t)max_q_len + 127) / 128;
        const int64_t total = qtiles * heads_q * batch;
        if (total >= (int64_t(1) << 24)) return SSA_ERR_UNSUPPORTED;
        PrefillArgs a{};
        a.q = q;
        a.k = k_cache;
        a.v = v_cache;
        a.o = o;
        a.lse = lse;
        a.qs[0] = 0;
        a.qs[1] = (int64_t)heads_q * d_qk;
        a.qs[2] = d_qk;
        a.os[0] = 0;
        a.os[1] = (int64_t)heads_q * d_v;
        a.os[2] = d_v;
        for (int i = 0; i < 3; ++i) {
            a.ks[i] = k_strides[i];
            a.vs[i] = v_strides[i];
        }
        a.B = batch;
        a.N = 0;
        a.Hq = heads_q;
        a.Hkv = heads_kv;
        a.group = heads_q / heads_kv;
        a.block = pattern.block;
        a.sink = pattern.sink;
        a.local = pattern.local;
        a.scale_log2 = scale * 1.4426950408889634f;
        a.num_qtiles = (int32_t)qtiles;
        a.total_wgs = (int32_t)total;
        a.page_table = page_table;
        a.ctx_lens = ctx_lens;
        a.cu_q = cu_q;
        a.max_pages = max_pages;
        a.page_size = page_size;
        return ssa::launch_prefill_paged(dtype == SSA_BF16, d_qk, d_v, a, stream) == hipSuccess
                   ? SSA_OK
                   : SSA_ERR_HIP;
    }

    const DecodePlan &dp = plan.dplan;
    if (dp.kind == ssa::kDecodeLatent &&
        (v_cache != k_cache || v_strides[0] != k_strides[0] || v_strides[1] != k_strides[1] ||
         v_strides[2] != k_strides[2]))
        return SSA_ERR_UNSUPPORTED;
    if ((int64_t)total_q * heads_q > kInt32Max || (int64_t)heads_kv * dp.head_chunks > 65535 ||
        total_q > 65535 || batch > 65535 || heads_q > 65535 ||
        (int64_t)dp.max_splits * heads_kv * dp.head_chunks * total_q > kInt32Max)
        return SSA_ERR_UNSUPPORTED;
    if (!workspace || !aligned16(workspace) || workspace_bytes < plan.total) return SSA_ERR_WORKSPACE;

    char *ws = static_cast<char *>(workspace);
    int32_t *row_seq = reinterpret_cast<int32_t *>(ws);
    int32_t *row_ctx = row_seq + total_q;
    DecodeArgs a{};
    a.q = q;
    a.kc = k_cache;
    a.vc = v_cache;
    for (int i = 0; i < 3; ++i) {
        a.ks[i] = k_strides[i];
        a.vs[i] = v_strides[i];
    }
    a.page_table = page_table;
    a.ctx_lens = ctx_lens;
    a.max_pages = max_pages;
    a.page_size = page_size;
    a.B = total_q;
    a.Hq = heads_q;
    a.Hkv = heads_kv;
    a.group = heads_q / heads_kv;
    a.block = pattern.block;
    a.sink = pattern.sink;
    a.local = pattern.local;
    a.full = 0;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.o = o;
    a.lse = lse;
    a.ws_o = reinterpret_cast<float *>(ws + plan.rows_bytes);
    a.ws_lse = reinterpret_cast<float *>(ws + plan.rows_bytes + plan.wl.lse_offset);
    a.plan = dp;
    a.row_seq = row_seq;
    a.row_ctx = row_ctx;
    a.n_seqs = batch;
    if (ssa::launch_extend_rows(cu_q, ctx_lens, batch, max_q_len, total_q, row_seq, row_ctx, stream) !=
        hipSuccess)
        return SSA_ERR_HIP;
    return ssa::launch_decode(dtype == SSA_BF16, d_qk, d_v, a, stream) == hipSuccess ? SSA_OK : SSA_ERR_HIP;
}

size_t ssa_extend_workspace_size(ssa_dtype dtype, int32_t batch, int32_t total_q, int32_t max_q_len,
                                 int32_t heads_q, int32_t heads_kv, int32_t d_qk, int32_t d_v,
                                 int32_t page_size, int32_t max_pages, ssa_pattern pattern) {
    if (!extend_shape_ok(dtype, batch, total_q, max_q_len, heads_q, heads_kv, d_qk, d_v, page_size,
                         max_pages, pattern) ||
        batch == 0 || total_q == 0)
        return 0;
    ExtendPlan plan;
    if (!extend_plan(dtype, total_q, max_q_len, heads_q, heads_kv, d_qk, d_v, page_size, max_pages,
                     pattern, &plan))
        return 0;
    return plan.total;
}

ssa_status hybrid_decode(ssa_dtype dtype, const void *q, const void *k_cache, const void *v_cache,
                         const int64_t k_strides[3], const int64_t v_strides[3],
                         const int32_t *page_table, int32_t max_pages, const int32_t *ctx_lens,
                         const int32_t *topk, int32_t topk_k, int32_t batch, int32_t heads_q,
                         int32_t heads_kv, int32_t d_qk, int32_t d_v, int32_t page_size, void *o,
                         float *lse, void *workspace, size_t workspace_bytes, ssa_pattern pattern,
                         float scale, hipStream_t stream) {
    if (topk_k < 1) return SSA_ERR_INVALID_ARG;
    return decode_common(dtype, q, k_cache, v_cache, k_strides, v_strides, page_table, max_pages,
                         ctx_lens, batch, heads_q, heads_kv, d_qk, d_v, page_size, o, lse, workspace,
                         workspace_bytes, pattern, scale, false, stream, topk, topk_k);
}

size_t hybrid_decode_workspace_size(ssa_dtype dtype, int32_t batch, int32_t heads_q, int32_t heads_kv,
                                    int32_t d_qk, int32_t d_v, int32_t page_size, int32_t max_pages,
                                    int32_t topk_k, ssa_pattern pattern) {
    if (!dtype_ok(dtype) || batch < 1 || heads_q < 1 || heads_kv < 1 || heads_q % heads_kv ||
        page_size < 1 || max_pages < 1 || d_qk < 1 || d_v < 1 || topk_k < 1 || !pattern_ok(pattern))
        return 0;
    DecodePlan plan;
    if (!make_plan(dtype, batch, heads_q, heads_kv, d_qk, d_v, page_size, max_pages, pattern, false,
                   &plan, topk_k) ||
        !add_list_splits(&plan, topk_k))
        return 0;
    return workspace_layout(batch, heads_q, d_v, plan).total;
}

const char *ssa_status_string(ssa_status status) {
    switch (status) {
        case SSA_OK: return "SSA_OK";
        case SSA_ERR_INVALID_ARG: return "SSA_ERR_INVALID_ARG: bad size, stride, pattern, scale or pointer";
        case SSA_ERR_UNSUPPORTED: return "SSA_ERR_UNSUPPORTED: no compiled kernel for this dtype/shape";
        case SSA_ERR_WORKSPACE: return "SSA_ERR_WORKSPACE: workspace missing, misaligned or too small";
        case SSA_ERR_HIP: return "SSA_ERR_HIP: kernel launch failed";
    }
    return "unknown ssa_status";
}

}  // extern "C"
