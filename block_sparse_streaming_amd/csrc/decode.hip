// Streaming sparse attention decode (and the dense full-attention decode) over a
// paged KV cache, for gfx950.
//
// Operation: one new query per sequence at position L-1 (its key/value already
// in the cache). SSA attends to the keys j <= L-1 with j < s*b or
// j >= ((L-1)/b - l + 1)*b (LongCat ZigZag Attention digest, section 01 part
// (1), the SSA paragraph; section 02 compares this streaming sparse decode
// kernel with a full-attention decode kernel, which attends to all of 0..L-1).
//
// The attended keys are two contiguous token ranges, R1 = [0, min(sb, L)) and
// R2 = [max(sb, (qb-l+1)b), L); the full kernel uses R1 = [0, L). Their
// concatenation is cut into splits of `split_tokens` tokens; one work-group
// computes a split's partial softmax (normalised output + log2-sum-exp) into
// the workspace and a second kernel merges the splits of each (sequence, head)
// with log-sum-exp weights. Page translation is per token: token t is at
// page_table[t / P], slot t % P, so consecutive tokens are consecutive rows of
// a page and every gather is a run of full rows.
//
// Two split kernels:
//  * decode_split_valu: 16 lanes per token, a group of G <= 8 query heads per
//    kv head, fp32 or bf16, head dim 64/128/256. Memory-bound GEMV work, so it
//    stays on the VALU; each lane keeps its own online-softmax state and the
//    16 token groups of a work-group are merged through LDS.
//  * decode_split_latent: the absorbed-MLA shape (576-dim latent row whose
//    first 512 entries are the value), up to 64 query heads per kv head. Each
//    split is a 64x576x(tokens) and a 64x(tokens)x512 product, so it runs on
//    v_mfma_f32_16x16x32_bf16: S^T = K q^T (one 16-head column block per wave),
//    then O^T = V^T P^T with P taken straight from the score registers. Chunks
//    of 32 latent rows stream global -> LDS through a 4-deep ring (three
//    chunks requested at the start, the next one as each chunk is taken);
//    each row is stored once and the V^T operand is gathered from it with
//    transpose reads.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace ssa {
namespace {

struct Sel {
    int64_t r1_end;    // R1 = [0, r1_end)
    int64_t r2_begin;  // R2 = [r2_begin, L)
    int64_t total;     // |R1| + |R2|
};

// Context length (query position + 1) and page-table row of query row r.
// Row-map entries are clamped to the table (a row the map left unwritten,
// of a chunk longer than max_q_len, reads only valid pages).
// Context length of query row r, clamped to the page table's capacity so that
// no length reads past its table row.
__device__ __forceinline__ int64_t row_context(const DecodeArgs &a, int r) {
    const int64_t L = a.row_ctx ? a.row_ctx[r] : a.ctx_lens[r], cap = (int64_t)a.max_pages * a.page_size;
    return L < cap ? L : cap;
}
__device__ __forceinline__ int64_t row_sequence(const DecodeArgs &a, int r) {
    if (!a.row_seq) return r;
    const int s = a.row_seq[r];
    return s < 0 ? 0 : (s >= a.n_seqs ? a.n_seqs - 1 : s);
}

// Splits of the listed tokens (hybrid decode); they follow the window's.
__device__ __forceinline__ int list_splits(const DecodeArgs &a) {
    return a.topk_k > 0 ? (a.topk_k + a.plan.split_tokens - 1) / a.plan.split_tokens : 0;
}

__device__ __forceinline__ Sel select_tokens(int64_t L, const DecodeArgs &a) {
    if (a.full) return Sel{L, L, L};
    const int64_t b = a.block, sb = (int64_t)a.sink * b;
    const int64_t qb = (int64_t)((uint32_t)(L - 1) / (uint32_t)a.block);  // L <= INT32_MAX
    const int64_t r1 = sb < L ? sb : L;
    const int64_t lo0 = (qb - a.local + 1) * b;
    const int64_t lo = lo0 > sb ? lo0 : sb;
    const int64_t n2 = L > lo ? L - lo : 0;
    return Sel{r1, lo, r1 + n2};
}

// ---------------------------------------------------------------------------
// VALU split kernel.
// ---------------------------------------------------------------------------
constexpr int kValuThreads = 256;
constexpr int kTpt = 16;                       // lanes per token
constexpr int kGroups = kValuThreads / kTpt;   // token groups per work-group

// E elements of one lane's slice of a cache row, kept as raw 32-bit words.
template <typename Elem, int E>
struct RowSlice {
    static constexpr int kWords = E * (int)sizeof(Elem) / 4;
    uint32_t w[kWords];
};

// kStream: the rows are read once per call (cache rows), so the loads carry
// the non-temporal hint. Measured on the ragged 65-sequence batch: 93-94 us
// per call with plain loads, 88.5-90.5 us with the hint (the latent kernel's
// direct transfers with the same hint were slower, and q, which the splits
// of a row share, stays cached).
template <typename Elem, int E, bool kStream = false>
__device__ __forceinline__ void load_slice(const Elem *p, RowSlice<Elem, E> &r) {
    constexpr int W = RowSlice<Elem, E>::kWords;
    if constexpr (W >= 4) {
#pragma unroll
        for (int c = 0; c < W / 4; ++c) {
            const u32x4 *src = (const u32x4 *)((const uint32_t *)p + 4 * c);
            u32x4 v;
            if constexpr (kStream) v = __builtin_nontemporal_load(src);
            else v = *src;
#pragma unroll
            for (int e = 0; e < 4; ++e) r.w[4 * c + e] = v[e];
        }
    } else {
        u32x2 v;
        if constexpr (kStream) v = __builtin_nontemporal_load((const u32x2 *)p);
        else v = *(const u32x2 *)p;
        r.w[0] = v[0];
        r.w[1] = v[1];
    }
}

template <typename Elem, int E>
__device__ __forceinline__ float slice_elem(const RowSlice<Elem, E> &r, int e) {
    if constexpr (std::is_same_v<Elem, float>) return __uint_as_float(r.w[e]);
    else return (e & 1) ? bf16_hi(r.w[e >> 1]) : bf16_lo(r.w[e >> 1]);
}

// One work-group computes one split (up to split_tokens attended tokens) for
// the G query heads of one kv head. Sixteen lanes share a token (each holds
// D/16 elements of its key and value rows); the sixteen token groups of the
// work-group take interleaved positions. A chunk gives every lane TPL tokens
// whose rows are all requested at once; the next chunk's page ids are read
// while this chunk's rows are in flight. Each lane keeps its own online
// softmax state, and the token groups are merged through LDS at the end.
// kList: the call has listed tokens (hybrid decode); without them the
// window-only path keeps no per-token state between the page-id read and the
// row read.
template <bool kBF16, int D, int G, bool kList>
__global__ __launch_bounds__(kValuThreads) void decode_split_valu(const DecodeArgs a) {
    using Elem = std::conditional_t<kBF16, uint16_t, float>;
    constexpr int E = D / kTpt;
    using Slice = RowSlice<Elem, E>;
    constexpr int kTpl = Slice::kWords <= 4 ? 8 : 32 / Slice::kWords;  // tokens per lane per chunk
    constexpr int kChunk = kGroups * kTpl;
    __shared__ float sm_m[kGroups][G];
    __shared__ float sm_l[kGroups][G];
    __shared__ float sm_o[kGroups][G][D];

    const int split = blockIdx.x, g = blockIdx.y, bb = blockIdx.z;
    const int tid = threadIdx.x, tg = tid / kTpt, tl = tid % kTpt;
    // One split per row (a.plan.direct): the result goes straight to o and
    // lse, as the merge would write it for a single split.
    auto put_out = [&](int hh, int d, float v, float lse2) __attribute__((always_inline)) {
        const int64_t row = (int64_t)bb * a.Hq + g * G + hh;
        if constexpr (kBF16) ((uint16_t *)a.o)[row * D + d] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xffffu);
        else ((float *)a.o)[row * D + d] = v;
        if (d == 0 && a.lse) a.lse[row] = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
    };
    // A split slot past the row's splits holds lse = -inf, so the merge needs
    // neither the context length nor the split count. Written directly, a row
    // with no attended key has o = 0 and lse = -inf.
    auto no_split = [&]() __attribute__((always_inline)) {
        if (a.plan.direct) {
            for (int t = tid; t < G * D; t += kValuThreads) put_out(t / D, t % D, 0.f, -INFINITY);
            return;
        }
        for (int hh = tid; hh < G; hh += kValuThreads)
            a.ws_lse[((int64_t)bb * a.Hq + g * G + hh) * a.plan.max_splits + split] = -INFINITY;
    };
    const int64_t L = row_context(a, bb);
    if (L <= 0) {
        no_split();
        return;
    }
    const Sel sel = select_tokens(L, a);
    // Splits [0, n_win) cover the window's positions; the next list_splits(a)
    // cover the listed tokens (hybrid decode), positions of the list.
    const int n_win = (int)((sel.total + a.plan.split_tokens - 1) / a.plan.split_tokens);
    const bool listed = kList && split >= n_win;
    const int64_t p_begin = (int64_t)(listed ? split - n_win : split) * a.plan.split_tokens;
    const int64_t p_lim = listed ? (int64_t)a.topk_k : sel.total;
    if (p_begin >= p_lim) {
        no_split();
        return;
    }
    const int64_t p_end = p_begin + a.plan.split_tokens < p_lim ? p_begin + a.plan.split_tokens : p_lim;
    // Positions and tokens fit in 32 bits (context lengths are int32).
    const uint32_t up_end = (uint32_t)p_end, ur1 = (uint32_t)sel.r1_end, ur2 = (uint32_t)sel.r2_begin;
    const uint32_t uP = (uint32_t)a.page_size;
    const int64_t seq = row_sequence(a, bb);
    const int32_t *ptab = a.page_table + seq * a.max_pages;
    const uint32_t uL = (uint32_t)L, ur2end = ur2 < uL ? ur2 : uL;
    // Token of a window position (clamped to the split's last position).
    auto window_token = [&](uint32_t c0, int u) __attribute__((always_inline)) -> uint32_t {
        uint32_t pp = c0 + (uint32_t)(tg + kGroups * u);
        pp = pp < up_end ? pp : up_end - 1;
        return pp < ur1 ? pp : ur2 + (pp - ur1);
    };

    // Token of lane group tg's u-th position in the chunk starting at c0
    // (clamped to the split's last position; masked later). A listed token
    // inside the window, past the context or negative is skipped: token 0
    // stands in for it and its bit in `ok` is clear.
    auto token_of = [&](uint32_t c0, int u, bool &ok) __attribute__((always_inline)) -> uint32_t {
        if (!listed) {
            ok = true;
            return window_token(c0, u);
        }
        uint32_t pp = c0 + (uint32_t)(tg + kGroups * u);
        pp = pp < up_end ? pp : up_end - 1;
        const int t0 = a.topk[seq * a.topk_k + pp];
        ok = t0 >= (int)ur1 && (uint32_t)t0 < ur2end;
        return ok ? (uint32_t)t0 : 0u;
    };
    // Page ids of the next chunk, and with a list its tokens and attended bits.
    int32_t pid[kTpl];
    uint32_t tok_next[kList ? kTpl : 1];
    uint32_t ok_next = 0xffffffffu;
    auto load_pids = [&](uint32_t c0) __attribute__((always_inline)) {
        if constexpr (kList) {
            ok_next = 0;
#pragma unroll
            for (int u = 0; u < kTpl; ++u) {
                bool ok;
                tok_next[u] = token_of(c0, u, ok);
                ok_next |= (ok ? 1u : 0u) << u;
                pid[u] = ptab[tok_next[u] / uP];
            }
        } else {
#pragma unroll
            for (int u = 0; u < kTpl; ++u) pid[u] = ptab[window_token(c0, u) / uP];
        }
    };
    Slice kr[kTpl], vr[kTpl];
    const Elem *kc = (const Elem *)a.kc + g * a.ks[2] + tl * E;
    const Elem *vc = (const Elem *)a.vc + g * a.vs[2] + tl * E;
    auto load_rows = [&](uint32_t c0) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kTpl; ++u) {
            uint32_t tok;
            if constexpr (kList) tok = tok_next[u];
            else tok = window_token(c0, u);
            const int64_t slot = (int64_t)(tok % uP);
            load_slice<Elem, E, true>(kc + pid[u] * a.ks[0] + slot * a.ks[1], kr[u]);
            load_slice<Elem, E, true>(vc + pid[u] * a.vs[0] + slot * a.vs[1], vr[u]);
        }
    };

    const uint32_t c_first = (uint32_t)p_begin;
    load_pids(c_first);
    float qv[G][E];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        const Elem *qp = (const Elem *)a.q + ((int64_t)bb * a.Hq + g * G + hh) * D + tl * E;
        Slice qs;
        load_slice<Elem, E>(qp, qs);
#pragma unroll
        for (int e = 0; e < E; ++e) qv[hh][e] = slice_elem<Elem, E>(qs, e) * a.scale_log2;
    }

    float m[G], ls[G], acc[G][E];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        m[hh] = -INFINITY;
        ls[hh] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[hh][e] = 0.f;
    }

    for (uint32_t c0 = c_first; c0 < up_end; c0 += kChunk) {
        load_rows(c0);
        const uint32_t ok_cur = ok_next;
        if (c0 + kChunk < up_end) load_pids(c0 + kChunk);
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            float s[kTpl];
#pragma unroll
            for (int u = 0; u < kTpl; ++u) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) d += qv[hh][e] * slice_elem<Elem, E>(kr[u], e);
                d += __shfl_xor(d, 8);
                d += __shfl_xor(d, 4);
                d += __shfl_xor(d, 2);
                d += __shfl_xor(d, 1);
                s[u] = (c0 + (uint32_t)(tg + kGroups * u) < up_end && ((ok_cur >> u) & 1u)) ? d : -INFINITY;
            }
            float mx = m[hh];
#pragma unroll
            for (int u = 0; u < kTpl; ++u) mx = fmaxf(mx, s[u]);
            const float m_use = mx == -INFINITY ? 0.f : mx;
            const float alpha = fast_exp2(m[hh] - m_use);
            float pr[kTpl];
            float rs = 0.f;
#pragma unroll
            for (int u = 0; u < kTpl; ++u) {
                pr[u] = fast_exp2(s[u] - m_use);
                rs += pr[u];
            }
            ls[hh] = ls[hh] * alpha + rs;
            m[hh] = mx;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                float o = acc[hh][e] * alpha;
#pragma unroll
                for (int u = 0; u < kTpl; ++u) o += pr[u] * slice_elem<Elem, E>(vr[u], e);
                acc[hh][e] = o;
            }
        }
    }

    // Merge the token groups of this work-group.
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        if (tl == 0) {
            sm_m[tg][hh] = m[hh];
            sm_l[tg][hh] = ls[hh];
        }
#pragma unroll
        for (int e = 0; e < E; ++e) sm_o[tg][hh][tl * E + e] = acc[hh][e];
    }
    __syncthreads();
    for (int t = tid; t < G * D; t += kValuThreads) {
        const int hh = t / D, d = t % D;
        float M = -INFINITY;
#pragma unroll
        for (int q = 0; q < kGroups; ++q) M = fmaxf(M, sm_m[q][hh]);
        float Z = 0.f, O = 0.f;
#pragma unroll
        for (int q = 0; q < kGroups; ++q) {
            const float w = fast_exp2(sm_m[q][hh] - M);
            Z += w * sm_l[q][hh];
            O += w * sm_o[q][hh][d];
        }
        // A split with no attended key (all of its listed tokens skipped):
        // o = 0 and lse = -inf, which the merge weights by zero.
        const float ov = Z > 0.f ? O / Z : 0.f, lse2 = Z > 0.f ? M + log2f(Z) : -INFINITY;
        if (a.plan.direct) {
            put_out(hh, d, ov, lse2);
            continue;
        }
        const int64_t slot = ((int64_t)bb * a.Hq + g * G + hh) * a.plan.max_splits + split;
        a.ws_o[slot * D + d] = ov;
        if (d == 0) a.ws_lse[slot] = lse2;
    }
}

// ---------------------------------------------------------------------------
// Latent (absorbed-MLA) split kernel: d_qk = 576, d_v = 512, bf16, V = K[:512].
// ---------------------------------------------------------------------------
constexpr int kLatDqk = 576;
constexpr int kLatDv = 512;
constexpr int kLatCh = 32;                            // latent rows per LDS buffer
constexpr int kLatUnits = kLatDqk / 8;                // 16-byte units per row
constexpr int kLatThreads = 256;
constexpr int kLatBufs = 4;                           // ring depth
constexpr int kLatLead = 3;                           // LDS operands read this many MFMAs ahead
constexpr int kLatRowsPerWave = kLatCh / 4;           // rows each wave transfers per chunk
constexpr int kLatDma = kLatRowsPerWave * kLatUnits / 64;  // transfers per wave per chunk
constexpr int kLatMaxPages = kDecodeLatentMaxPages;   // page ids of one split kept in LDS
constexpr float kLatSlack = 8.f;                      // lazy-rescale slack (log2 units)
static_assert(kLatDma * 64 == kLatRowsPerWave * kLatUnits, "a wave moves whole rows");

// XOR swizzle of the 16-byte units of latent row r (1152 B, a multiple of
// 128 B, so unswizzled rows all start in the same banks). A linear map of the
// low four row bits, chosen so that both access patterns are conflict-free
// whether the LDS serves 128 or 256 bytes per cycle: 8 or 16 consecutive
// rows read at one unit (score operand), and 4 or 8 consecutive rows x 2
// units (transpose reads). Depends on r mod 16 only.
__device__ __forceinline__ int lat_swz(int r) {
    return ((r >> 2) & 1) | (r & 2) | (((r ^ (r >> 2) ^ (r >> 3)) & 1) << 2);
}

// One work-group computes one split (up to split_tokens attended tokens of
// one sequence) for up to 64 query heads of one kv head; wave w owns heads
// 16w..16w+15. The split's latent rows arrive in 32-token chunks through a
// ring of four LDS buffers: three are requested at the start and each chunk,
// once taken, frees the buffer of the one before it for the chunk three
// ahead (requesting all four of a 128-token split at the start measured
// slower: the first chunk then shares the memory system with the fourth).
// Per chunk: S^T = K q^T, an online softmax with lazy rescaling, and
// O^T += V^T P^T with P taken straight from the score registers; both
// products run on v_mfma_f32_16x16x32_bf16 and the V^T operand is gathered
// from the row-major buffer by transpose reads. q stays in AGPRs (it is only
// an MFMA source) so the VGPRs hold the output accumulators.
__global__ __launch_bounds__(kLatThreads, 1) void decode_split_latent(const DecodeArgs a) {
    __shared__ __attribute__((aligned(1024))) uint16_t c_b0[kLatCh * kLatDqk];
    __shared__ __attribute__((aligned(1024))) uint16_t c_b1[kLatCh * kLatDqk];
    __shared__ __attribute__((aligned(1024))) uint16_t c_b2[kLatCh * kLatDqk];
    __shared__ __attribute__((aligned(1024))) uint16_t c_b3[kLatCh * kLatDqk];
    __shared__ int32_t pids[kLatMaxPages];
    __shared__ int64_t rowtab[4][kLatRowsPerWave];
    // A split of listed tokens: each position's row offset (relative to kc)
    // and, one bit per position, whether it is attended.
    __shared__ int64_t lrows[kDecodeLatentMaxListSplit];
    __shared__ uint32_t lok[kDecodeLatentMaxListSplit / 32];

    // Work-groups of one XCD (own L2) take whole sequences, so the splits of a
    // sequence share q in that L2.
    const int nx = gridDim.x, ny = gridDim.y;
    const int lin = xcd_remap(blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z), nx * ny * gridDim.z);
    const int split = lin % nx;
    const int hcg = (lin / nx) % ny, bb = lin / (nx * ny);
    const int hc = hcg % a.plan.head_chunks, g = hcg / a.plan.head_chunks;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, kg = lane >> 4;
    const int heads_here = a.group - hc * 64 < 64 ? a.group - hc * 64 : 64;
    // A split slot past the row's splits holds lse = -inf, so the merge needs
    // neither the context length nor the split count.
    auto no_split = [&]() __attribute__((always_inline)) {
        for (int h = tid; h < heads_here; h += kLatThreads)
            a.ws_lse[((int64_t)bb * a.Hq + g * a.group + hc * 64 + h) * a.plan.max_splits + split] = -INFINITY;
    };

    const int64_t L = row_context(a, bb);
    if (L <= 0) {
        no_split();
        return;
    }
    const Sel sel = select_tokens(L, a);
    // Splits [0, n_win) cover the window's positions; the next list_splits(a)
    // cover the listed tokens (hybrid decode), positions of the list.
    const int n_win = (int)((sel.total + a.plan.split_tokens - 1) / a.plan.split_tokens);
    const bool listed = split >= n_win;
    const int64_t p_begin = (int64_t)(listed ? split - n_win : split) * a.plan.split_tokens;
    const int64_t p_lim = listed ? (int64_t)a.topk_k : sel.total;
    if (p_begin >= p_lim) {
        no_split();
        return;
    }
    const int64_t p_end = p_begin + a.plan.split_tokens < p_lim ? p_begin + a.plan.split_tokens : p_lim;
    const int ntok = (int)(p_end - p_begin);
    const int nch = (ntok + kLatCh - 1) / kLatCh;

    // Page ids of the split: positions [p_begin, p_end) map to at most two
    // token runs (one per attended range), each a run of logical pages.
    const int P = a.page_size;
    const int64_t e1 = p_end < sel.r1_end ? p_end : sel.r1_end;           // part in range 1: [p_begin, e1)
    const int64_t s2 = p_begin > sel.r1_end ? p_begin : sel.r1_end;       // part in range 2: [s2, p_end)
    const int64_t lp1 = p_begin / P;
    const int n1 = e1 > p_begin ? (int)((e1 - 1) / P - lp1 + 1) : 0;
    const int64_t t2 = sel.r2_begin + (s2 - sel.r1_end);                  // first token of part 2
    const int64_t lp2 = t2 / P;
    const int n2 = p_end > s2 ? (int)((sel.r2_begin + (p_end - sel.r1_end) - 1) / P - lp2 + 1) : 0;
    const bool active = wave * 16 < heads_here;
    const int head = g * a.group + hc * 64 + wave * 16 + l16;  // this lane's query head

    // q^T operand (16 heads x 576 per wave) in registers. Every wave loads
    // (one past the heads here loads wave 0's rows and never uses them), with
    // no branch, and the loads go out before the page-id loads so that the
    // two round trips overlap; both are complete before any transfer, so the
    // transfer waits below count transfers only.
    bf16x8 qf[kLatDqk / 32];
    {
        const int qhead = active ? head : head - wave * 16;
        const uint16_t *qp = (const uint16_t *)a.q + ((int64_t)bb * a.Hq + qhead) * kLatDqk + 8 * kg;
#pragma unroll
        for (int ks = 0; ks < kLatDqk / 32; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qp + ks * 32));
    }
    const int64_t seq = row_sequence(a, bb);
    const uint32_t up_end = (uint32_t)p_end, ur1 = (uint32_t)sel.r1_end, ur2 = (uint32_t)sel.r2_begin;
    const uint32_t uP = (uint32_t)P;
    if (!listed) {
        for (int t = tid; t < n1 + n2; t += kLatThreads)
            pids[t] = a.page_table[seq * a.max_pages + (t < n1 ? lp1 + t : lp2 + (t - n1))];
    } else {
        // Every listed position's row, found through the list and the page
        // table, once for the whole split: two dependent loads here, beside
        // the q loads, instead of two per chunk behind the transfers in
        // flight (a wait on a plain load also waits for those). A token
        // inside the window, past the context or negative (padding) is
        // skipped: its key is masked and token 0's row stands in for it.
        // Whole waves per pass, so that each ballot covers 64 positions.
        const uint32_t uL = (uint32_t)L, ur2end = ur2 < uL ? ur2 : uL;
        const int padded = (ntok + 63) & ~63;  // <= kDecodeLatentMaxListSplit (host check)
        for (int p = tid; p < padded; p += kLatThreads) {
            bool ok = false;
            int64_t off = 0;
            if (p < ntok) {
                const int t0 = a.topk[seq * a.topk_k + p_begin + p];
                ok = t0 >= (int)ur1 && (uint32_t)t0 < ur2end;
                const uint32_t tok = ok ? (uint32_t)t0 : 0u;
                const uint32_t lp = tok / uP;
                off = (int64_t)a.page_table[seq * a.max_pages + lp] * a.ks[0] + (int64_t)(tok - lp * uP) * a.ks[1];
            }
            lrows[p] = off;
            const uint64_t bits = __builtin_amdgcn_ballot_w64(ok);
            if (lane == 0) {
                lok[p >> 5] = (uint32_t)bits;
                lok[(p >> 5) + 1] = (uint32_t)(bits >> 32);
            }
        }
    }
    // q is only ever an MFMA source operand, which may sit in AGPRs: park it
    // there so the VGPRs hold the output accumulators and the scores.
#pragma unroll
    for (int ks = 0; ks < kLatDqk / 32; ++ks) asm volatile("" : "+a"(qf[ks]));
    __syncthreads();

    const uint16_t *kc = (const uint16_t *)a.kc + g * a.ks[2];
    // Element offset (relative to kc) of the latent row at split position pp,
    // clamped to the split. Positions and tokens fit in 32 bits.
    const uint32_t ulp1 = (uint32_t)lp1, ulp2 = (uint32_t)lp2;
    auto row_off = [&](uint32_t pp) __attribute__((always_inline)) -> int64_t {
        pp = pp < up_end ? pp : up_end - 1;
        const uint32_t tok = pp < ur1 ? pp : ur2 + (pp - ur1);
        const uint32_t lp = tok / uP;
        const int idx = pp < ur1 ? (int)(lp - ulp1) : n1 + (int)(lp - ulp2);
        return (int64_t)pids[idx] * a.ks[0] + (int64_t)(tok - lp * uP) * a.ks[1];
    };
    // Transfers of chunk c: wave w moves rows 8w..8w+7. Lane slot p = 64n + lane
    // of its transfer n is row 8w + p / 72 at physical unit p % 72, which holds
    // logical unit (p % 72) ^ lat_swz(row). The wave's eight row offsets are
    // computed once by lanes 0..7 into rowtab (rows past the split's end
    // repeat its last row); a listed split takes them from lrows.
    auto issue = [&](int c, uint16_t *buf) __attribute__((always_inline)) {
        const int rel = c * kLatCh + wave * kLatRowsPerWave + lane;  // position in the split
        if (lane < kLatRowsPerWave) {
            if (!listed) rowtab[wave][lane] = row_off((uint32_t)p_begin + (uint32_t)rel);
            else rowtab[wave][lane] = lrows[rel < ntok ? rel : ntok - 1];
        }
#pragma unroll
        for (int n = 0; n < kLatDma; ++n) {
            const int p = n * 64 + lane;
            const int r = p / kLatUnits;
            const int unit = (p % kLatUnits) ^ lat_swz(wave * kLatRowsPerWave + r);
            dma16_untracked(kc + rowtab[wave][r] + unit * 8, lds_addr(buf + (wave * kLatDma + n) * 512));
        }
    };

    // Lane-constant LDS byte offsets.
    // Score operand: row tb*16 + l16, unit 4ks + kg, swizzled by lat_swz(l16)
    // (the tb*16 offset does not change the swizzle): two variants by ks parity.
    const int ksw = lat_swz(l16);
    const uint32_t k_lane = (uint32_t)l16 * (kLatDqk * 2);
    const uint32_t k_even = (uint32_t)((kg ^ ksw) << 4), k_odd = (uint32_t)(((4 + kg) ^ ksw) << 4);
    // Transpose reads: lane s of group kg reads token 16h + 4kg + s/4 at value
    // column 16d + 4(s%4); its swizzle depends only on the lane.
    const int tr_tok = 4 * kg + (l16 >> 2);
    const int vsw = lat_swz(tr_tok);
    const int uo = (l16 & 3) >> 1;
    uint32_t v_lane[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
        v_lane[q4] = (uint32_t)tr_tok * (kLatDqk * 2) + (uint32_t)(((2 * q4 + uo) ^ vsw) << 4) + 8u * (l16 & 1);

    // S^T of chunk c from `buf`: element r of s[tb] is token tb*16 + 4kg + r of
    // the chunk (for head l16), -inf past the split's end.
    auto scores = [&](const uint16_t *buf, int c, f32x4 (&s)[2]) __attribute__((always_inline)) {
        uint32_t kl = k_lane, ke = k_even, ko = k_odd;
        asm volatile("" : "+v"(kl), "+v"(ke), "+v"(ko));
        const char *rowp = (const char *)buf + kl;
        s[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        s[1] = f32x4{0.f, 0.f, 0.f, 0.f};
        // One wave per SIMD: an operand read just before its MFMA exposes the
        // whole LDS latency, so operands are read kLatLead MFMAs ahead (the
        // fences keep the compiler from regrouping reads and waits).
        constexpr int NS = 2 * (kLatDqk / 32);  // MFMA n: ks = n / 2, token block n % 2
        bf16x8 kf[NS];
        auto load = [&](int n) __attribute__((always_inline)) {
            const int ks = n >> 1, tb = n & 1;
            kf[n] = *(const bf16x8 *)(rowp + tb * 16 * (kLatDqk * 2) + 128 * (ks >> 1) + ((ks & 1) ? ko : ke));
        };
#pragma unroll
        for (int n = 0; n < kLatLead; ++n) load(n);
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            if (n + kLatLead < NS) load(n + kLatLead);
            __builtin_amdgcn_sched_barrier(0);
            s[n & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[n], qf[n >> 1], s[n & 1], 0, 0, 0);
        }
        const int nvalid = ntok - c * kLatCh;
        const uint32_t vm = listed ? lok[c] : 0xffffffffu;  // positions 32c .. 32c+31
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = tb * 16 + 4 * kg + r;
                if (t >= nvalid || !((vm >> t) & 1u)) s[tb][r] = -INFINITY;
            }
    };

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 oacc[kLatDv / 16];
#pragma unroll
    for (int d = 0; d < kLatDv / 16; ++d) oacc[d] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One chunk: scores, online softmax (lazy rescale), then O^T += V^T P^T.
    // Slot e of lane (head l16, kg) in the P^T operand is token
    // 16(e/4) + 4kg + e%4 of the chunk.
    auto compute = [&](const uint16_t *buf, int c) __attribute__((always_inline)) {
        f32x4 s[2];
        scores(buf, c, s);
        float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                         fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
        mx = max_xor32(max_xor16(mx)) * a.scale_log2;
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kLatSlack)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = fast_exp2(m_run - m_new);  // 0 on the first chunk
            l_run *= alpha;
#pragma unroll
            for (int d = 0; d < kLatDv / 16; ++d) oacc[d] *= alpha;
            m_run = m_new;
        }
        float p[8];
        float rs = 0.f;
        // Before any attended key (possible only for listed tokens) m_run is
        // -inf and every score of the chunk is masked: p = 0.
        const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[4 * tb + r] = fast_exp2(__builtin_fmaf(s[tb][r], a.scale_log2, neg_m));
                rs += p[4 * tb + r];
            }
        l_run += rs;
        const u32x4 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                          pack_bf16x2(p[6], p[7])};
        const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
        uint32_t vl[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            vl[q4] = v_lane[q4];
            asm volatile("" : "+v"(vl[q4]));
        }
        const char *cb = (const char *)buf;
        constexpr int NO = kLatDv / 16;
        bf16x8 vf[NO];
        auto vload = [&](int d) __attribute__((always_inline)) {
            const char *vp = cb + vl[d & 3] + 128 * (d >> 2);
            const i16x4 lo = lds_read_tr16(vp);
            const i16x4 up = lds_read_tr16(vp + 16 * (kLatDqk * 2));
            vf[d] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
        };
#pragma unroll
        for (int d = 0; d < kLatLead; ++d) vload(d);
#pragma unroll
        for (int d = 0; d < NO; ++d) {
            if (d + kLatLead < NO) vload(d + kLatLead);
            __builtin_amdgcn_sched_barrier(0);
            oacc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[d], pf, oacc[d], 0, 0, 0);
        }
    };

    // Ring of four buffers, one barrier per chunk: wait for this wave's share
    // of chunk c (the transfers still allowed in flight are those of chunks
    // c+1 and c+2, when they exist); the barrier publishes chunk c and proves
    // every wave is done with chunk c-1, whose buffer then takes chunk c+3.
    auto cbuf = [&](auto k) __attribute__((always_inline)) -> uint16_t * {
        constexpr int b = decltype(k)::value % kLatBufs;
        if constexpr (b == 0) return c_b0;
        else if constexpr (b == 1) return c_b1;
        else if constexpr (b == 2) return c_b2;
        else return c_b3;
    };
    auto step = [&](int c, auto k) __attribute__((always_inline)) {
        constexpr int b = decltype(k)::value;
        if (c + 2 < nch) wait_vmcnt<2 * kLatDma>();
        else if (c + 1 < nch) wait_vmcnt<kLatDma>();
        else wait_vmcnt<0>();
        barrier_lds_drained();
        if (c + 3 < nch) issue(c + 3, cbuf(std::integral_constant<int, b + 3>{}));
        if (active) compute(cbuf(k), c);
    };
    issue(0, c_b0);
    if (1 < nch) issue(1, c_b1);
    if (2 < nch) issue(2, c_b2);
    for (int c = 0; c < nch; c += kLatBufs) {
        step(c, std::integral_constant<int, 0>{});
        if (c + 1 >= nch) break;
        step(c + 1, std::integral_constant<int, 1>{});
        if (c + 2 >= nch) break;
        step(c + 2, std::integral_constant<int, 2>{});
        if (c + 3 >= nch) break;
        step(c + 3, std::integral_constant<int, 3>{});
    }

    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    // Every wave is done with the ring buffers: wave w stages its 16 partial
    // rows in buffer w below.
    barrier_lds_drained();
    if (!active) return;
    // A split with no attended key (all of its listed tokens skipped) writes
    // o = 0 and lse = -inf, which the merge weights by zero.
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t slot = ((int64_t)bb * a.Hq + head) * a.plan.max_splits + split;
    // Partial outputs in bf16: per split they would otherwise weigh as much
    // as the split's latent rows (64 heads x 512 x 4 B against 128 x 1152 B).
    // They go out through LDS as whole 1 KB rows, one store instruction per
    // head: written straight from the accumulators, each store instruction
    // covered 8-byte pieces of 16 rows, and those scattered stores cost as
    // much as a quarter of an SSA call. The staged rows' 16-byte units are
    // XOR-swizzled by head so that the 16 heads of one write hit distinct
    // banks.
    char *stage = (char *)(wave == 0 ? c_b0 : wave == 1 ? c_b1 : wave == 2 ? c_b2 : c_b3);
    static_assert(16 * kLatDv * 2 <= kLatCh * kLatDqk * 2, "a wave's partial rows fit one buffer");
    constexpr int kRowB = kLatDv * 2;  // 1 KB
#pragma unroll
    for (int d = 0; d < kLatDv / 16; ++d) {
        const int unit = (2 * d + (kg >> 1)) ^ l16;
        *(u32x2 *)(stage + l16 * kRowB + unit * 16 + 8 * (kg & 1)) =
            u32x2{pack_bf16x2(oacc[d][0] * inv, oacc[d][1] * inv), pack_bf16x2(oacc[d][2] * inv, oacc[d][3] * inv)};
    }
    const int64_t slot0 = ((int64_t)bb * a.Hq + (head - l16)) * a.plan.max_splits + split;  // head l16 = 0
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const u32x4 v = *(const u32x4 *)(stage + r * kRowB + ((lane ^ r) * 16));
        uint16_t *wrow = (uint16_t *)a.ws_o + (slot0 + (int64_t)r * a.plan.max_splits) * kLatDv;
        *(u32x4 *)(wrow + lane * 8) = v;
    }
    if (kg == 0) a.ws_lse[slot] = l_tot > 0.f ? m_run + log2f(l_tot) : -INFINITY;
}

// ---------------------------------------------------------------------------
// Merge of the splits of one (sequence, query head): one wave each.
// ---------------------------------------------------------------------------
constexpr int kMergeThreads = 256;
constexpr int kMergeBatch = 8;  // splits whose partial outputs are loaded together

// Lane i owns output elements E*i .. E*i + E - 1 (E = D / 64). The split
// weights exp2(lse_s - M) / Z are computed once per split by lane s % 64 and
// broadcast with readlane.
template <bool kBF16, int D>
__global__ __launch_bounds__(kMergeThreads) void decode_merge(const DecodeArgs a) {
    using Elem = std::conditional_t<kBF16, uint16_t, float>;
    constexpr int E = D / 64;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * (kMergeThreads / 64) + (threadIdx.x >> 6);  // bb * Hq + h
    if (row >= a.B * a.Hq) return;
    Elem *out = (Elem *)a.o + (int64_t)row * D + E * lane;
    const int64_t slot0 = (int64_t)row * a.plan.max_splits;
    const float *wl = a.ws_lse + slot0;
    // The latent split kernel (the only one with D = 512) stores its partial
    // outputs in bf16; the others in fp32.
    constexpr bool kPartBF16 = D == 512;
    using Part = std::conditional_t<kPartBF16, uint16_t, float>;
    const Part *wo = (const Part *)a.ws_o + slot0 * D + E * lane;

    // Partial rows of splits s0 .. s0+7 (clamped to nb - 1).
    float part[kMergeBatch][E];
    auto load_batch = [&](int s0, int nb) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
            const int s = s0 + u < nb ? s0 + u : nb - 1;
            const Part *src = wo + (int64_t)s * D;
            if constexpr (kPartBF16) {
                static_assert(E == 8, "bf16 partials: 8 per lane");
                const u32x4 v = *(const u32x4 *)src;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    part[u][2 * e] = bf16_lo(v[e]);
                    part[u][2 * e + 1] = bf16_hi(v[e]);
                }
            } else if constexpr (E >= 4) {
#pragma unroll
                for (int e4 = 0; e4 < E / 4; ++e4) {
                    const f32x4 v = *(const f32x4 *)(src + 4 * e4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) part[u][4 * e4 + e] = v[e];
                }
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) part[u][e] = src[e];
            }
        }
    };
    // Every split slot of the row holds an lse: -inf for a slot past the
    // row's splits (or a split with no attended key), so the split count and
    // the context length are not needed, and the first batch of partial rows
    // is requested together with the lse of the first 64 splits. A slot with
    // a zero weight may hold a stale partial row: it never enters a product
    // (uniform branches below, not multiplications by zero).
    const int ns = a.plan.max_splits;
    const int nb0 = ns < 64 ? ns : 64;
    load_batch(0, nb0);
    const float lse0 = lane < nb0 ? wl[lane] : -INFINITY;
    float M = lse0;
    for (int s = lane + 64; s < ns; s += 64) M = fmaxf(M, wl[s]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    if (M == -INFINITY) {  // no key at all (context length 0)
#pragma unroll
        for (int e = 0; e < E; ++e) out[e] = Elem(0);
        if (lane == 0 && a.lse) a.lse[row] = -INFINITY;
        return;
    }
    float Z = fast_exp2(lse0 - M);
    for (int s = lane + 64; s < ns; s += 64) Z += fast_exp2(wl[s] - M);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) Z += __shfl_xor(Z, o);
    const float inv = 1.f / Z;

    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    for (int s64 = 0; s64 < ns; s64 += 64) {
        const float lw = s64 == 0 ? lse0 : (s64 + lane < ns ? wl[s64 + lane] : -INFINITY);
        const float wlane = fast_exp2(lw - M) * inv;
        const uint64_t used = __builtin_amdgcn_ballot_w64(wlane != 0.f);
        const int nb = ns - s64 < 64 ? ns - s64 : 64;
        for (int s0 = 0; s0 < nb; s0 += kMergeBatch) {
            if (!((used >> s0) & ((1u << kMergeBatch) - 1))) continue;  // uniform: no weight here
            if (s0 > 0 || s64 > 0) load_batch(s0, nb);
#pragma unroll
            for (int u = 0; u < kMergeBatch; ++u) {
                if (s0 + u < nb && ((used >> (s0 + u)) & 1)) {  // uniform
                    const float wf = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wlane), s0 + u));
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(wf, part[u][e], acc[e]);
                }
            }
        }
        wo += (int64_t)64 * D;
    }
    if constexpr (kBF16) {
#pragma unroll
        for (int e = 0; e < E; e += 2) {
            if constexpr (E == 1) {
                out[0] = (uint16_t)(pack_bf16x2(acc[0], 0.f) & 0xffffu);
            } else {
                *(uint32_t *)(out + e) = pack_bf16x2(acc[e], acc[e + 1]);
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) out[e] = acc[e];
    }
    if (lane == 0 && a.lse) a.lse[row] = (M + log2f(Z)) * kLn2;
}

template <bool kBF16, int D, int G>
hipError_t launch_valu(const DecodeArgs &a, hipStream_t stream) {
    void *args[] = {(void *)&a};
    const void *k = a.topk_k > 0 ? (const void *)decode_split_valu<kBF16, D, G, true>
                                 : (const void *)decode_split_valu<kBF16, D, G, false>;
    return hipLaunchKernel(k,
                           dim3(a.plan.max_splits, a.Hkv, a.B), dim3(kValuThreads), args, 0, stream);
}

template <bool kBF16, int D>
hipError_t launch_valu_g(const DecodeArgs &a, hipStream_t stream) {
    switch (a.group) {
        case 1: return launch_valu<kBF16, D, 1>(a, stream);
        case 2: return launch_valu<kBF16, D, 2>(a, stream);
        case 4: return launch_valu<kBF16, D, 4>(a, stream);
        case 8:
            if constexpr (D <= 128) return launch_valu<kBF16, D, 8>(a, stream);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

template <bool kBF16>
hipError_t launch_valu_d(int d, const DecodeArgs &a, hipStream_t stream) {
    switch (d) {
        case 64: return launch_valu_g<kBF16, 64>(a, stream);
        case 128: return launch_valu_g<kBF16, 128>(a, stream);
        case 256: return launch_valu_g<kBF16, 256>(a, stream);
        default: return hipErrorInvalidValue;
    }
}


// Row map of packed query rows. Work-group (x, b) writes rows
// cu_q[b] + 256 x + tid of sequence b: one round of (uniform) loads, no search.
// Writes stay inside [0, total_q) whatever the prefix sums hold, and the
// length is clamped to the sequence's.
__global__ __launch_bounds__(256) void extend_rows(const int32_t *cu_q, const int32_t *ctx_lens,
                                                   int32_t total_q, int32_t *row_seq, int32_t *row_ctx) {
    const int b = blockIdx.y;
    const int r0 = cu_q[b], r1 = cu_q[b + 1], ctx = ctx_lens[b];
    const int r = r0 + blockIdx.x * 256 + threadIdx.x;
    if (r >= r1 || r < 0 || r >= total_q) return;
    const int v = ctx - (r1 - 1 - r);
    row_seq[r] = b;
    row_ctx[r] = v < ctx ? v : ctx;
}

}  // namespace

bool decode_valu_supported(bool bf16, int d_qk, int d_v, int group) {
    (void)bf16;
    if (d_qk != d_v || (d_qk != 64 && d_qk != 128 && d_qk != 256)) return false;
    if (group != 1 && group != 2 && group != 4 && group != 8) return false;
    return group * d_v <= 1024;
}

bool decode_latent_supported(bool bf16, int d_qk, int d_v, int group) {
    return bf16 && d_qk == kLatDqk && d_v == kLatDv && group >= 16 && group % 16 == 0;
}

hipError_t launch_decode(bool bf16, int d_qk, int d_v, const DecodeArgs &a, hipStream_t stream) {
    hipError_t err;
    if (a.plan.kind == kDecodeLatent) {
        if (!bf16 || d_qk != kLatDqk || d_v != kLatDv) return hipErrorInvalidValue;
        void *args[] = {(void *)&a};
        err = hipLaunchKernel((const void *)decode_split_latent,
                              dim3(a.plan.max_splits, a.Hkv * a.plan.head_chunks, a.B),
                              dim3(kLatThreads), args, 0, stream);
    } else {
        err = bf16 ? launch_valu_d<true>(d_qk, a, stream) : launch_valu_d<false>(d_qk, a, stream);
    }
    if (err != hipSuccess || a.plan.direct) return err;
    const void *merge;
    switch (d_v) {
        case 64: merge = bf16 ? (const void *)decode_merge<true, 64> : (const void *)decode_merge<false, 64>; break;
        case 128: merge = bf16 ? (const void *)decode_merge<true, 128> : (const void *)decode_merge<false, 128>; break;
        case 256: merge = bf16 ? (const void *)decode_merge<true, 256> : (const void *)decode_merge<false, 256>; break;
        case 512: merge = bf16 ? (const void *)decode_merge<true, 512> : (const void *)decode_merge<false, 512>; break;
        default: return hipErrorInvalidValue;
    }
    void *margs[] = {(void *)&a};
    const int rows_per_wg = kMergeThreads / 64;
    const int64_t wgs = ((int64_t)a.B * a.Hq + rows_per_wg - 1) / rows_per_wg;
    return hipLaunchKernel(merge, dim3((unsigned)wgs), dim3(kMergeThreads), margs, 0, stream);
}

hipError_t launch_extend_rows(const int32_t *cu_q, const int32_t *ctx_lens, int32_t batch,
                              int32_t max_q_len, int32_t total_q, int32_t *row_seq, int32_t *row_ctx,
                              hipStream_t stream) {
    void *args[] = {(void *)&cu_q, (void *)&ctx_lens, (void *)&total_q, (void *)&row_seq, (void *)&row_ctx};
    return hipLaunchKernel((const void *)extend_rows, dim3((max_q_len + 255) / 256, batch), dim3(256), args,
                           0, stream);
}

}  // namespace ssa
