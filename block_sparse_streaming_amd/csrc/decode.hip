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
//    of 32 tokens are staged in LDS twice: row-major (for S) and transposed (for
//    P.V), the next chunk's global loads in flight during the current chunk.
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

__device__ __forceinline__ Sel select_tokens(int64_t L, const DecodeArgs &a) {
    if (a.full) return Sel{L, L, L};
    const int64_t b = a.block, sb = (int64_t)a.sink * b;
    const int64_t qb = (L - 1) / b;
    const int64_t r1 = sb < L ? sb : L;
    const int64_t lo0 = (qb - a.local + 1) * b;
    const int64_t lo = lo0 > sb ? lo0 : sb;
    const int64_t n2 = L > lo ? L - lo : 0;
    return Sel{r1, lo, r1 + n2};
}

__device__ __forceinline__ int64_t sel_token(const Sel &s, int64_t p) {
    return p < s.r1_end ? p : s.r2_begin + (p - s.r1_end);
}

// Element offset of token `tok`'s row (head 0) in a cache with strides `str`.
__device__ __forceinline__ int64_t token_row(const DecodeArgs &a, int bb, int64_t tok,
                                             const int64_t *str) {
    const int64_t page = a.page_table[(int64_t)bb * a.max_pages + tok / a.page_size];
    return page * str[0] + (tok % a.page_size) * str[1];
}

// ---------------------------------------------------------------------------
// VALU split kernel.
// ---------------------------------------------------------------------------
constexpr int kValuThreads = 256;
constexpr int kTpt = 16;                       // lanes per token
constexpr int kGroups = kValuThreads / kTpt;   // token groups per work-group
constexpr int kUnroll = 4;                     // tokens per group per step

template <typename Elem, int E>
__device__ __forceinline__ void load_row(const Elem *p, float (&out)[E]) {
    if constexpr (std::is_same_v<Elem, float>) {
#pragma unroll
        for (int c = 0; c < E / 4; ++c) {
            const f32x4 w = *(const f32x4 *)(p + 4 * c);
#pragma unroll
            for (int e = 0; e < 4; ++e) out[4 * c + e] = w[e];
        }
    } else if constexpr (E == 4) {
        const u32x2 w = *(const u32x2 *)p;
        out[0] = bf16_lo(w[0]); out[1] = bf16_hi(w[0]);
        out[2] = bf16_lo(w[1]); out[3] = bf16_hi(w[1]);
    } else {
#pragma unroll
        for (int c = 0; c < E / 8; ++c) {
            const u32x4 w = *(const u32x4 *)(p + 8 * c);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                out[8 * c + 2 * e] = bf16_lo(w[e]);
                out[8 * c + 2 * e + 1] = bf16_hi(w[e]);
            }
        }
    }
}

template <bool kBF16, int D, int G>
__global__ __launch_bounds__(kValuThreads) void decode_split_valu(const DecodeArgs a) {
    using Elem = std::conditional_t<kBF16, uint16_t, float>;
    constexpr int E = D / kTpt;
    __shared__ float sm_m[kGroups][G];
    __shared__ float sm_l[kGroups][G];
    __shared__ float sm_o[kGroups][G][D];

    const int split = blockIdx.x, g = blockIdx.y, bb = blockIdx.z;
    const int tid = threadIdx.x, tg = tid / kTpt, tl = tid % kTpt;
    const int64_t L = a.ctx_lens[bb];
    if (L <= 0) return;
    const Sel sel = select_tokens(L, a);
    const int64_t p_begin = (int64_t)split * a.plan.split_tokens;
    if (p_begin >= sel.total) return;
    const int64_t p_end = p_begin + a.plan.split_tokens < sel.total ? p_begin + a.plan.split_tokens
                                                                      : sel.total;

    float qv[G][E];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        const Elem *qp = (const Elem *)a.q + ((int64_t)bb * a.Hq + g * G + hh) * D + tl * E;
        load_row<Elem, E>(qp, qv[hh]);
#pragma unroll
        for (int e = 0; e < E; ++e) qv[hh][e] *= a.scale_log2;
    }

    float m[G], ls[G], acc[G][E];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        m[hh] = -INFINITY;
        ls[hh] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[hh][e] = 0.f;
    }

    const Elem *kc = (const Elem *)a.kc + g * a.ks[2] + tl * E;
    const Elem *vc = (const Elem *)a.vc + g * a.vs[2] + tl * E;
    for (int64_t p0 = p_begin; p0 < p_end; p0 += kGroups * kUnroll) {
        float kr[kUnroll][E], vr[kUnroll][E];
        bool valid[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t pp = p0 + u * kGroups + tg;
            valid[u] = pp < p_end;
            if (valid[u]) {
                const int64_t tok = sel_token(sel, pp);
                load_row<Elem, E>(kc + token_row(a, bb, tok, a.ks), kr[u]);
                load_row<Elem, E>(vc + token_row(a, bb, tok, a.vs), vr[u]);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) kr[u][e] = vr[u][e] = 0.f;
            }
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            float s[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) d += qv[hh][e] * kr[u][e];
                d += __shfl_xor(d, 8);
                d += __shfl_xor(d, 4);
                d += __shfl_xor(d, 2);
                d += __shfl_xor(d, 1);
                s[u] = valid[u] ? d : -INFINITY;
            }
            float mx = m[hh];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) mx = fmaxf(mx, s[u]);
            const float m_use = mx == -INFINITY ? 0.f : mx;
            const float alpha = fast_exp2(m[hh] - m_use);
            float pr[kUnroll];
            float rs = 0.f;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                pr[u] = fast_exp2(s[u] - m_use);
                rs += pr[u];
            }
            ls[hh] = ls[hh] * alpha + rs;
            m[hh] = mx;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                float o = acc[hh][e] * alpha;
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) o += pr[u] * vr[u][e];
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
        const int64_t slot = ((int64_t)bb * a.Hq + g * G + hh) * a.plan.max_splits + split;
        a.ws_o[slot * D + d] = O / Z;
        if (d == 0) a.ws_lse[slot] = M + log2f(Z);
    }
}

// ---------------------------------------------------------------------------
// Latent (absorbed-MLA) split kernel: d_qk = 576, d_v = 512, bf16, V = K[:512].
// ---------------------------------------------------------------------------
constexpr int kLatDqk = 576;
constexpr int kLatDv = 512;
constexpr int kLatCh = 32;                  // tokens per LDS chunk
constexpr int kKnStr = kLatDqk + 8;         // row-major K chunk, padded
constexpr int kVtStr = kLatCh + 8;          // transposed V chunk, padded
constexpr int kLatThreads = 256;

// Position of token quad `quad` (tokens 4quad..4quad+3 of a 32-token chunk) in a
// V^T row. In the 16x16 accumulator a lane of row group kg holds tokens
// 4kg..4kg+3 of each 16-token block; the P.V B operand feeds those 8 tokens as
// one 8-wide slot, so they are stored adjacently: pos = 8*kg + 4*block.
__device__ __forceinline__ int lat_quad_pos(int quad) { return 8 * (quad & 3) + 4 * (quad >> 2); }

__global__ __launch_bounds__(kLatThreads, 1) void decode_split_latent(const DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t kn[kLatCh * kKnStr];
    __shared__ __attribute__((aligned(16))) uint16_t vt[kLatDv * kVtStr];

    const int split = blockIdx.x;
    const int hc = blockIdx.y % a.plan.head_chunks, g = blockIdx.y / a.plan.head_chunks;
    const int bb = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, kg = lane >> 4;

    const int64_t L = a.ctx_lens[bb];
    if (L <= 0) return;
    const Sel sel = select_tokens(L, a);
    const int64_t p_begin = (int64_t)split * a.plan.split_tokens;
    if (p_begin >= sel.total) return;
    const int64_t p_end = p_begin + a.plan.split_tokens < sel.total ? p_begin + a.plan.split_tokens
                                                                      : sel.total;
    const int64_t ntok = p_end - p_begin;
    const int nch = (int)((ntok + kLatCh - 1) / kLatCh);

    const int heads_here = a.group - hc * 64 < 64 ? a.group - hc * 64 : 64;
    const bool active = wave * 16 < heads_here;
    const int head = g * a.group + hc * 64 + wave * 16 + l16;  // this lane's query head

    // q^T operand (16 heads x 576 per wave) in registers.
    bf16x8 qf[kLatDqk / 32];
    {
        const uint16_t *qp = (const uint16_t *)a.q + ((int64_t)bb * a.Hq + head) * kLatDqk + 8 * kg;
#pragma unroll
        for (int ks = 0; ks < kLatDqk / 32; ++ks) {
            u32x4 w = {0u, 0u, 0u, 0u};
            if (active) w = *(const u32x4 *)(qp + ks * 32);
            qf[ks] = __builtin_bit_cast(bf16x8, w);
        }
    }

    const uint16_t *kc = (const uint16_t *)a.kc + g * a.ks[2];
    // Staging registers for one chunk: two (token quad, 16-byte column) units of
    // the first 512 dims and one 16-byte column of the last 64 dims.
    u32x4 pre[9];
    auto fetch = [&](int c) {
        const int64_t base = p_begin + (int64_t)c * kLatCh;
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
            const int u = tid + kLatThreads * t2;
            const int dc = u & 63, quad = u >> 6;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int64_t pp = base + 4 * quad + rr;
                pre[4 * t2 + rr] = u32x4{0u, 0u, 0u, 0u};
                if (pp < p_end)
                    pre[4 * t2 + rr] = *(const u32x4 *)(kc + token_row(a, bb, sel_token(sel, pp), a.ks) + dc * 8);
            }
        }
        const int64_t pp = base + (tid >> 3);
        pre[8] = u32x4{0u, 0u, 0u, 0u};
        if (pp < p_end)
            pre[8] = *(const u32x4 *)(kc + token_row(a, bb, sel_token(sel, pp), a.ks) + (64 + (tid & 7)) * 8);
    };
    auto stash = [&]() {
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
            const int u = tid + kLatThreads * t2;
            const int dc = u & 63, quad = u >> 6;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) *(u32x4 *)(kn + (4 * quad + rr) * kKnStr + dc * 8) = pre[4 * t2 + rr];
            const int pos = lat_quad_pos(quad);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                u32x2 w2 = {pick_pair(pre[4 * t2 + 0], pre[4 * t2 + 1], e),
                            pick_pair(pre[4 * t2 + 2], pre[4 * t2 + 3], e)};
                *(u32x2 *)(vt + (dc * 8 + e) * kVtStr + pos) = w2;
            }
        }
        *(u32x4 *)(kn + (tid >> 3) * kKnStr + (64 + (tid & 7)) * 8) = pre[8];
    };

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 oacc[kLatDv / 16];
#pragma unroll
    for (int d = 0; d < kLatDv / 16; ++d) oacc[d] = f32x4{0.f, 0.f, 0.f, 0.f};

    fetch(0);
    for (int c = 0; c < nch; ++c) {
        __syncthreads();
        stash();
        __syncthreads();
        if (c + 1 < nch) fetch(c + 1);
        if (!active) continue;

        // S^T = K q^T: element r of block tb is token tb*16 + 4*kg + r, head l16.
        f32x4 sacc[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            sacc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
            const uint16_t *krow = kn + (tb * 16 + l16) * kKnStr + 8 * kg;
#pragma unroll
            for (int ks = 0; ks < kLatDqk / 32; ++ks) {
                const bf16x8 kf = *(const bf16x8 *)(krow + ks * 32);
                sacc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], sacc[tb], 0, 0, 0);
            }
        }
        const int64_t nvalid = ntok - (int64_t)c * kLatCh;
        float mx = -INFINITY;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tk = tb * 16 + 4 * kg + r;
                const float x = tk < nvalid ? sacc[tb][r] * a.scale_log2 : -INFINITY;
                sacc[tb][r] = x;
                mx = fmaxf(mx, x);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float p[8];
        float rs = 0.f;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[4 * tb + r] = fast_exp2(sacc[tb][r] - m_use);
                rs += p[4 * tb + r];
            }
        l_run = l_run * alpha + rs;
        m_run = m_new;
        const u32x4 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                          pack_bf16x2(p[6], p[7])};
        const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
        for (int d = 0; d < kLatDv / 16; ++d) {
            oacc[d] *= alpha;
            const bf16x8 vf = *(const bf16x8 *)(vt + (d * 16 + l16) * kVtStr + 8 * kg);
            oacc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, oacc[d], 0, 0, 0);
        }
    }

    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (!active) return;
    const float inv = 1.f / l_tot;
    const int64_t slot = ((int64_t)bb * a.Hq + head) * a.plan.max_splits + split;
    float *wo = a.ws_o + slot * kLatDv + 4 * kg;
#pragma unroll
    for (int d = 0; d < kLatDv / 16; ++d) *(f32x4 *)(wo + d * 16) = oacc[d] * inv;
    if (kg == 0) a.ws_lse[slot] = m_run + log2f(l_tot);
}

// ---------------------------------------------------------------------------
// Merge of the splits of one (sequence, query head).
// ---------------------------------------------------------------------------
template <bool kBF16>
__global__ __launch_bounds__(256) void decode_merge(const DecodeArgs a, int D) {
    using Elem = std::conditional_t<kBF16, uint16_t, float>;
    const int h = blockIdx.x, bb = blockIdx.y, tid = threadIdx.x;
    const int64_t L = a.ctx_lens[bb];
    Elem *out = (Elem *)a.o + ((int64_t)bb * a.Hq + h) * D;
    int ns = 0;
    if (L > 0) {
        const Sel sel = select_tokens(L, a);
        ns = (int)((sel.total + a.plan.split_tokens - 1) / a.plan.split_tokens);
    }
    if (ns == 0) {
        for (int d = tid; d < D; d += blockDim.x) out[d] = Elem(0);
        if (tid == 0 && a.lse) a.lse[(int64_t)bb * a.Hq + h] = -INFINITY;
        return;
    }
    const int64_t slot0 = ((int64_t)bb * a.Hq + h) * a.plan.max_splits;
    const float *wl = a.ws_lse + slot0;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, wl[s]);
    float Z = 0.f;
    for (int s = 0; s < ns; ++s) Z += fast_exp2(wl[s] - M);
    const float inv = 1.f / Z;
    const float *wo = a.ws_o + slot0 * D;
    for (int d = tid; d < D; d += blockDim.x) {
        float o = 0.f;
        for (int s = 0; s < ns; ++s) o += fast_exp2(wl[s] - M) * wo[(int64_t)s * D + d];
        o *= inv;
        if constexpr (kBF16) {
            out[d] = (uint16_t)(pack_bf16x2(o, 0.f) & 0xffffu);
        } else {
            out[d] = o;
        }
    }
    if (tid == 0 && a.lse) a.lse[(int64_t)bb * a.Hq + h] = (M + log2f(Z)) * kLn2;
}

template <bool kBF16, int D, int G>
hipError_t launch_valu(const DecodeArgs &a, hipStream_t stream) {
    void *args[] = {(void *)&a};
    return hipLaunchKernel((const void *)decode_split_valu<kBF16, D, G>,
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
    if (err != hipSuccess) return err;
    int D = d_v;
    void *margs[] = {(void *)&a, (void *)&D};
    return hipLaunchKernel(bf16 ? (const void *)decode_merge<true> : (const void *)decode_merge<false>,
                           dim3(a.Hq, a.B), dim3(256), margs, 0, stream);
}

}  // namespace ssa
