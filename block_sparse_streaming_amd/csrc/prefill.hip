// Streaming sparse attention (SSA) prefill for gfx950.
//
// Operation (LongCat ZigZag Attention digest, section 01 part (1), the SSA
// paragraph; part (2), b=128 s=1 l=7): query i attends to key j iff j <= i and
// (j < s*b or j >= (i/b - l + 1)*b); out = softmax(scale * q k^T) v.
//
// Design (one work-group = 128 query rows of one head, 4 waves x 32 rows):
//  * The key set of a query tile is the union of at most two contiguous ranges,
//    the sink range [0, min(sb, q1)) and the local range [lo(q0), q1); only
//    these are visited, in 64-key sub-tiles (<= 2*(s+l) sub-tiles per tile for
//    b = 128), so the work is linear in the sequence length.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    in the 32x32 accumulator layout every lane holds ONE query column and 16
//    keys, so the row max / row sum of the online softmax are per-lane plus a
//    single exchange between the two half-waves.
//  * O^T = V^T P^T reuses the score registers directly as the B operand (no
//    shuffles); V is staged into LDS transposed, with its key order permuted to
//    match the accumulator layout, so each A-operand fetch is one 16-byte read.
//  * Only sub-tiles that cross a window edge or the diagonal are masked.
//  * Work-group ids are remapped so that each XCD (own L2) runs a contiguous
//    run of query tiles of one head: the sink tile and overlapping local tiles
//    are then L2 hits.
//  * fp32 inputs take v_mfma_f32_32x32x2f32 (full fp32 products, no xf32); V
//    then needs no transpose because each lane feeds one key per instruction.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace ssa {
namespace {

constexpr int kBM = 128;      // query rows per work-group
constexpr int kBN = 64;       // keys per sub-tile
constexpr int kThreads = 256;

// Position of key kk (0..63) of a sub-tile inside a V^T row: bits 2 and 3 are
// swapped so that the 8 keys one lane feeds to one P.V instruction (4 keys of
// its half-wave from each of two 4-row groups of the accumulator) are adjacent.
__device__ __forceinline__ int vt_quad_pos(int quad) {
    return 4 * ((quad & ~3) | ((quad & 1) << 1) | ((quad >> 1) & 1));
}

template <bool kBF16, int DQK, int DV>
__global__ __launch_bounds__(kThreads, 2) void ssa_prefill_kernel(const PrefillArgs a) {
    using Elem = std::conditional_t<kBF16, uint16_t, float>;
    // LDS: K tile row-major (one row per key); V^T (bf16: one row per value dim)
    // or V row-major (fp32). Rows are padded by 16 bytes against bank conflicts.
    constexpr int KSTR = kBF16 ? DQK + 8 : DQK + 4;
    constexpr int VSTR = kBF16 ? kBN + 8 : DV + 4;
    constexpr int VROWS = kBF16 ? DV : kBN;
    constexpr int NDB = DV / 32;  // 32-wide output blocks
    __shared__ __attribute__((aligned(16))) Elem k_lds[kBN * KSTR];
    __shared__ __attribute__((aligned(16))) Elem v_lds[VROWS * VSTR];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;

    const int wg = xcd_remap(blockIdx.x, a.total_wgs);
    const int qt = wg % a.num_qtiles;
    const int hb = wg / a.num_qtiles;
    const int h = hb % a.Hq, bb = hb / a.Hq;
    const int g = h / a.group;

    const int64_t N = a.N, b = a.block;
    const int64_t sb = (int64_t)a.sink * b;
    const int64_t q0 = (int64_t)qt * kBM;
    const int64_t q1 = q0 + kBM < N ? q0 + kBM : N;
    const int64_t i = q0 + wave * 32 + l32;  // this lane's query row
    const bool row_ok = i < N;
    const int64_t lo_i = (i / b - a.local + 1) * b;  // first local key of row i
    const int64_t lo_first = (q0 / b - a.local + 1) * b;
    const int64_t lo_last = ((q1 - 1) / b - a.local + 1) * b;
    const int64_t sink_end = sb < q1 ? sb : q1;
    const int64_t loc_begin = lo_first > sink_end ? lo_first : sink_end;

    const Elem *qbase = (const Elem *)a.q + bb * a.qs[0] + h * a.qs[2];
    const Elem *kbase = (const Elem *)a.k + bb * a.ks[0] + g * a.ks[2];
    const Elem *vbase = (const Elem *)a.v + bb * a.vs[0] + g * a.vs[2];

    // Q^T operand, resident in registers for the whole tile.
    constexpr int NQ = kBF16 ? DQK / 16 : DQK / 2;
    using QFrag = std::conditional_t<kBF16, bf16x8, float>;
    QFrag qf[NQ];
    if constexpr (kBF16) {
        const Elem *qrow = qbase + i * a.qs[1] + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < NQ; ++ks) {
            u32x4 w = {0u, 0u, 0u, 0u};
            if (row_ok) w = *(const u32x4 *)(qrow + ks * 16);
            qf[ks] = __builtin_bit_cast(bf16x8, w);
        }
    } else {
        const Elem *qrow = qbase + i * a.qs[1] + hi;
#pragma unroll
        for (int ks = 0; ks < NQ; ++ks) qf[ks] = row_ok ? qrow[2 * ks] : 0.f;
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x16 oacc[NDB];
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;

    for (int rg = 0; rg < 2; ++rg) {
        const int64_t ra = rg == 0 ? 0 : loc_begin;
        const int64_t re = rg == 0 ? sink_end : q1;
        for (int64_t j0 = ra; j0 < re; j0 += kBN) {
            // A sub-tile needs no mask when it lies inside its range, below the
            // diagonal of the tile's first row and, for the local range, above
            // the window start of the tile's last row.
            const bool need_mask =
                !((j0 + kBN <= re) && (j0 + kBN - 1 <= q0) && (rg == 0 || j0 >= lo_last));

            // Keys past the range end are zero-filled, never read: nothing outside
            // the tile's attended set (re <= q1 <= N) reaches the arithmetic.
            __syncthreads();  // previous sub-tile fully consumed
            if constexpr (kBF16) {
                constexpr int KCH = DQK / 8;
#pragma unroll
                for (int c = tid; c < kBN * KCH; c += kThreads) {
                    const int row = c / KCH, col = c % KCH;
                    const int64_t j = j0 + row;
                    u32x4 w = {0u, 0u, 0u, 0u};
                    if (j < re) w = *(const u32x4 *)(kbase + j * a.ks[1] + col * 8);
                    *(u32x4 *)(k_lds + row * KSTR + col * 8) = w;
                }
                constexpr int VCH = DV / 8;
                constexpr int UNITS = (kBN / 4) * VCH;
#pragma unroll
                for (int u = tid; u < UNITS; u += kThreads) {
                    const int dc = u % VCH, quad = u / VCH;
                    u32x4 rows[4];
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int64_t j = j0 + 4 * quad + rr;
                        rows[rr] = u32x4{0u, 0u, 0u, 0u};
                        if (j < re) rows[rr] = *(const u32x4 *)(vbase + j * a.vs[1] + dc * 8);
                    }
                    const int pos = vt_quad_pos(quad);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        u32x2 w2 = {pick_pair(rows[0], rows[1], e), pick_pair(rows[2], rows[3], e)};
                        *(u32x2 *)(v_lds + (dc * 8 + e) * VSTR + pos) = w2;
                    }
                }
            } else {
                constexpr int KCH = DQK / 4;
#pragma unroll
                for (int c = tid; c < kBN * KCH; c += kThreads) {
                    const int row = c / KCH, col = c % KCH;
                    const int64_t j = j0 + row;
                    f32x4 w = {0.f, 0.f, 0.f, 0.f};
                    if (j < re) w = *(const f32x4 *)(kbase + j * a.ks[1] + col * 4);
                    *(f32x4 *)(k_lds + row * KSTR + col * 4) = w;
                }
                constexpr int VCH = DV / 4;
#pragma unroll
                for (int c = tid; c < kBN * VCH; c += kThreads) {
                    const int row = c / VCH, col = c % VCH;
                    const int64_t j = j0 + row;
                    f32x4 w = {0.f, 0.f, 0.f, 0.f};
                    if (j < re) w = *(const f32x4 *)(vbase + j * a.vs[1] + col * 4);
                    *(f32x4 *)(v_lds + row * VSTR + col * 4) = w;
                }
            }
            __syncthreads();

            // S^T = K Q^T for two 32-key blocks. Accumulator element r of lane
            // (l32, hi) is key 8*(r/4) + 4*hi + r%4 of the block, query l32.
            f32x16 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
                const Elem *krow = k_lds + (kb * 32 + l32) * KSTR;
#pragma unroll
                for (int ks = 0; ks < NQ; ++ks) {
                    if constexpr (kBF16) {
                        const bf16x8 kf = *(const bf16x8 *)(krow + ks * 16 + 8 * hi);
                        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[kb], 0, 0, 0);
                    } else {
                        const float kf = krow[2 * ks + hi];
                        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kf, qf[ks], sacc[kb], 0, 0, 0);
                    }
                }
            }

            // Online softmax in base 2 (scores pre-multiplied by scale*log2 e).
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float x = sacc[kb][r] * a.scale_log2;
                    if (need_mask) {
                        const int64_t j = j0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                        const bool ok = (j < re) && (j <= i) && (j < sb || j >= lo_i);
                        x = ok ? x : -INFINITY;
                    }
                    sacc[kb][r] = x;
                    mx = fmaxf(mx, x);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_use);
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fast_exp2(sacc[kb][r] - m_use);
                    sacc[kb][r] = p;
                    rs += p;
                }
            l_run = l_run * alpha + rs;
            m_run = m_new;
#pragma unroll
            for (int d = 0; d < NDB; ++d)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;

            // O^T += V^T P^T.
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if constexpr (kBF16) {
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        u32x4 pw;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            pw[e] = pack_bf16x2(sacc[kb][8 * c + 2 * e], sacc[kb][8 * c + 2 * e + 1]);
                        const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
                        for (int d = 0; d < NDB; ++d) {
                            const bf16x8 vf = *(const bf16x8 *)(v_lds + (d * 32 + l32) * VSTR + kb * 32 +
                                                                16 * c + 8 * hi);
                            oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, oacc[d], 0, 0, 0);
                        }
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
#pragma unroll
                        for (int d = 0; d < NDB; ++d) {
                            const float vf = v_lds[key * VSTR + d * 32 + l32];
                            oacc[d] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf, sacc[kb][r], oacc[d], 0, 0, 0);
                        }
                    }
                }
            }
        }
    }

    // Epilogue: O = O / l, lse = ln 2 * (m + log2 l).
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.f / l_tot;
    if (row_ok) {
        Elem *orow = (Elem *)a.o + bb * a.os[0] + i * a.os[1] + h * a.os[2];
#pragma unroll
        for (int d = 0; d < NDB; ++d)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int col = d * 32 + 8 * rq + 4 * hi;
                const float v0 = oacc[d][4 * rq + 0] * inv, v1 = oacc[d][4 * rq + 1] * inv;
                const float v2 = oacc[d][4 * rq + 2] * inv, v3 = oacc[d][4 * rq + 3] * inv;
                if constexpr (kBF16) {
                    *(u32x2 *)(orow + col) = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
                } else {
                    *(f32x4 *)(orow + col) = f32x4{v0, v1, v2, v3};
                }
            }
        if (a.lse && hi == 0) a.lse[((int64_t)bb * a.Hq + h) * N + i] = (m_run + log2f(l_tot)) * kLn2;
    }
}

template <bool kBF16, int DQK, int DV>
hipError_t launch(const PrefillArgs &a, hipStream_t stream) {
    void *args[] = {(void *)&a};
    return hipLaunchKernel((const void *)ssa_prefill_kernel<kBF16, DQK, DV>, dim3(a.total_wgs),
                           dim3(kThreads), args, 0, stream);
}

}  // namespace

bool prefill_supported(bool bf16, int d_qk, int d_v) {
    if (bf16) return (d_qk == 64 && d_v == 64) || (d_qk == 128 && d_v == 128) || (d_qk == 192 && d_v == 128);
    return (d_qk == 64 && d_v == 64) || (d_qk == 128 && d_v == 128);
}

hipError_t launch_prefill(bool bf16, int d_qk, int d_v, const PrefillArgs &a, hipStream_t stream) {
    if (bf16) {
        if (d_qk == 64 && d_v == 64) return launch<true, 64, 64>(a, stream);
        if (d_qk == 128 && d_v == 128) return launch<true, 128, 128>(a, stream);
        if (d_qk == 192 && d_v == 128) return launch<true, 192, 128>(a, stream);
    } else {
        if (d_qk == 64 && d_v == 64) return launch<false, 64, 64>(a, stream);
        if (d_qk == 128 && d_v == 128) return launch<false, 128, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace ssa
