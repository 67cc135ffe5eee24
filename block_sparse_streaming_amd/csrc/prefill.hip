// Streaming sparse attention (SSA) prefill for gfx950.
//
// Operation (LongCat ZigZag Attention digest, section 01 part (1), the SSA
// paragraph; part (2), b=128 s=1 l=7): query i attends to key j iff j <= i and
// (j < s*b or j >= (i/b - l + 1)*b); out = softmax(scale * q k^T) v.
//
// Design (one work-group = 128 query rows of one head, 4 waves x 32 rows):
//  * The key set of a query tile is the union of at most two contiguous ranges,
//    the sink range [0, min(sb, q1)) and the local range [lo(q0), q1); only
//    these are visited, in 64-key sub-tiles (16 sub-tiles per steady-state
//    tile at b = 128), so the work is linear in the sequence length.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    in the 32x32 accumulator layout every lane holds ONE query column and 16
//    keys, so the row max / row sum of the online softmax are per-lane plus a
//    single exchange between the two half-waves.
//  * O^T = V^T P^T reuses the score registers directly as the B operand (no
//    shuffles). V stays row-major in LDS; the A operand is gathered with the
//    gfx950 LDS transpose read, two 8-byte reads per instruction.
//  * bf16 K/V sub-tiles are streamed global -> LDS by direct transfers into
//    two buffers: sub-tile t+1 is in flight while t is computed, and no
//    registers are spent on staging. Rows are XOR-swizzled in 16-byte units so
//    that both the score-operand reads (16 keys, one column) and the transpose
//    reads (4 keys x 64 bytes) hit distinct LDS banks.
//  * Only sub-tiles that cross a window edge or the diagonal are masked. A
//    wave whose rows attend every sub-tile of the steady-state loop whole runs
//    a second copy of the loop with no mask code (chosen once per loop: a
//    per-sub-tile choice leaves the paths' registers apart and costs moves
//    where they join).
//  * Work-group ids are remapped so that each XCD (own L2) runs a contiguous
//    run of query tiles of one head: the sink tile and overlapping local tiles
//    are then L2 hits.
//  * Each transfer addresses a wave-uniform base in SGPRs plus a 32-bit lane
//    offset computed once, so a transfer costs no vector address arithmetic.
//  * The output tile is staged through LDS and written as whole 16-byte row
//    pieces.
//  * fp32 inputs take v_mfma_f32_32x32x2f32 (full fp32 products, no xf32) on a
//    register-staged loop in which the waves of a 32-row work-group split the
//    key sub-tiles and merge their softmax states; V then needs no transpose
//    because each lane feeds one key per instruction.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace ssa {
namespace {

constexpr int kThreads = 256;
// Growth of a row max (log2 units) tolerated before the accumulators are
// rescaled; probabilities stay below 2^8, far from fp32/bf16 overflow.
constexpr float kRescaleSlack = 8.f;

// Compile-time tag: whether a sub-tile is known to need no mask.
template <bool W>
struct Whole {
    static constexpr bool value = W;
};

// ---------------------------------------------------------------------------
// bf16: pipelined direct-to-LDS kernel.
// ---------------------------------------------------------------------------
// XOR swizzle of the 16-byte column unit of K row `row` (CK units per row):
// 16 consecutive rows read at one column land in 16 distinct bank groups.
template <int CK>
__device__ __forceinline__ int k_swz(int row) {
    if constexpr (CK % 16 == 0) return row & 15;  // rows a multiple of 256 B
    else return (row >> 1) & 7;                   // rows 128 B mod 256 B
}
// XOR swizzle of V rows: 4 consecutive rows x 4 consecutive units (one
// transpose read of a half-wave) land in 16 distinct bank groups.
template <int CV>
__device__ __forceinline__ int v_swz(int row) {
    if constexpr (CV % 16 == 0) return 4 * (row & 3);
    else return 4 * ((row >> 1) & 1);
}

// MODE kModeDual: one pass yields both SSA attention and full causal
// attention. The SSA sub-tiles come first, so the running state after the
// last of them is the SSA result (written to o / lse); the walk then goes on
// over the keys SSA leaves out, [min(s*b, q1), lo(q1-1)) with key j taken by
// row i iff j < lo(i), and ends with full causal attention (o_full / lse_full,
// and the mix).
// MODE kModePaged: the new tokens of each sequence (a prefill chunk, or a few
// decode tokens) against a paged cache. A tile is 128 consecutive new rows of
// one sequence, at the last positions of its context; every key row is found
// through the page table (page ids of the next sub-tile are read one stage
// ahead, one per lane, and shared with ds_bpermute).
template <int DQK, int DV, int MODE>
__global__ __launch_bounds__(kThreads, 2) void ssa_prefill_bf16(const PrefillArgs a) {
    constexpr bool DUAL = MODE == kModeDual, PAGED = MODE == kModePaged;
    constexpr int CK = DQK / 8, CV = DV / 8;   // 16-byte units per K / V row
    constexpr int NIK = CK / 4, NIV = CV / 4;  // direct transfers per wave per sub-tile
    constexpr int NDMA = NIK + NIV;
    // Memory operations a stage leaves in flight: its transfers, plus in
    // paged mode the page-id read of the stage after it.
    constexpr int NW = NDMA + (PAGED ? 1 : 0);
    constexpr int NQ = DQK / 16, NDB = DV / 32;
    static_assert(CK % 4 == 0 && CV % 4 == 0, "tile rows must split into whole waves");
    __shared__ __attribute__((aligned(1024))) uint16_t k_buf0[kBN * DQK];
    __shared__ __attribute__((aligned(1024))) uint16_t k_buf1[kBN * DQK];
    __shared__ __attribute__((aligned(1024))) uint16_t v_buf0[kBN * DV];
    __shared__ __attribute__((aligned(1024))) uint16_t v_buf1[kBN * DV];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS bases stay scalar
    const int l32 = lane & 31, hi = lane >> 5;

    int qt, hb;
    if constexpr (DUAL) {
        // Full causal work grows with the tile index: dispatch the longest
        // tiles first, all heads of one tile index together. Consecutive
        // work-groups go to different XCDs, so when B * Hq is a multiple of 8
        // every tile of a head runs on the same XCD (its L2).
        const int per = a.total_wgs / a.num_qtiles;  // B * Hq
        qt = a.num_qtiles - 1 - (int)blockIdx.x / per;
        hb = (int)blockIdx.x % per;
    } else {
        const int wg = xcd_remap(blockIdx.x, a.total_wgs);
        qt = wg % a.num_qtiles;
        hb = wg / a.num_qtiles;
    }
    // The divisions above run on the vector unit; taking their (uniform)
    // results back to scalar registers keeps every base address derived from
    // them scalar, which the scalar-base transfers below need.
    qt = __builtin_amdgcn_readfirstlane(qt);
    hb = __builtin_amdgcn_readfirstlane(hb);
    const int h = __builtin_amdgcn_readfirstlane(hb % a.Hq), bb = __builtin_amdgcn_readfirstlane(hb / a.Hq);
    const int g = __builtin_amdgcn_readfirstlane(h / a.group);

    // Sequence geometry. Paged: the chunk's rows [0, q_len) sit at positions
    // pos0 .. pos0 + q_len - 1 of a context of ctx tokens; row r of the chunk
    // is packed row q_start + r of q and o. Plain: the whole sequence.
    Geo geo = geo_of(a);
    int pos0 = 0, q_start = 0, q0, q1;
    if constexpr (PAGED) {
        q_start = a.cu_q[bb];
        const int q_len = a.cu_q[bb + 1] - q_start;
        if (qt * kBM >= q_len) return;  // this sequence has fewer tiles (uniform)
        const int64_t cap = (int64_t)a.max_pages * a.page_size;  // no length reads past the table row
        geo.N = a.ctx_lens[bb] < cap ? a.ctx_lens[bb] : (int)cap;
        pos0 = geo.N - q_len;
        pos0 = pos0 > 0 ? pos0 : 0;     // q_len <= ctx is a precondition; stay in bounds
        q0 = pos0 + qt * kBM;
        q1 = imin(pos0 + imin(q_len, qt * kBM + kBM), geo.N);
    } else {
        q0 = qt * kBM;
        q1 = imin(q0 + kBM, a.N);
    }
    const TileRanges tr = tile_ranges_at(geo, q0, q1);
    const int n_end = PAGED ? q1 : a.N;     // rows at positions >= n_end are not computed
    // Visit order of the sub-tiles (plain mode, d_qk = 192): the full 128-key
    // pairs of the local range before its last two sub-tiles are visited by
    // absolute pair index modulo their count, so that the tiles running side
    // by side on an XCD read the same key pairs at the same time (the softmax
    // does not depend on the order). At 256K tokens x 64 heads this cuts the
    // L2 misses 2.3x (their working set otherwise exceeds an XCD's L2); at
    // d = 128 there are no re-reads to save and the order costs time. The
    // sink range and the last two sub-tiles keep their place.
    const int rot_n = (DQK > 128 && !DUAL && !PAGED) ? (tr.n_total - tr.n_sink - 2) >> 1 : 0;
    const int rot_off = rot_n > 1 ? (tr.loc_begin >> 7) % rot_n : 0;
    auto visit = [&](int t) __attribute__((always_inline)) -> int {
        const int u = t - tr.n_sink;
        if (rot_n > 1 && u >= 0 && u < 2 * rot_n) {
            int p = (u >> 1) - rot_off;
            p = p < 0 ? p + rot_n : p;
            return tr.n_sink + 2 * p + (u & 1);
        }
        return t;
    };
    const int i = tr.q0 + wave * 32 + l32;  // this lane's query row (its position)
    const bool row_ok = i < n_end;
    const int lo_i = local_start(geo, i);
    // Index of row i along the token axis of q / o (packed rows when paged).
    const int64_t row_idx = PAGED ? (int64_t)q_start + (i - pos0) : (int64_t)i;

    const uint16_t *qbase = (const uint16_t *)a.q + bb * a.qs[0] + h * a.qs[2];
    const uint16_t *kbase = (const uint16_t *)a.k + (PAGED ? 0 : bb * a.ks[0]) + g * a.ks[2];
    const uint16_t *vbase = (const uint16_t *)a.v + (PAGED ? 0 : bb * a.vs[0]) + g * a.vs[2];
    const int ks1 = (int)a.ks[1], vs1 = (int)a.vs[1];  // token strides (< 2^24, host-checked)

    // Q^T operand, resident in registers for the whole tile.
    bf16x8 qf[NQ];

    // The K / V transfers. For d_qk <= 128 they are issued untracked: the
    // compiler's own tracking of these LDS writes does not survive the loop
    // and adds a full wait before one of the two buffers' P.V reads, stalling
    // on the transfer just issued for the next sub-tile; the explicit waits
    // and barriers below order both buffers. d_qk = 192 (ten transfers per
    // wave and stage) keeps the tracked form, whose loop has no such wait
    // and no M0 save / restore per transfer.
    constexpr bool kTrackedDma = DQK > 128;
    auto dma = [&](const void *src, uint16_t *dst) __attribute__((always_inline)) {
        if constexpr (kTrackedDma) dma16(src, dst);
        else dma16_untracked(src, lds_addr(dst));
    };
    // A transfer from a wave-uniform base plus a per-lane byte offset (rows of
    // one contiguous range, or of one page). The dual kernel keeps the 64-bit
    // form: the scalar bases cost it registers it does not have.
    auto dma_at = [&](const char *base, uint32_t off, uint16_t *dst) __attribute__((always_inline)) {
        if constexpr (kTrackedDma || DUAL) dma(base + off, dst);
        else dma16_sbase_untracked(base, off, lds_addr(dst));
    };
    auto load_q = [&]() __attribute__((always_inline)) {
        const uint16_t *qrow = qbase + row_idx * a.qs[1] + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < NQ; ++ks) {
            u32x4 w = {0u, 0u, 0u, 0u};
            if (row_ok) w = *(const u32x4 *)(qrow + ks * 16);
            qf[ks] = __builtin_bit_cast(bf16x8, w);
        }
    };
    if constexpr (kTrackedDma) load_q();

    // Direct transfers: lane slot p of transfer n covers tile row p / C at
    // physical unit p % C, which holds logical unit (p % C) ^ swz(row). Byte
    // offsets from the sub-tile's first row, computed once per lane; in a
    // sub-tile cut short by its range end, rows past the end re-read the
    // range's last row (masked later), so nothing outside the tile's attended
    // key set is touched.
    auto dma_off = [&](int p, int C, int swz, int stride, int rows_valid) -> uint32_t {
        int row = p / C;
        const int unit = (p % C) ^ swz;
        row = row < rows_valid ? row : rows_valid - 1;
        return (uint32_t)(row * stride + unit * 8) * 2u;
    };
    // Full sub-tiles reuse offsets computed once, when the registers allow it
    // (d_qk = 192 has too many transfers per wave and recomputes them).
    constexpr bool kKeepOffsets = NIK + NIV <= 8;
    uint32_t koff[NIK], voff[NIV];
    if constexpr (kKeepOffsets) {
#pragma unroll
        for (int n = 0; n < NIK; ++n) {
            const int p = (wave * NIK + n) * 64 + lane;
            koff[n] = dma_off(p, CK, k_swz<CK>(p / CK), ks1, kBN);
        }
#pragma unroll
        for (int n = 0; n < NIV; ++n) {
            const int p = (wave * NIV + n) * 64 + lane;
            voff[n] = dma_off(p, CV, v_swz<CV>(p / CV), vs1, kBN);
        }
    }
    // Paged mode: lane l holds the page and slot of key row l of the next
    // sub-tile to be issued (rows past the range end take its last row). The
    // page id comes by a direct transfer into a per-wave LDS slot when the
    // LDS budget of two work-groups per CU leaves room (an explicit counter
    // wait then covers exactly that transfer); otherwise by a register load,
    // before whose use the compiler waits for every transfer in flight.
    constexpr int kLdsBytes = 2 * kBN * (DQK + DV) * 2;
    constexpr bool kIdsInLds = PAGED && 2 * (kLdsBytes + 4 * 64 * 4) <= 160 * 1024;
    __shared__ int32_t id_slot[kIdsInLds ? 4 * 64 : 1];
    const int32_t *ptab = PAGED ? a.page_table + (int64_t)bb * a.max_pages : nullptr;
    int pg_next = 0, sl_next = 0;
    auto read_ids = [&](int t) __attribute__((always_inline)) {
        const SubTile st = sub_tile<false>(tr, t);
        const int tok = st.j0 + imin(lane, st.re - st.j0 - 1);
        const int lp = tok / a.page_size;
        sl_next = tok - lp * a.page_size;
        if constexpr (kIdsInLds) dma4_untracked(ptab + lp, lds_addr(id_slot) + wave * 256);
        else pg_next = ptab[lp];
    };
    auto issue_paged = [&](int t, uint16_t *kb, uint16_t *vb) __attribute__((always_inline)) {
        const SubTile st = sub_tile<false>(tr, t);
        const int rows_valid = st.re - st.j0;
        int pg;
        if constexpr (kIdsInLds) {
            // In flight: this stage's ids, then the previous stage's transfers.
            wait_vmcnt<NDMA>();
            asm volatile("" ::: "memory");
            pg = id_slot[wave * 64 + lane];
            wait_lgkmcnt0();  // read before the next transfer rewrites the slot
            asm volatile("" ::: "memory");
        } else {
            pg = pg_next;
        }
        const int sl = sl_next;
        // Read the next stage's ids before this stage's transfers, so that the
        // transfers stay the youngest operations in flight. The last stage
        // re-reads its own ids, which keeps the count fixed.
        read_ids(imin(t + 1, tr.n_total - 1));
        // A full sub-tile inside one page (pages of 64 tokens or more, blocks
        // aligned to 64): one page base and the contiguous path's offsets.
        const int sl0 = __builtin_amdgcn_readfirstlane(sl);
        if (kKeepOffsets && rows_valid >= kBN && sl0 + kBN <= a.page_size) {
            const int64_t pg0 = __builtin_amdgcn_readfirstlane(pg);
            const char *kt = (const char *)(kbase + pg0 * a.ks[0] + (int64_t)sl0 * a.ks[1]);
            const char *vt = (const char *)(vbase + pg0 * a.vs[0] + (int64_t)sl0 * a.vs[1]);
#pragma unroll
            for (int n = 0; n < NIK; ++n) dma_at(kt, koff[n], kb + (wave * NIK + n) * 512);
#pragma unroll
            for (int n = 0; n < NIV; ++n) dma_at(vt, voff[n], vb + (wave * NIV + n) * 512);
            return;
        }
        auto src = [&](int p, int C, int swz, int64_t s0, int64_t s1) __attribute__((always_inline)) {
            const int row = imin(p / C, rows_valid - 1);
            const int64_t page = __shfl(pg, row), slot = __shfl(sl, row);
            return page * s0 + slot * s1 + (((p % C) ^ swz) * 8);
        };
#pragma unroll
        for (int n = 0; n < NIK; ++n) {
            const int p = (wave * NIK + n) * 64 + lane;
            dma(kbase + src(p, CK, k_swz<CK>(p / CK), a.ks[0], a.ks[1]), kb + (wave * NIK + n) * 512);
        }
#pragma unroll
        for (int n = 0; n < NIV; ++n) {
            const int p = (wave * NIV + n) * 64 + lane;
            dma(vbase + src(p, CV, v_swz<CV>(p / CV), a.vs[0], a.vs[1]), vb + (wave * NIV + n) * 512);
        }
    };
    auto issue = [&](int t, uint16_t *kb, uint16_t *vb) __attribute__((always_inline)) {
        if constexpr (PAGED) {
            issue_paged(t, kb, vb);
            return;
        }
        const SubTile st = sub_tile<DUAL>(tr, visit(t));
        const int rows_valid = st.re - st.j0;
        const char *kt = (const char *)(kbase + (int64_t)st.j0 * a.ks[1]);
        const char *vt = (const char *)(vbase + (int64_t)st.j0 * a.vs[1]);
        if (kKeepOffsets && rows_valid >= kBN) {
#pragma unroll
            for (int n = 0; n < NIK; ++n) dma_at(kt, koff[n], kb + (wave * NIK + n) * 512);
#pragma unroll
            for (int n = 0; n < NIV; ++n) dma_at(vt, voff[n], vb + (wave * NIV + n) * 512);
        } else {
#pragma unroll
            for (int n = 0; n < NIK; ++n) {
                const int p = (wave * NIK + n) * 64 + lane;
                dma_at(kt, dma_off(p, CK, k_swz<CK>(p / CK), ks1, rows_valid), kb + (wave * NIK + n) * 512);
            }
#pragma unroll
            for (int n = 0; n < NIV; ++n) {
                const int p = (wave * NIV + n) * 64 + lane;
                dma_at(vt, dma_off(p, CV, v_swz<CV>(p / CV), vs1, rows_valid), vb + (wave * NIV + n) * 512);
            }
        }
    };

    float m_run = -INFINITY, l_run = 0.f;
    f32x16 oacc[NDB];
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;

    // LDS byte offsets that depend only on the lane.
    // K (score operand): row l32 (+32 per key block), unit (2ks + hi) ^ swz;
    // since 2ks and hi occupy different bits, unit*16 = (32ks) ^ kz.
    const uint32_t k_lane = (uint32_t)l32 * (DQK * 2);
    const uint32_t kz = (uint32_t)((hi ^ k_swz<CK>(l32)) << 4);
    // V (transpose reads): lane s of 16-lane group G reads key row
    // 4*hi + s/4 (+ block offsets) at value column 16*(G&1) + 4*(s&3) + 32d.
    // The row swizzle depends only on s, so the physical unit of column block
    // d is 4*(d ^ y) + x and each block's address is a lane constant.
    const int grp = lane >> 4, s16 = lane & 15;
    const int tr_row = 4 * hi + (s16 >> 2);
    const int tr_col = 16 * (grp & 1) + 4 * (s16 & 3);
    const int vy = v_swz<CV>(tr_row) >> 2;
    uint32_t v_lane[NDB];
#pragma unroll
    for (int d = 0; d < NDB; ++d)
        v_lane[d] = (uint32_t)tr_row * (DV * 2) + (uint32_t)((4 * (d ^ vy) + (tr_col >> 3)) << 4) +
                    (uint32_t)((tr_col & 4) << 1);
    const int jl = 4 * hi;  // key offset of this lane's accumulator rows

    // Rows of this wave: r_first .. r_last (clamped to the sequence), and the
    // window starts of its first and last rows.
    const int r_first = tr.q0 + wave * 32;
    const int r_last = r_first + 31 < n_end - 1 ? r_first + 31 : n_end - 1;
    const int lo_first_w = local_start(geo, r_first), lo_last_w = local_start(geo, r_last);

    // Whether sub-tile t is attended by every row of this wave at every key:
    // then it needs no mask.
    auto whole_at = [&](int t) __attribute__((always_inline)) -> bool {
        const SubTile st = sub_tile<DUAL>(tr, t);
        if (DUAL && t >= tr.n_total) return r_first < n_end && st.j0 + kBN <= lo_first_w;
        const bool local = t >= tr.n_sink;
        return r_first < n_end && st.j0 + kBN <= st.re && (!local || st.j0 >= lo_last_w) &&
               st.j0 + kBN - 1 <= r_first;
    };

    // One sub-tile. With a true `whole` tag the caller knows the sub-tile
    // needs no mask, and this copy has no mask code at all: a copy that
    // chooses among the mask classes at run time keeps the scores of its
    // paths in different registers and pays for moving them where the paths
    // join.
    auto compute = [&](auto whole, int t, const uint16_t *kb, const uint16_t *vb) __attribute__((always_inline)) {
        const SubTile st = sub_tile<DUAL>(tr, visit(t));
        bool no_mask = true, causal_only = false;
        int edge = i;  // in a causal_only sub-tile, keys up to edge are attended
        if constexpr (decltype(whole)::value) {
        } else if (DUAL && t >= tr.n_total) {
            // Complement sub-tile: key j (>= s*b) is attended iff j < lo_i,
            // which also keeps out the re-read rows past the range end.
            if (r_first >= n_end || st.j0 >= lo_last_w) return;
            no_mask = st.j0 + kBN <= lo_first_w;
            causal_only = !no_mask;
            edge = lo_i - 1;
        } else {
            // What this sub-tile means for this wave's rows (wave-uniform):
            // keys of a local sub-tile lie past the sink range, so there a key
            // is attended iff lo_i <= j <= i; in the sink range iff j <= i.
            const bool local = t >= tr.n_sink;
            const int kend = st.j0 + kBN < st.re ? st.j0 + kBN : st.re;  // exclusive
            if (r_first >= n_end || st.j0 > r_last || (local && kend <= lo_first_w)) return;  // nothing attended
            const bool full = st.j0 + kBN <= st.re && (!local || st.j0 >= lo_last_w);
            no_mask = full && st.j0 + kBN - 1 <= r_first;  // every key <= every row
            causal_only = full && !no_mask;                // only j <= i can fail
        }
        // Re-derive the lane offsets here (the empty asm hides their origin)
        // so that address arithmetic is not hoisted out of the loop into
        // registers that would stay live across it.
        uint32_t kl = k_lane, kzz = kz;
        asm volatile("" : "+v"(kl), "+v"(kzz));
        uint32_t vl[NDB];
#pragma unroll
        for (int d = 0; d < NDB; ++d) {
            vl[d] = v_lane[d];
            asm volatile("" : "+v"(vl[d]));
        }
        const char *kc = (const char *)kb + kl;
        const char *vc = (const char *)vb;
        // S^T = K Q^T for two 32-key blocks: accumulator element r of lane
        // (l32, hi) is key 8*(r/4) + 4*hi + r%4 of the block, query l32.
        f32x16 sacc[2];
#pragma unroll
        for (int kbk = 0; kbk < 2; ++kbk) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kbk][r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < NQ; ++ks) {
                const uint32_t off = kbk * 32 * DQK * 2 + (((uint32_t)(32 * (ks & 7)) ^ kzz) + (ks >> 3) * 256);
                const bf16x8 kf = *(const bf16x8 *)(kc + off);
                sacc[kbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[kbk], 0, 0, 0);
            }
        }

        // Online softmax in base 2. The max is taken on raw scores (scale > 0),
        // and p = 2^(s*c - m) is one FMA and one exp. The running max m_run is
        // only moved when some lane's max grows by more than kRescaleSlack
        // (in log2 units): until then p <= 2^kRescaleSlack and the O/l rescale
        // is skipped. O and l always use the same m_run, so O / l is exact.
        float mx = -INFINITY;
        if (causal_only) {
            const int d0 = edge - (st.j0 + jl);  // key offset k is attended iff k <= d0
#pragma unroll
            for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float x = kbk * 32 + 8 * (r >> 2) + (r & 3) <= d0 ? sacc[kbk][r] : -INFINITY;
                    sacc[kbk][r] = x;
                    mx = fmaxf(mx, x);
                }
        } else if (!no_mask) {
            const int jb = st.j0 + jl;
#pragma unroll
            for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = jb + kbk * 32 + 8 * (r >> 2) + (r & 3);
                    const bool ok = (j < st.re) & (j <= i) & ((j < tr.sb) | (j >= lo_i));
                    const float x = ok ? sacc[kbk][r] : -INFINITY;
                    sacc[kbk][r] = x;
                    mx = fmaxf(mx, x);
                }
        } else {
#pragma unroll
            for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kbk][r]);
        }
        mx = max_xor32(mx) * a.scale_log2;
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
            l_run *= alpha;
#pragma unroll
            for (int d = 0; d < NDB; ++d)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
            m_run = m_new;
        }
        const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
        float rs = 0.f;
#pragma unroll
        for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(__builtin_fmaf(sacc[kbk][r], a.scale_log2, neg_m));
                sacc[kbk][r] = p;
                rs += p;
            }
        l_run += rs;

        // O^T += V^T P^T. Instruction c of key block kbk consumes keys
        // kbk*32 + 16c + {0..3, 8..11} (+4 on the upper half-wave): exactly the
        // accumulator elements 8c..8c+7 of the score block.
#pragma unroll
        for (int kbk = 0; kbk < 2; ++kbk) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                u32x4 pw;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    pw[e] = pack_bf16x2(sacc[kbk][8 * c + 2 * e], sacc[kbk][8 * c + 2 * e + 1]);
                const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
                constexpr int kRowBytes = DV * 2;
                const uint32_t blk = (uint32_t)(kbk * 32 + 16 * c) * kRowBytes;
#pragma unroll
                for (int d = 0; d < NDB; ++d) {
                    const i16x4 lo = lds_read_tr16(vc + vl[d] + blk);
                    const i16x4 up = lds_read_tr16(vc + vl[d] + blk + 8 * kRowBytes);
                    const i16x8 v8 = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
                    oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v8), pf,
                                                                      oacc[d], 0, 0, 0);
                }
            }
        }
    };

    // Writes O / l of the running state to `out` (row i) and its lse.
    auto store_out = [&](void *out, float *lse_out) __attribute__((always_inline)) {
        const float l_tot = l_run + __shfl_xor(l_run, 32);
        const float inv = 1.f / l_tot;
        uint16_t *orow = (uint16_t *)out + bb * a.os[0] + row_idx * a.os[1] + h * a.os[2];
#pragma unroll
        for (int d = 0; d < NDB; ++d)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const u32x2 w{pack_bf16x2(oacc[d][4 * rq] * inv, oacc[d][4 * rq + 1] * inv),
                              pack_bf16x2(oacc[d][4 * rq + 2] * inv, oacc[d][4 * rq + 3] * inv)};
                if (row_ok) *(u32x2 *)(orow + d * 32 + 8 * rq + 4 * hi) = w;
            }
        if (row_ok && lse_out && hi == 0) {
            const int64_t li = PAGED ? row_idx * a.Hq + h : ((int64_t)bb * a.Hq + h) * a.N + i;
            lse_out[li] = (m_run + log2f(l_tot)) * kLn2;
        }
    };
    // The final output of the single-result modes, staged through LDS (the
    // V buffers, free once every wave has passed the barrier below): each
    // wave writes its 32 x DV tile row-major (16-byte units XOR-swizzled by
    // row), then reads it back as whole rows, so that every global store
    // writes 16 contiguous bytes and a store instruction covers whole rows
    // instead of 8-byte pieces of 32 rows.
    auto store_out_staged = [&]() __attribute__((always_inline)) {
        const float l_tot = l_run + __shfl_xor(l_run, 32);
        const float inv = 1.f / l_tot;
        constexpr int kRowB = DV * 2, kUnits = kRowB / 16;
        static_assert(kUnits == 8 || kUnits == 16, "rows of 128 or 256 bytes");
        barrier_lds_drained();
        char *stage = (char *)(wave < 2 ? v_buf0 : v_buf1) + (wave & 1) * 32 * kRowB;
#pragma unroll
        for (int d = 0; d < NDB; ++d)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const u32x2 w{pack_bf16x2(oacc[d][4 * rq] * inv, oacc[d][4 * rq + 1] * inv),
                              pack_bf16x2(oacc[d][4 * rq + 2] * inv, oacc[d][4 * rq + 3] * inv)};
                const int unit = (4 * d + rq) ^ (l32 & (kUnits - 1));
                *(u32x2 *)(stage + l32 * kRowB + unit * 16 + 8 * hi) = w;
            }
        const int r_base = tr.q0 + wave * 32;  // position of the wave's first row
        const int64_t idx_base = PAGED ? (int64_t)q_start + (r_base - pos0) : (int64_t)r_base;
        uint16_t *obase = (uint16_t *)a.o + bb * a.os[0] + h * a.os[2];
#pragma unroll
        for (int n = 0; n < 32 * kUnits / 64; ++n) {
            const int lin = n * 64 + lane;
            const int r = lin / kUnits, u = lin % kUnits;
            const u32x4 v = *(const u32x4 *)(stage + r * kRowB + ((u ^ (r & (kUnits - 1))) * 16));
            if (r_base + r < n_end) *(u32x4 *)(obase + (idx_base + r) * a.os[1] + u * 8) = v;
        }
        if (row_ok && a.lse && hi == 0) {
            const int64_t li = PAGED ? row_idx * a.Hq + h : ((int64_t)bb * a.Hq + h) * a.N + i;
            a.lse[li] = (m_run + log2f(l_tot)) * kLn2;
        }
    };
    auto step = [&](auto whole, int t, const uint16_t *kb, const uint16_t *vb) __attribute__((always_inline)) {
        compute(whole, t, kb, vb);
        // The SSA result. Copies without masks run past the SSA range only.
        if constexpr (DUAL && !decltype(whole)::value) {
            if (t == tr.n_total - 1) store_out(a.o, a.lse);
        }
    };

    // Two-stage pipeline: sub-tile t+1 streams into the other buffer while t
    // is computed. Buffers are separate LDS objects so that, for the tracked
    // transfers of d_qk = 192, the compiler can tell the in-flight transfers
    // from the buffer being read; the steady-state loop issues and waits
    // unconditionally and the last one or two sub-tiles are peeled, so every
    // wait is a fixed count.
    const int T = DUAL ? tr.n_all : tr.n_total;
    int t = 0;
    if (T > 0) {
        if constexpr (PAGED) {
            read_ids(0);
            wait_vmcnt<0>();
        }
        issue(0, k_buf0, v_buf0);
    }
    if constexpr (!kTrackedDma) {
        // q after the first sub-tile's transfers, and one wait for both
        // (each is needed before the first product). The compiler does not
        // see the untracked transfers; without this wait it would order the
        // q loads by a full wait inside the loop, which would also wait for
        // the next sub-tile's transfers.
        load_q();
        wait_vmcnt<0>();
    }
    // The loop covers sub-tiles [0, n_loop). A wave whose rows attend all of
    // them whole (every tile past the first l blocks when the block size is a
    // multiple of 64) runs a copy without mask code; the other waves of the
    // work-group may run the general copy, with the same transfers and
    // barriers in the same order. In dual mode the diagonal sub-tiles sit
    // between the local and the complement range: the SSA range runs the
    // general copy, and the complement range, whole for every row when the
    // tile's rows share one window start, chooses its copy by itself.
    const int n_loop = 2 * ((T - 1) / 2);
    auto pair = [&](auto whole) __attribute__((always_inline)) {
        issue(t + 1, k_buf1, v_buf1);
        wait_vmcnt<NW>();
        barrier_no_fence();
        step(whole, t, k_buf0, v_buf0);
        barrier_lds_drained();
        issue(t + 2, k_buf0, v_buf0);
        wait_vmcnt<NW>();
        barrier_no_fence();
        step(whole, t + 1, k_buf1, v_buf1);
        barrier_lds_drained();
    };
    int t_whole = 0;  // first sub-tile of the range checked for the copy without masks
    if constexpr (DUAL) {
        for (; t + 2 < T && t < tr.n_total; t += 2) pair(Whole<false>{});
        t_whole = t;
    }
    // The dual kernel with d_qk = 192 has no registers for a second copy.
    constexpr bool kWholeCopy = !(DUAL && DQK > 128);
    bool whole_loop = false;
    if (kWholeCopy && t < n_loop) {
        // Whole-ness is monotone over each range (the window start bounds a
        // local or complement sub-tile from one side, the rows from the
        // other), so the ends of each range decide it.
        const int ts = imin(tr.n_sink, n_loop) - 1;  // last sink sub-tile in the loop
        if (DUAL && t_whole >= tr.n_total) whole_loop = whole_at(t_whole) && whole_at(n_loop - 1);
        else whole_loop = (ts < 0 || whole_at(ts)) &&
                          (tr.n_sink >= n_loop || (whole_at(tr.n_sink) && whole_at(n_loop - 1)));
    }
    if (kWholeCopy && whole_loop) {
        for (; t + 2 < T; t += 2) pair(Whole<kWholeCopy>{});
    } else {
        for (; t + 2 < T; t += 2) pair(Whole<false>{});
    }
    if (t + 1 < T) {
        issue(t + 1, k_buf1, v_buf1);
        wait_vmcnt<NW>();
        barrier_no_fence();
        step(Whole<false>{}, t, k_buf0, v_buf0);
        wait_vmcnt<0>();
        barrier_no_fence();
        step(Whole<false>{}, t + 1, k_buf1, v_buf1);
    } else if (t < T) {
        wait_vmcnt<0>();
        barrier_no_fence();
        step(Whole<false>{}, t, k_buf0, v_buf0);
    }

    // Epilogue: O = O / l, lse = ln 2 * (m + log2 l).
    if constexpr (!DUAL) {
        store_out_staged();
    } else {
        store_out(a.o_full, a.lse_full);
        if (a.o_mix) {
            // alpha * O_full + (1 - alpha) * O_ssa, from the fp32 full result
            // and the rounded SSA result this lane stored earlier (a wave's
            // accesses to one address stay in order; the opaque offset keeps
            // the compiler from carrying the stored values in registers).
            // o_mix overlaps no other buffer, so every piece of the SSA row is
            // loaded before the first store: one wait, not one per piece.
            const float l_tot = l_run + __shfl_xor(l_run, 32);
            const float wf = a.alpha / l_tot, ws = 1.f - a.alpha;
            int64_t off = bb * a.os[0] + (int64_t)i * a.os[1] + h * a.os[2];
            uint16_t *mrow = (uint16_t *)a.o_mix + off;
            asm volatile("" : "+v"(off));
            const uint16_t *srow = (const uint16_t *)a.o + off;
            auto up = [](uint32_t w, int half) { return __uint_as_float(half ? w & 0xffff0000u : w << 16); };
            if (row_ok) {
                u32x2 sv[NDB][4];
#pragma unroll
                for (int d = 0; d < NDB; ++d)
#pragma unroll
                    for (int rq = 0; rq < 4; ++rq) sv[d][rq] = *(const u32x2 *)(srow + d * 32 + 8 * rq + 4 * hi);
#pragma unroll
                for (int d = 0; d < NDB; ++d)
#pragma unroll
                    for (int rq = 0; rq < 4; ++rq) {
                        float m[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            m[e] = __builtin_fmaf(oacc[d][4 * rq + e], wf, ws * up(sv[d][rq][e >> 1], e & 1));
                        *(u32x2 *)(mrow + d * 32 + 8 * rq + 4 * hi) =
                            u32x2{pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3])};
                    }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// fp32: register-staged kernel on the fp32 MFMA.
// ---------------------------------------------------------------------------
// One work-group = 32 query rows of one head, NW waves (8 at d = 64, 4 at
// d = 128, as the LDS allows). All waves hold the same rows; the rows' key
// ranges are cut into 32-key sub-tiles, wave w takes sub-tiles w, w + NW, ...
// and keeps its own online-softmax state, and the states are merged through
// LDS at the end. Small fp32 workloads (2K tokens x 4 heads) thus fill the
// chip, and 32-key sub-tiles keep the waves' shares within one sub-tile of
// each other. Each wave stages its sub-tile's K and V through a private LDS
// slice (rows padded by 4 floats), so no barrier is needed until the merge;
// the next sub-tile's rows are loaded into registers while this one is
// computed.
constexpr int kF32Rows = 32;
constexpr int kF32Keys = 32;

template <int DQK, int DV>
constexpr int f32_waves() { return DQK <= 64 ? 8 : 4; }

template <int DQK, int DV>
__global__ __launch_bounds__((64 * f32_waves<DQK, DV>()), 1) void ssa_prefill_f32(const PrefillArgs a) {
    constexpr int NW = f32_waves<DQK, DV>();
    constexpr int KSTR = DQK + 4, VSTR = DV + 4;  // padded rows (floats)
    constexpr int VOFF = kF32Keys * KSTR;          // V rows follow the K rows in a slice
    constexpr int SLICE = kF32Keys * (KSTR + VSTR);
    constexpr int NQ = DQK / 2, NDB = DV / 32;
    constexpr int NLK = kF32Keys * DQK / 4 / 64, NLV = kF32Keys * DV / 4 / 64;  // 16-byte loads per lane
    constexpr int OSTR = DV + 1;                    // merge rows, padded
    static_assert(kF32Rows * OSTR + 2 * kF32Rows <= SLICE, "merge state fits a wave's slice");
    __shared__ __attribute__((aligned(16))) float slices[NW][SLICE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    const int wg = xcd_remap(blockIdx.x, a.total_wgs);
    const int qt = __builtin_amdgcn_readfirstlane(wg % a.num_qtiles);
    const int hb = __builtin_amdgcn_readfirstlane(wg / a.num_qtiles);
    const int h = hb % a.Hq, bb = hb / a.Hq;
    const int g = h / a.group;

    const Geo geo = geo_of(a);
    const int q0 = qt * kF32Rows;
    const TileRanges tr = tile_ranges_at(geo, q0, imin(q0 + kF32Rows, a.N));
    // 32-key sub-tiles of the two ranges.
    const int n_sink = (tr.sink_end + kF32Keys - 1) / kF32Keys;
    const int n_total = n_sink + (tr.q1 - tr.loc_begin + kF32Keys - 1) / kF32Keys;
    struct Sub {
        int j0, re;
        bool need_mask;
    };
    auto sub_at = [&](int t) __attribute__((always_inline)) {
        Sub st;
        const bool local = t >= n_sink;
        st.j0 = local ? tr.loc_begin + (t - n_sink) * kF32Keys : t * kF32Keys;
        st.re = local ? tr.q1 : tr.sink_end;
        st.need_mask = !((st.j0 + kF32Keys <= st.re) && (st.j0 + kF32Keys - 1 <= tr.q0) &&
                         (!local || st.j0 >= tr.lo_last));
        return st;
    };
    const int i = q0 + l32;
    const bool row_ok = i < a.N;
    const int lo_i = local_start(a, i);

    const float *qbase = (const float *)a.q + bb * a.qs[0] + h * a.qs[2];
    const float *kbase = (const float *)a.k + bb * a.ks[0] + g * a.ks[2];
    const float *vbase = (const float *)a.v + bb * a.vs[0] + g * a.vs[2];

    float qf[NQ];
    {
        const float *qrow = qbase + (int64_t)i * a.qs[1] + hi;
#pragma unroll
        for (int ks = 0; ks < NQ; ++ks) qf[ks] = row_ok ? qrow[2 * ks] : 0.f;
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x16 oacc[NDB];
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;

    float *slice = slices[wave];
    // Rows j0 .. j0 + 31 of K and V in registers: load n covers row
    // (lane + 64 n) / (D / 4), 16 bytes; rows past the range end are zero
    // and never read from memory.
    f32x4 kreg[NLK], vreg[NLV];
    auto load_rows = [&](const Sub &st) __attribute__((always_inline)) {
#pragma unroll
        for (int n = 0; n < NLK; ++n) {
            const int c = lane + 64 * n, row = c / (DQK / 4), col = c % (DQK / 4);
            const int j = st.j0 + row;
            kreg[n] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (j < st.re) kreg[n] = *(const f32x4 *)(kbase + (int64_t)j * a.ks[1] + col * 4);
        }
#pragma unroll
        for (int n = 0; n < NLV; ++n) {
            const int c = lane + 64 * n, row = c / (DV / 4), col = c % (DV / 4);
            const int j = st.j0 + row;
            vreg[n] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (j < st.re) vreg[n] = *(const f32x4 *)(vbase + (int64_t)j * a.vs[1] + col * 4);
        }
    };
    auto store_rows = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int n = 0; n < NLK; ++n) {
            const int c = lane + 64 * n, row = c / (DQK / 4), col = c % (DQK / 4);
            *(f32x4 *)(slice + row * KSTR + col * 4) = kreg[n];
        }
#pragma unroll
        for (int n = 0; n < NLV; ++n) {
            const int c = lane + 64 * n, row = c / (DV / 4), col = c % (DV / 4);
            *(f32x4 *)(slice + VOFF + row * VSTR + col * 4) = vreg[n];
        }
    };

    if (wave < n_total) load_rows(sub_at(wave));
    for (int t = wave; t < n_total; t += NW) {
        const Sub st = sub_at(t);
        store_rows();
        if (t + NW < n_total) load_rows(sub_at(t + NW));  // in flight during this sub-tile
        f32x16 sacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
        const float *krow = slice + l32 * KSTR;
#pragma unroll
        for (int ks = 0; ks < NQ; ++ks)
            sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[2 * ks + hi], qf[ks], sacc, 0, 0, 0);
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float x = sacc[r] * a.scale_log2;
            if (st.need_mask) {
                const int j = st.j0 + 8 * (r >> 2) + 4 * hi + (r & 3);
                const bool ok = (j < st.re) & (j <= i) & ((j < tr.sb) | (j >= lo_i));
                x = ok ? x : -INFINITY;
            }
            sacc[r] = x;
            mx = fmaxf(mx, x);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float rs = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(sacc[r] - m_use);
            sacc[r] = p;
            rs += p;
        }
        l_run = l_run * alpha + rs;
        m_run = m_new;
#pragma unroll
        for (int d = 0; d < NDB; ++d)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = 8 * (r >> 2) + 4 * hi + (r & 3);
#pragma unroll
            for (int d = 0; d < NDB; ++d)
                oacc[d] = __builtin_amdgcn_mfma_f32_32x32x2f32(slice[VOFF + key * VSTR + d * 32 + l32], sacc[r],
                                                               oacc[d], 0, 0, 0);
        }
        // The next sub-tile's rows overwrite this slice only after these
        // reads (LDS operations of a wave complete in order; the compiler
        // keeps the order of accesses to one array).
        wait_lgkmcnt0();
        asm volatile("" ::: "memory");
    }

    // Merge. Each wave leaves its unnormalised O (row l32, column c at
    // slice[l32 * OSTR + c]) and its row max and sum; wave 0 combines them.
    const float l_tot = l_run + __shfl_xor(l_run, 32);
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) slice[l32 * OSTR + d * 32 + 8 * (r >> 2) + 4 * hi + (r & 3)] = oacc[d][r];
    if (hi == 0) {
        slice[kF32Rows * OSTR + l32] = m_run;
        slice[kF32Rows * OSTR + kF32Rows + l32] = l_tot;
    }
    __syncthreads();
    if (wave != 0) return;
    float mw[NW], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        mw[w] = slices[w][kF32Rows * OSTR + l32];
        M = fmaxf(M, mw[w]);
    }
    const float M_use = M == -INFINITY ? 0.f : M;
    float ew[NW], L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        ew[w] = fast_exp2(mw[w] - M_use);
        L += ew[w] * slices[w][kF32Rows * OSTR + kF32Rows + l32];
    }
    if (!row_ok) return;
    const float inv = 1.f / L;
    float *orow = (float *)a.o + bb * a.os[0] + (int64_t)i * a.os[1] + h * a.os[2];
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            const int col = d * 32 + 8 * rq + 4 * hi;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < NW; ++w)
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] += ew[w] * slices[w][l32 * OSTR + col + e];
            *(f32x4 *)(orow + col) = v * inv;
        }
    if (a.lse && hi == 0) a.lse[((int64_t)bb * a.Hq + h) * a.N + i] = (M + log2f(L)) * kLn2;
}

template <typename K>
hipError_t launch(K kernel, const PrefillArgs &a, hipStream_t stream) {
    void *args[] = {(void *)&a};
    return hipLaunchKernel((const void *)kernel, dim3(a.total_wgs), dim3(kThreads), args, 0, stream);
}

}  // namespace

bool prefill_supported(bool bf16, int d_qk, int d_v) {
    if (bf16) return (d_qk == 64 && d_v == 64) || (d_qk == 128 && d_v == 128) || (d_qk == 192 && d_v == 128);
    return (d_qk == 64 && d_v == 64) || (d_qk == 128 && d_v == 128);
}

hipError_t launch_prefill(bool bf16, int d_qk, int d_v, const PrefillArgs &a, hipStream_t stream) {
    if (bf16) {
        if (d_qk == 64 && d_v == 64) return launch(ssa_prefill_bf16<64, 64, kModePlain>, a, stream);
        if (d_qk == 128 && d_v == 128) return launch(ssa_prefill_bf16<128, 128, kModePlain>, a, stream);
        if (d_qk == 192 && d_v == 128) return launch(ssa_prefill_bf16<192, 128, kModePlain>, a, stream);
    } else {
        // 32-row tiles (see ssa_prefill_f32).
        PrefillArgs f = a;
        f.num_qtiles = (a.N + kF32Rows - 1) / kF32Rows;
        const int64_t wgs = (int64_t)f.num_qtiles * a.Hq * a.B;
        if (wgs > 0x7fffffff) return hipErrorInvalidValue;
        f.total_wgs = (int32_t)wgs;
        void *args[] = {(void *)&f};
        if (d_qk == 64 && d_v == 64)
            return hipLaunchKernel((const void *)ssa_prefill_f32<64, 64>, dim3(f.total_wgs),
                                   dim3(64 * f32_waves<64, 64>()), args, 0, stream);
        if (d_qk == 128 && d_v == 128)
            return hipLaunchKernel((const void *)ssa_prefill_f32<128, 128>, dim3(f.total_wgs),
                                   dim3(64 * f32_waves<128, 128>()), args, 0, stream);
    }
    return hipErrorInvalidValue;
}

bool prefill_dual_supported(bool bf16, int d_qk, int d_v) { return bf16 && prefill_supported(true, d_qk, d_v); }

hipError_t launch_prefill_dual(bool bf16, int d_qk, int d_v, const PrefillArgs &a, hipStream_t stream) {
    if (bf16) {
        if (d_qk == 64 && d_v == 64) return launch(ssa_prefill_bf16<64, 64, kModeDual>, a, stream);
        if (d_qk == 128 && d_v == 128) return launch(ssa_prefill_bf16<128, 128, kModeDual>, a, stream);
        if (d_qk == 192 && d_v == 128) return launch(ssa_prefill_bf16<192, 128, kModeDual>, a, stream);
    }
    return hipErrorInvalidValue;
}

bool prefill_paged_supported(bool bf16, int d_qk, int d_v) { return bf16 && prefill_supported(true, d_qk, d_v); }

hipError_t launch_prefill_paged(bool bf16, int d_qk, int d_v, const PrefillArgs &a, hipStream_t stream) {
    if (bf16) {
        if (d_qk == 64 && d_v == 64) return launch(ssa_prefill_bf16<64, 64, kModePaged>, a, stream);
        if (d_qk == 128 && d_v == 128) return launch(ssa_prefill_bf16<128, 128, kModePaged>, a, stream);
        if (d_qk == 192 && d_v == 128) return launch(ssa_prefill_bf16<192, 128, kModePaged>, a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace ssa
