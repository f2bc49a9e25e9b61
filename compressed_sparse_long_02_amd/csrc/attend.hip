// attend.hip -- shared-KV multi-query attention over {compressed entries} U
// {sliding window}, for both branches of the hybrid layer.
//
// Method: x-techcon article on DeepSeek-V4, section 2: CSA step 3 -- the 128 most
// recent uncompressed tokens are attended together with the selected compressed
// entries; HCA subsection -- after 128:1 compression, dense attention over all
// entries plus the same window; both use shared-KV multi-query attention.  Stored
// rows follow the mixed-precision KV layout of the same article (bf16 RoPE dims,
// fp8 for the rest).  Readings: one joint softmax over the union; key = value =
// the stored row; logits = scale * q.v.
//
// Design (gfx950): a block owns one query token x 64 heads x one split of the
// attended row list (CSA: the selected indices then the window; HCA: entries
// 0..n(t)-1 then the window); the splits of one query run on one XCD.  Rows are
// gathered 32 at a time into registers ahead of the compute, then converted once
// into a bank-skewed bf16 LDS tile (fp8 -> bf16 with the hardware OCP conversion).
//  * bf16 / packed rows (k_attend_mq, 8 waves): wave w takes 16 heads and half of
//    the head dim; S^T = K.Q^T with 16x16x32 bf16 MFMA (Q in registers, K fragments
//    from LDS), the two halves added through LDS; a softmax with a fixed reference
//    per head (no rescaling, a second pass only if a logit outruns it); P stays in
//    registers as a bf16 hi + lo pair and O^T += V^T.P^T reads V^T from the same
//    row-major tile by the gfx950 LDS transpose read.
//  * fp32 rows (k_attend, 4 waves of 16 heads): 16x16x4 f32 MFMA, an online
//    softmax with a lazy rescale, P staged through LDS.
// Splits write (o, lse) partials that k_attend_combine merges in a fixed order
// (deterministic, no atomics).  The split's o is normalised (a weighted mean of value
// rows); for a bf16 output the packed-row kernel stores it as fp16 scaled by
// ATT_PART_SCALE (half the bytes written and read back; relative error 2^-12, eight
// times below the bf16 output's own rounding); an fp32 output, and the other kernels,
// keep fp32 partials.
#include <type_traits>

#include "compress_dec.h"
#include "device.h"
#include "launch.h"

namespace csl {

constexpr int ATT_NT = 256;
constexpr int MQ_NT = 512;   // threads of the bf16 / packed-row attention kernel (8 waves)
constexpr int ATT_TILE = 32;

__device__ __forceinline__ int64_t att_n_visible(int64_t t, int m, int64_t n_cap) {
    if (t < 0) return 0;
    const int64_t n = (t + 1) / m;
    return n < n_cap ? n : n_cap;
}

// Stored row of compressed entry s (0 <= s < n_cap) of sequence b: dense rows per
// sequence, or, with a block table, row s % epb of physical block bt[b][s / epb] (a
// block id outside [0, n_blocks) is an absent block: nullptr, the row is skipped).
__device__ __forceinline__ const uint8_t* att_entry_row(const AttendArgs& a, int b, int64_t s, int64_t rb) {
    if (!a.bt) return a.kvc + (int64_t)b * a.kvc_bstride + s * rb;
    const uint32_t su = (uint32_t)s, ep = (uint32_t)a.epb;
    const uint32_t lb = su / ep;
    const int32_t blk = a.bt[(int64_t)b * a.bt_stride + lb];
    if (blk < 0 || blk >= a.n_blocks) return nullptr;
    return a.kvc + (int64_t)blk * a.blk_bytes + (int64_t)(su - lb * ep) * rb;
}

// Final normalisation of a query's (unsplit) softmax, base 2: the accumulated rows give
// lse2 = m_ref + log2(l); a sink logit s (natural units) joins the denominator.
// Returns the factor that turns the accumulated output into the result, and the lse
// (natural log).  Without a sink the factor is 1/l, as before.
__device__ __forceinline__ void att_finish(float m_ref, float l, const float* sink, int h, float& inv, float& lse) {
    if (!sink) {
        inv = l > 0.f ? 1.f / l : 0.f;
        lse = l > 0.f ? (m_ref + log2f(l)) * CSL_LN2 : -INFINITY;
        return;
    }
    const float s2 = sink[h] * CSL_LOG2E;
    const float L2 = l > 0.f ? m_ref + log2f(l) : -INFINITY;
    const float T = fmaxf(L2, s2);
    const float lse2 = T + log2f(exp2f(L2 - T) + exp2f(s2 - T));
    inv = l > 0.f ? exp2f(m_ref - lse2) : 0.f;
    lse = lse2 * CSL_LN2;
}

constexpr int ATT_MAX_SIDX = 1536;   // CSA split lengths are capped to this (host plan)

constexpr float ATT_TAU = 8.0f;   // lazy rescale: keep the reference max until it trails by 2^8
constexpr float ATT_HEADROOM = 64.0f;   // largest x - m_ref (base 2) accepted without a rescale
constexpr float ATT_REF_LIFT = 32.0f;   // m_ref starts this far above the first tile's largest logit
// fp16 split partials hold o * 2^-8: magnitudes up to 65504 * 2^8 stay finite, and below
// 2^-6 (fp16 subnormals after the scale) the absolute error stays under 2^-17
constexpr float ATT_PART_SCALE = 1.0f / 256.0f;

// ---------------------------------------------------------------------------
// fp32 rows (the fp32 parity configuration): 4 waves of 16 heads, 16x16x4 f32 MFMA, an
// online softmax with a lazy rescale.  bf16 and packed rows go to k_attend_mq.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(ATT_NT, 2) k_attend(AttendArgs a) {
    constexpr int KSTR = D + 4;                          // floats per K-tile row (bank padding)
    constexpr int CPR = D / 4;                           // 16-byte chunks per row
    constexpr int NCH = ATT_TILE * CPR;
    constexpr int NJ = (NCH + ATT_NT - 1) / ATT_NT;      // chunks per thread per tile
    __shared__ __attribute__((aligned(16))) float kl[ATT_TILE * KSTR];
    __shared__ const uint8_t* rowptr[2 * ATT_TILE];
    __shared__ uint32_t rowmask[2];
    __shared__ int sidx[ATT_MAX_SIDX];
    constexpr int64_t rb = 4 * (int64_t)D;

    const int sp = blockIdx.x, hb = blockIdx.y;
    const int64_t bq = blockIdx.z;
    const int b = (int)(bq / a.Tq);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, col = lane & 15;
    const int64_t t = a.q_pos[bq];
    const int64_t n_ent = a.idx ? (int64_t)a.k : att_n_visible(t, a.m, a.n_cap);
    const int64_t n_win = (t >= 0 && a.W > 0) ? (t + 1 < a.W ? t + 1 : a.W) : 0;
    const int64_t w0 = t - n_win + 1;
    const int64_t L_all = n_ent + n_win;
    const int64_t v_begin = (int64_t)sp * a.rps;
    int64_t v_end = v_begin + a.rps;
    if (v_end > L_all) v_end = L_all;
    const int ntiles = v_end > v_begin ? (int)((v_end - v_begin + ATT_TILE - 1) / ATT_TILE) : 0;

    // ---- the split's slice of the index list, staged once (CSA)
    if (a.idx) {
        const int64_t e_end = v_end < n_ent ? v_end : n_ent;
        for (int64_t v = v_begin + tid; v < e_end; v += ATT_NT) sidx[v - v_begin] = a.idx[bq * a.k + v];
    }

    // ---- Q fragments (B operand of S^T = K Q^T): head h = hb*64 + wv*16 + col
    const int h_a = hb * 64 + wv * 16 + col;
    constexpr int QKS = D / 4;
    float qf[QKS];
    {
        const float* qrow = (const float*)a.q + (bq * a.H + h_a) * D;
#pragma unroll
        for (int ks = 0; ks < QKS; ++ks) qf[ks] = h_a < a.H ? qrow[4 * ks + g] : 0.f;
    }
    __syncthreads();

    // rows of tile `it` -> rowptr slot it&1 and the validity mask (wave 0, lanes 0..31)
    auto resolve = [&](int it) {
        if (tid < 64) {
            const uint8_t* p = nullptr;
            if (tid < ATT_TILE) {
                const int64_t v = v_begin + (int64_t)it * ATT_TILE + tid;
                if (v < v_end) {
                    if (v < n_ent) {
                        const int64_t s = a.idx ? (int64_t)sidx[v - v_begin] : v;
                        if (s >= 0 && s < a.n_cap) p = att_entry_row(a, b, s, rb);
                    } else {
                        const int64_t pos = w0 + (v - n_ent);
                        int64_t slot = (pos - a.kvw_pos0) % a.kvw_rows;
                        if (slot < 0) slot += a.kvw_rows;
                        p = a.kvw + (int64_t)b * a.kvw_bstride + slot * rb;
                    }
                }
                rowptr[(it & 1) * ATT_TILE + tid] = p;
            }
            const uint64_t m = __ballot(p != nullptr);
            if (tid == 0) rowmask[it & 1] = (uint32_t)m;
        }
    };
    // Register prefetch of a tile: thread `tid` owns chunks c = tid + ATT_NT*j of the
    // tile (row c / CPR, 16-byte piece c % CPR), the same for every tile.  The loads
    // of tile it+1 are issued right after tile it reaches LDS and are consumed at the
    // top of the next iteration, so a whole tile of MFMA work hides their latency.
    // Every load is issued (an empty row re-reads the query row and is zeroed), which
    // keeps the load stream branch-free.
    u32x4 R[NJ];
    uint32_t okm = 0;
    auto load_regs = [&](int it) {
        const uint8_t** rp = rowptr + (it & 1) * ATT_TILE;
        okm = 0;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int c = tid + ATT_NT * j;
            const int rr = c / CPR;
            const uint8_t* p = c < NCH ? rp[rr] : nullptr;
            const bool okc = p != nullptr;
            R[j] = ld_global<u32x4>(okc ? p + 16 * (c - rr * CPR) : a.q);
            okm |= okc ? 1u << j : 0u;
        }
    };

    constexpr int NDB = D / 16;
    v4f o[NDB];          // O^T: lane holds dims 16*db + 4g + i of head col
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = v4f{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const float sl2 = a.scale * CSL_LOG2E;

    if (ntiles > 0) {
        resolve(0);
        __syncthreads();
        load_regs(0);
    }
    for (int it = 0; it < ntiles; ++it) {
        lds_barrier();                                  // the previous tile's K/V reads are done
        // ---- the prefetched chunks -> the padded K tile
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int c = tid + ATT_NT * j;
            if (c >= NCH) continue;
            const int rr = c / CPR, pc = c - rr * CPR;
            const u32x4 v = ((okm >> j) & 1u) ? R[j] : u32x4{0, 0, 0, 0};
            *(u32x4*)(kl + (size_t)rr * KSTR + 4 * pc) = v;
        }
        if (it + 1 < ntiles) resolve(it + 1);
        lds_barrier();                                  // K tile and the next rows' pointers visible
        if (it + 1 < ntiles) load_regs(it + 1);         // in flight during the MFMA work below
        const uint32_t rmask = rowmask[it & 1];
        // ---- S^T = K Q^T: rows 16*r2 + 4g + i of head col, two independent MFMA chains
        v4f s[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
        {
            const float* k0 = kl + (size_t)col * KSTR + g;
            const float* k1 = k0 + 16 * KSTR;
#pragma unroll
            for (int ks = 0; ks < QKS; ++ks) {
                s[0] = mfma_f32(k0[4 * ks], qf[ks], s[0]);
                s[1] = mfma_f32(k1[4 * ks], qf[ks], s[1]);
            }
        }
        // ---- online softmax (base 2) for head col over this tile's 32 rows, lazy rescale
        float x[2][4];
        float mx = -INFINITY;
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool okr = (rmask >> (16 * r2 + 4 * g + i)) & 1u;
                x[r2][i] = okr ? s[r2][i] * sl2 : -INFINITY;
                mx = fmaxf(mx, x[r2][i]);
            }
        mx = cross4_max(mx);
        float corr = 1.f;
        const bool need = mx > m_run + ATT_TAU;             // the reference max moves up
        if (need) {
            corr = exp2f(m_run - mx);                        // 0 on the first valid tile
            m_run = mx;
        }
        float rs = 0.f;
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[r2][i] = m_run == -INFINITY ? 0.f : exp2f(x[r2][i] - m_run);
                rs += x[r2][i];
            }
        l_run = l_run * corr + cross4_sum(rs);
        if (__builtin_amdgcn_read_exec() & __ballot(need)) {   // wave-uniform: some head rescaled
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[db][i] *= corr;
        }
        // ---- O^T += V^T P^T: P^T (rows x heads) is the S^T accumulator layout, so the
        //      probabilities never leave registers
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float* vr = kl + (size_t)(16 * r2 + 4 * g + i) * KSTR + col;
#pragma unroll
                for (int db = 0; db < NDB; ++db) o[db] = mfma_f32(vr[16 * db], x[r2][i], o[db]);
            }
        // the next iteration starts with a barrier before the K tile is rewritten
    }

    // ---- finish: normalise, write output or the split's partial
    const int hh = wv * 16 + col;                  // head within the block
    const int h = hb * 64 + hh;
    float inv, lse;
    if (a.nsplit == 1) {
        att_finish(m_run, l_run, h < a.H ? a.sink : nullptr, h, inv, lse);
    } else {                                        // a split's partial: no sink (the combine adds it)
        inv = l_run > 0.f ? 1.f / l_run : 0.f;
        lse = l_run > 0.f ? (m_run + log2f(l_run)) * CSL_LN2 : -INFINITY;
    }
    if (a.nsplit == 1) {
        if (h < a.H) {
            if (a.out_fmt == F32) {
                float* orow = (float*)a.out + (bq * a.H + h) * D + 4 * g;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    *(float4*)(orow + 16 * db) = make_float4(o[db][0] * inv, o[db][1] * inv, o[db][2] * inv, o[db][3] * inv);
            } else {
                uint16_t* orow = (uint16_t*)a.out + (bq * a.H + h) * D + 4 * g;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    *(u32x2*)(orow + 16 * db) = u32x2{f32_to_bf16_rne(o[db][0] * inv) | (f32_to_bf16_rne(o[db][1] * inv) << 16),
                                                      f32_to_bf16_rne(o[db][2] * inv) | (f32_to_bf16_rne(o[db][3] * inv) << 16)};
            }
            if (a.lse && g == 0) a.lse[bq * a.H + h] = lse;
        }
    } else {
        const int64_t prow = ((bq * a.nhb + hb) * a.nsplit + sp) * 64 + hh;
        float* orow = a.ws_o + prow * D + 4 * g;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            *(float4*)(orow + 16 * db) = make_float4(o[db][0] * inv, o[db][1] * inv, o[db][2] * inv, o[db][3] * inv);
        if (g == 0) a.ws_lse[prow] = lse;
    }
}

// ---------------------------------------------------------------------------
// bf16 / packed rows: register-blocked kernel.  A block (8 waves, two per SIMD) owns
// one query x 64 heads x one split of the attended rows.  Wave w covers the 16 heads
// 16*(w&3) .. +15 and the half w>>2 of the head dim.  Rows are gathered 32 at a time
// into registers two tiles ahead and converted once into a bank-skewed bf16 LDS tile
// (double-buffered); Q (16 heads x d/2, bf16) and O^T (16 heads x d/2, fp32) stay in
// registers.
//   S^T = K Q^T : 16x16x32 bf16 over the wave's d/2 dims (A = K rows from LDS,
//   B = Q from registers); the two halves are added through LDS, in the same
//   order by both waves, so they hold bit-identical scores and softmax state.
//   O^T += V^T P^T : 16x16x32 bf16 over the 32 rows of the tile; lane slot j < 4
//   is row 4g + j and slot 4 + j is row 16 + 4g + j, which is how the S^T
//   accumulators sit in the lane, so P never leaves registers; V^T comes from two
//   LDS transpose reads (rows 4g.. and 16 + 4g..).
// ---------------------------------------------------------------------------
// Tile rows in LDS: a stride of D + 128 bf16 (a multiple of the 256-byte bank width
// for D % 128 == 0) and row r shifted by mq_skew(r) = 16 bytes x f(r), f(r) a
// bijection of r mod 16 (r mod 8 -> even steps, the next bit -> odd).  The 16 rows a
// 16-byte K-fragment read touches then start on 16 different bank groups, and so do
// the 8 rows x 32 bytes of each half of a transposed V^T read.
__device__ __forceinline__ int mq_skew(int row) { return 8 * (((row & 7) << 1) | ((row >> 3) & 1)); }

template <int D, int FMT>
struct MqLds {
    static constexpr int KSTR = D + 128;                         // bf16 per K-tile row (with the skew room)
    static constexpr int TILE_ELEMS = ATT_TILE * KSTR;
    // 16-byte chunks per thread and tile: bf16 chunks (RoPE dims, or every dim of a
    // bf16 row) and fp8 chunks (the other dims of a packed row, r <= D/4)
    static constexpr int JB = FMT == BF16 ? (ATT_TILE * D / 8 + MQ_NT - 1) / MQ_NT : (ATT_TILE * D / 4 / 8 + MQ_NT - 1) / MQ_NT;
    static constexpr int J8 = FMT == BF16 ? 0 : (ATT_TILE * D / 16 + MQ_NT - 1) / MQ_NT;
};

template <int D, int FMT>
__global__ void __launch_bounds__(MQ_NT, 2) k_attend_mq(AttendArgs a) {
    using L = MqLds<D, FMT>;
    constexpr int KSTR = L::KSTR;
    constexpr int QH = D / 64;                          // k-steps of 32 dims per half
    constexpr int NDH = D / 32;                         // 16-dim output blocks per half
    constexpr int JB = L::JB, J8 = L::J8, NJ = JB + J8;
    constexpr int PF = 2;                               // tiles whose rows are in flight
    constexpr int RCH = 8;                              // tiles whose rows one resolve pass covers
    static_assert(RCH >= PF + 1, "a chunk's table is rewritten only after its last tile is done");
    __shared__ __attribute__((aligned(16))) uint16_t kl_s[2][L::TILE_ELEMS];   // tiles it&1
    __shared__ __attribute__((aligned(16))) v4f sx[MQ_NT / 64 * 2 * 64];   // [wave][r2][lane]
    __shared__ const uint8_t* rowptr[2][RCH * ATT_TILE];   // tile chunk c in table c & 1
    __shared__ uint32_t rowmask[2][RCH];
    __shared__ int sidx[ATT_MAX_SIDX];
    const int rbf = FMT == BF16 ? D : a.r;              // dims stored as bf16
    const int64_t rb = FMT == BF16 ? 2 * (int64_t)D : 2 * (int64_t)a.r + (D - a.r);

    // the splits of one query run on one XCD: its query rows and, later, the combine's
    // reads of its partials stay in that XCD's L2
    const unsigned lblk = xcd_local_id(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z),
                                       gridDim.x * gridDim.y * gridDim.z);
    const int sp = (int)(lblk % gridDim.x), hb = (int)((lblk / gridDim.x) % gridDim.y);
    const int64_t bq = lblk / (gridDim.x * gridDim.y);
    const int b = (int)(bq / a.Tq);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, col = lane & 15;
    const int hg = wv & 3, dh = wv >> 2;
    // The split's slice of the index list (CSA) first: it depends on nothing but the
    // split (the k selected entries come first in the row list), and global loads
    // complete in issue order, so its LDS staging waits for these loads alone.
    if (a.idx) {
        const int64_t vb = (int64_t)sp * a.rps;
        const int64_t e_end = vb + a.rps < a.k ? vb + a.rps : (int64_t)a.k;
        for (int64_t v = vb + tid; v < e_end; v += MQ_NT) sidx[v - vb] = a.idx[bq * a.k + v];
    }
    // Q fragments (B operands of S^T = K Q^T) of the wave's 16 heads, its half of the
    // dims: they are needed only at the first S^T, so their latency overlaps the chain
    // row indices -> row pointers -> rows
    u32x4 qb[QH];
    {
        const int h = hb * 64 + 16 * hg + col;
        const uint8_t* qrow = a.q + (bq * a.H + (h < a.H ? h : 0)) * (int64_t)D * 2;
#pragma unroll
        for (int ks = 0; ks < QH; ++ks) {
            const u32x4 v = *(const u32x4*)(qrow + (32 * (QH * dh + ks) + 8 * g) * 2);
            qb[ks] = h < a.H ? v : u32x4{0, 0, 0, 0};
        }
    }
    const int64_t t = a.q_pos[bq];
    const int64_t n_ent = a.idx ? (int64_t)a.k : att_n_visible(t, a.m, a.n_cap);
    const int64_t n_win = (t >= 0 && a.W > 0) ? (t + 1 < a.W ? t + 1 : a.W) : 0;
    const int64_t w0 = t - n_win + 1;
    const int64_t L_all = n_ent + n_win;
    const int64_t v_begin = (int64_t)sp * a.rps;
    int64_t v_end = v_begin + a.rps;
    if (v_end > L_all) v_end = L_all;
    const int ntiles = v_end > v_begin ? (int)((v_end - v_begin + ATT_TILE - 1) / ATT_TILE) : 0;

    // this thread's chunks of a tile, the same for every tile: j < JB are bf16 chunks
    // (row, 16-byte piece of the first 2*rbf bytes), the others fp8 chunks (row,
    // 16-byte piece of the fp8 part); -1 when beyond the tile
    int crow[NJ], cpc[NJ];
    {
        const int nbc = rbf / 8, n8c = (D - rbf) / 16;   // chunks per row of each kind
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const bool bf = j < JB;
            const int c = tid + MQ_NT * (bf ? j : j - JB);
            const int per = bf ? nbc : n8c;
            crow[j] = (per > 0 && c < ATT_TILE * per) ? c / per : -1;
            cpc[j] = per > 0 ? c - (c / per) * per : 0;
        }
    }
    lds_barrier();                                      // the index slice in LDS (not the Q loads)

    // Row pointers and validity masks of the RCH tiles of chunk c -> table c & 1, one
    // row per thread (waves 0..3), once per RCH tiles rather than by one wave on every
    // tile's critical path.  An empty row points at the query row (an in-bounds dummy
    // read; its chunks are zeroed when the tile is written).
    auto resolve_chunk = [&](int c) {
        for (int rr = tid; rr < RCH * ATT_TILE; rr += MQ_NT) {
            const uint8_t* p = nullptr;
            {
                const int64_t v = v_begin + (int64_t)(c * RCH) * ATT_TILE + rr;
                if (v < v_end) {
                    if (v < n_ent) {
                        const int64_t s = a.idx ? (int64_t)sidx[v - v_begin] : v;
                        if (s >= 0 && s < a.n_cap) p = att_entry_row(a, b, s, rb);
                    } else {
                        const int64_t pos = w0 + (v - n_ent);
                        int64_t slot = (pos - a.kvw_pos0) % a.kvw_rows;
                        if (slot < 0) slot += a.kvw_rows;
                        p = a.kvw + (int64_t)b * a.kvw_bstride + slot * rb;
                    }
                }
                rowptr[c & 1][rr] = p ? p : a.q;
            }
            const uint64_t m = __ballot(p != nullptr);       // lanes 0..31: one tile, 32..63: the next
            if ((rr & (ATT_TILE - 1)) == 0) rowmask[c & 1][rr / ATT_TILE] = (uint32_t)(m >> (lane & 32));
        }
    };
    // Register prefetch, PF tiles deep.  Every load is issued (an empty row re-reads
    // the query row; its chunks are zeroed when the tile is written to LDS), which
    // keeps the load stream branch-free.
    auto load_regs = [&](int it, u32x4 (&Rb)[NJ]) {
        const uint8_t** rp = rowptr[(it / RCH) & 1] + (it % RCH) * ATT_TILE;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const uint8_t* p = crow[j] >= 0 ? rp[crow[j]] : nullptr;
            const int off = j < JB ? 16 * cpc[j] : 2 * rbf + 16 * cpc[j];
            Rb[j] = ld_global<u32x4>(p ? p + off : a.q);
        }
    };

    // Softmax with a fixed reference per head: m_ref = ATT_REF_LIFT above the largest
    // logit (base 2) of the first tile that has a valid row; every probability is
    // exp2(x - m_ref) and is never rescaled, so the O^T accumulators stay in place.
    // fp32 / bf16 hold x - m_ref <= ATT_HEADROOM with room to spare; if a later logit
    // goes beyond, the block recomputes its split once with m_ref = the largest logit.
    v4f o[NDH];
    float m_ref, l_lane, m_seen = -INFINITY;
    const float sl2 = a.scale * CSL_LOG2E;
    v4f* sx_mine = sx + wv * 128 + lane;
    const v4f* sx_part = sx + (wv ^ 4) * 128 + lane;
    u32x4 R0[NJ], R1[NJ];
    bool ovf = false;

    // tile `it`: its prefetched rows (Rb) -> LDS buffer it&1 (fp8 -> bf16), invalid
    // rows zeroed
    auto write_tile = [&](int it, const u32x4 (&Rb)[NJ]) {
        uint8_t* kl = (uint8_t*)kl_s[it & 1];
        const uint32_t rmask = __builtin_amdgcn_readfirstlane(rowmask[(it / RCH) & 1][it % RCH]);   // block-uniform
        const bool full = rmask == 0xffffffffu;         // wave-uniform
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if (crow[j] < 0) continue;
            u32x4 v = Rb[j];
            if (!full && !((rmask >> crow[j]) & 1u)) v = u32x4{0, 0, 0, 0};
            uint8_t* rowp = kl + (size_t)(crow[j] * KSTR + mq_skew(crow[j])) * 2;
            if (j < JB) {
                *(u32x4*)(rowp + 16 * cpc[j]) = v;
            } else {
                u32x4 lo, hi;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    lo[2 * e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[e], 1.0f, false));
                    lo[2 * e + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[e], 1.0f, true));
                    hi[2 * e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[e + 2], 1.0f, false));
                    hi[2 * e + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[e + 2], 1.0f, true));
                }
                uint8_t* dst = rowp + (rbf + 16 * cpc[j]) * 2;
                *(u32x4*)dst = lo;
                *(u32x4*)(dst + 16) = hi;
            }
        }
    };

    // one tile (it, in LDS buffer it&1): S^T; after the exchange barrier, tile it+1
    // goes from Rnext into the other buffer (its last readers, tile it-1's P.V, are
    // past that barrier) while the probabilities and O^T of tile it are computed; the
    // closing barrier publishes tile it+1, and Rnext is refilled with tile it+1+PF
    auto tile = [&](int it, u32x4 (&Rnext)[NJ]) {
        const uint32_t rmask = __builtin_amdgcn_readfirstlane(rowmask[(it / RCH) & 1][it % RCH]);   // block-uniform
        const bool full = rmask == 0xffffffffu;         // wave-uniform
        const uint16_t* kt = kl_s[it & 1];
        // ---- partial S^T over this wave's half of the dims: s[r2] (rows 16*r2 + 4g + i)
        v4f s[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
        const uint16_t* k0 = kt + (size_t)(col * KSTR + mq_skew(col)) + 32 * QH * dh + 8 * g;
        const uint16_t* k1 = k0 + 16 * KSTR;
#pragma unroll
        for (int ks = 0; ks < QH; ++ks) {
            s[0] = mfma_bf16(*(const u32x4*)(k0 + 32 * ks), qb[ks], s[0]);
            s[1] = mfma_bf16(*(const u32x4*)(k1 + 32 * ks), qb[ks], s[1]);
        }
        sx_mine[0] = s[0];
        sx_mine[64] = s[1];
        lds_barrier();                                  // both halves of S^T visible; tile it-1 done
        if (it + 1 < ntiles) {
            write_tile(it + 1, Rnext);
        }
        // the next chunk's rows, in time for the load of its first tile after this tile
        if (it + 1 + PF < ntiles && (it + 1 + PF) % RCH == 0) resolve_chunk((it + 1 + PF) / RCH);
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
            const v4f p = sx_part[64 * r2];
            s[r2] = dh == 0 ? s[r2] + p : p + s[r2];    // low half + high half
        }
        // ---- probabilities (lane: head col, rows 16*r2 + 4g + i), as a bf16 pair
        //      hi + lo: P = hi + lo to ~2^-17 relative, so P.V keeps fp32-level accuracy
        //      even where V has large channels
        u32x4 pb, pl;
        {
            float x[2][4];
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
                for (int i = 0; i < 4; ++i) x[r2][i] = s[r2][i] * sl2;
            if (!full) {
#pragma unroll
                for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (!((rmask >> (16 * r2 + 4 * g + i)) & 1u)) x[r2][i] = -INFINITY;
            }
            float mx = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                             fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
            m_seen = fmaxf(m_seen, mx);
            if (__builtin_amdgcn_read_exec() & __ballot(m_ref == -INFINITY)) {   // no reference yet
                const float tmax = cross4_max(mx);
                if (m_ref == -INFINITY && tmax != -INFINITY) m_ref = tmax + ATT_REF_LIFT;
            }
            ovf |= mx > m_ref + ATT_HEADROOM;
            const float mr = m_ref == -INFINITY ? 0.f : m_ref;   // no reference: every x is -inf
            float ls = 0.f;
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[r2][i] = __builtin_amdgcn_exp2f(x[r2][i] - mr);   // 0 for invalid rows
                    ls += x[r2][i];
                }
            l_lane += ls;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a0 = x[e >> 1][2 * (e & 1)], a1 = x[e >> 1][2 * (e & 1) + 1];
                const uint32_t h = pack_bf16x2(a0, a1);
                pb[e] = h;
                pl[e] = pack_bf16x2(a0 - __uint_as_float(h << 16), a1 - __uint_as_float(h & 0xffff0000u));
            }
        }
        // ---- O^T += V^T P^T over this wave's dims (one V^T fragment feeds both head blocks)
        const int vr = 4 * g + (col >> 2);
        const uint16_t* vp0 = kt + (size_t)(vr * KSTR + mq_skew(vr)) + 16 * NDH * dh + 4 * (col & 3);
        const uint16_t* vp1 = vp0 + 16 * KSTR;
#pragma unroll
        for (int db = 0; db < NDH; ++db) {
            const u32x2 t0 = lds_read_tr16(vp0 + 16 * db);
            const u32x2 t1 = lds_read_tr16(vp1 + 16 * db);
            const u32x4 va = {t0[0], t0[1], t1[0], t1[1]};
            o[db] = mfma_bf16(va, pb, o[db]);
            o[db] = mfma_bf16(va, pl, o[db]);
        }
        lds_barrier();                                  // tile it+1 and its row pointers visible, S^T reads done
        if (it + 1 + PF < ntiles) load_regs(it + 1 + PF, Rnext);
    };

    // the first PF tiles' rows in flight, tile 0 first
    auto start_rows = [&]() {
        resolve_chunk(0);
        lds_barrier();
        if (0 < ntiles) load_regs(0, R0);
        if (1 < ntiles) load_regs(1, R1);
    };
    start_rows();

    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int db = 0; db < NDH; ++db) o[db] = v4f{0.f, 0.f, 0.f, 0.f};
        m_ref = pass == 0 ? -INFINITY : cross4_max(m_seen);
        l_lane = 0.f;
        ovf = false;
        if (pass > 0) {
            __syncthreads();                            // slots and tiles of the first pass are free
            start_rows();
        }
        // tile 0 into buffer 0; R0 then refilled with tile PF (its rows are in chunk 0)
        if (0 < ntiles) write_tile(0, R0);
        lds_barrier();
        if (PF < ntiles) load_regs(PF, R0);
        // tile it's successor comes from R[(it+1) % PF]
        for (int it = 0; it < ntiles; it += PF) {
            tile(it, R1);
            if (it + 1 < ntiles) tile(it + 1, R0);
        }
        // the whole block redoes the split only if some wave overflowed
        if (!__syncthreads_or(ovf ? 1 : 0)) break;
    }
    const float l_run = cross4_sum(l_lane), m_run = m_ref;

    // ---- finish: normalise, write the output or the split's partial (this wave's dims)
    {
        const int hh = 16 * hg + col;                   // head within the block
        const int h = hb * 64 + hh;
        float inv, lse;
        if (a.nsplit == 1) {
            att_finish(m_run, l_run, h < a.H ? a.sink : nullptr, h, inv, lse);
        } else {                                    // a split's partial: no sink (the combine adds it)
            inv = l_run > 0.f ? 1.f / l_run : 0.f;
            lse = l_run > 0.f ? (m_run + log2f(l_run)) * CSL_LN2 : -INFINITY;
        }
        const int d0 = 16 * NDH * dh + 4 * g;
        if (a.nsplit == 1) {
            if (h < a.H) {
                if (a.out_fmt == F32) {
                    float* orow = (float*)a.out + (bq * a.H + h) * D + d0;
#pragma unroll
                    for (int db = 0; db < NDH; ++db)
                        *(float4*)(orow + 16 * db) = make_float4(o[db][0] * inv, o[db][1] * inv, o[db][2] * inv,
                                                                 o[db][3] * inv);
                } else {
                    uint16_t* orow = (uint16_t*)a.out + (bq * a.H + h) * D + d0;
#pragma unroll
                    for (int db = 0; db < NDH; ++db)
                        *(u32x2*)(orow + 16 * db) = u32x2{pack_bf16x2(o[db][0] * inv, o[db][1] * inv),
                                                          pack_bf16x2(o[db][2] * inv, o[db][3] * inv)};
                }
                if (a.lse && g == 0 && dh == 0) a.lse[bq * a.H + h] = lse;
            }
        } else {
            const int64_t prow = ((bq * a.nhb + hb) * a.nsplit + sp) * 64 + hh;
            float* orow = a.ws_o + prow * D + d0;
#pragma unroll
            for (int db = 0; db < NDH; ++db)
                *(float4*)(orow + 16 * db) = make_float4(o[db][0] * inv, o[db][1] * inv, o[db][2] * inv, o[db][3] * inv);
            if (g == 0 && dh == 0) a.ws_lse[prow] = lse;
        }
    }
}

// ---------------------------------------------------------------------------
// Packed rows with the 64 bf16 RoPE dims (head dims 256 and 512): rows stay packed in
// LDS.  A block (8 waves, two per SIMD) owns one query x 64 heads x one split, in tiles
// of 32 rows.  Rows stream from HBM straight into LDS as they are stored (16 bytes a
// lane by global_load_lds), so LDS carries 576 instead of 1024 bytes per row and
// reader; MFMA operands are widened in registers (fp8 -> bf16, the hardware OCP
// conversion, exact).
//   The waves form two teams of four; wave w of a team owns the 16 heads 16 (w%4) ..
//   +15 across all dims (O^T, fp32, in registers) and computes its own scores and
//   softmax, so no wave waits for another within a tile.  Team t takes the tiles
//   u = t (mod 2), each over two steps: in step u the S^T = K.Q^T, the probabilities
//   and the first blocks of O^T += V^T.P^T; in step u+1 the other blocks.  The teams
//   are one step apart, so on every SIMD one wave's softmax and conversions run beside
//   the other wave's MFMAs; one barrier per step.
//   S^T: 16x16x32 bf16, A = K rows from LDS, B = Q from LDS.  The two 16-row MFMA blocks
//   take rows 8(x/4) + x%4 (+4), so each lane's eight scores are rows 8g .. 8g+7 of the
//   tile: exactly the k slots of its P^T operand in the 16x16x32 P.V, so P never leaves
//   registers.  V^T: one 8-bit LDS transpose read per 16 dims (fp8), two 16-bit ones
//   for the RoPE dims.
// ---------------------------------------------------------------------------
constexpr int F8_R = 64;           // RoPE dims this kernel takes (the pages' packed layout)
constexpr int F8_T = 32;           // rows of a tile
constexpr int F8_NST = 4;          // LDS stages: two tiles being computed, two in flight
constexpr int F8_RCH = 8;          // tiles whose row pointers one resolve pass covers
constexpr int F8_TNT = MQ_NT / 2;  // threads of a team

// a stored row of 576 (d 512) or 320 (d 256) bytes, zero: the copy source of absent rows
// and of the padding (the conversion of an fp8 NaN pattern would survive P = 0)
__device__ __attribute__((aligned(256))) uint8_t f8_zero_row[1024];

template <int D>
struct F8Lds {
    static constexpr int RB = D + F8_R;                      // bytes of a stored row
    static constexpr int P = RB / 16 + 1;                    // 16-byte slots per LDS row (one pad)
    static constexpr int RS = 16 * P;                        // LDS row stride: an odd number of slots
    // row r at r * RS + 64 * (r / 16): rows 0..15 on 16 different bank groups (P odd),
    // rows 16..31 four groups further, which also keeps the row sets of the K reads
    // ({0-3, 8-11, 16-19, 24-27} and +4) on 16 different groups
    static constexpr int SLOTS = 32 * P + 4;
    static constexpr int STAGE = 16 * SLOTS;                 // bytes of a stage
    // 1 KB copies per tile; the last one ends at the stage's end, overlapping its
    // predecessor with the same bytes
    static constexpr int NSEG = (SLOTS + 63) / 64;
    static constexpr int NI = (NSEG + MQ_NT / 64 - 1) / (MQ_NT / 64);   // copies per wave and tile
    // Q rows: 2 (mod 16) slots of 16 bytes, which the 16-byte Q-fragment reads (16 heads
    // x 4 consecutive slots) take at the full LDS rate on gfx950 (measured; an odd
    // number of slots halves it)
    static constexpr int QSTR = D + 16;                      // bf16 per Q row
    static constexpr int QBYTES = 64 * QSTR * 2;
    static constexpr int QP = QSTR / 8;                      // 16-byte slots per Q row (two pads)
    static constexpr int QSEG = QP;                          // 1 KB copies of Q (64 rows x QP slots)
    static constexpr int NQ = (QSEG + MQ_NT / 64 - 1) / (MQ_NT / 64);   // Q copies per wave
    static constexpr int TOTAL = QBYTES + F8_NST * STAGE;    // Q, stages (reused by the team merge)
    static constexpr int MERGE = 4 * (D / 16) * 64 * 16;     // team 1's O^T, then its softmax states
    static_assert(P % 2 == 1, "row stride must be an odd number of 16-byte slots");
    static_assert(NSEG >= 2, "stage layout");
    static_assert(MERGE + 4 * 2 * 64 * 4 <= TOTAL, "merge space");
    static_assert(F8_RCH >= 3, "a chunk's table is rewritten only after its last tile is done");
    static_assert(D % 128 == 0, "S^T reads its 32-dim steps in groups of four");
};

__device__ __forceinline__ int f8_row_off(int row, int rs) { return row * rs + 64 * (row >> 4); }

// 8 fp8 e4m3fn -> 8 bf16 (exact)
__device__ __forceinline__ u32x4 f8_widen(const u32x2& w) {
    u32x4 o;
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true));
    return o;
}

// LDS transpose read of bytes (gfx950): within each 16-lane group, lane i receives byte
// (i % 8) of the 64-bit chunks read by source lanes 2*j + i/8, j = 0..7.
__device__ __forceinline__ u32x2 lds_read_tr8(const uint8_t* p) {
    typedef int v2i __attribute__((ext_vector_type(2)));
    const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(p));
    return __builtin_bit_cast(u32x2, v);
}

// One wave-wide copy of 16 bytes a lane from global memory (each lane its own source)
// into 1 KB of LDS at lds_base + 16 * lane (global_load_lds_dwordx4; M0 holds the LDS
// base).  Written as asm so that the compiler's wait insertion does not see an LDS
// write it cannot place: it would otherwise wait for every copy in flight before any
// LDS access.  The copy has no result register; the kernel waits for its copies itself
// (vmcnt, then a barrier).  Copies it does not see only make the compiler's own vmcnt
// waits stricter, as vector-memory operations complete in issue order.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // M0 is reserved: the clobber is still honoured
__device__ __forceinline__ void copy16_to_lds(const void* src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds_base)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// PRE = true (one query per sequence): the split whose rows hold the entry the token
// completes first compresses that entry into the cache (every wave a channel part of the
// one-wave compression, its stores complete before the block's first barrier), so the
// copies of its tiles read the new row.  The compression's loads and stores all complete
// before the kernel issues its first tile copy, so they take no place in the kernel's
// counts of copies in flight.
template <int D, bool PRE>
__global__ void __launch_bounds__(MQ_NT) k_attend_f8(AttendArgs a, AttendPre pre) {
    using L = F8Lds<D>;
    constexpr int P = L::P, RS = L::RS, NI = L::NI, NST = F8_NST, RCH = F8_RCH, T = F8_T, R = F8_R;
    constexpr int QK = D / 32;                          // k-steps of S^T (32 dims)
    constexpr int NDB = D / 16;                         // 16-dim output blocks
    constexpr int NA = NDB / 16;                        // output blocks of a tile's first step
    constexpr int RK = R / 32, RV = R / 16;             // k-steps / output blocks over the RoPE dims
    constexpr int RB = L::RB;
    // s_waitcnt vmcnt(n), the other counters untouched (vmcnt in bits 3:0 and 15:14)
    static_assert(NI < 16, "vmcnt range");
    constexpr int WAIT_NEXT = 0x0F70 | NI;              // the copies of the next step's tile have landed
    constexpr int WAIT_ALL = 0x0F70;
    __shared__ __attribute__((aligned(16))) uint8_t lds[L::TOTAL];   // Q [head][dim] bf16, then stages
    __shared__ const uint8_t* rowptr[2][RCH * T];                    // tile chunk c in table c & 1
    __shared__ uint32_t rowmask[2][RCH];
    __shared__ int sidx[ATT_MAX_SIDX];
    const uint16_t* const q_s = (const uint16_t*)lds;
    uint8_t* const stages = lds + L::QBYTES;

    // the splits of one query run on one XCD: its query rows and, later, the combine's
    // reads of its partials stay in that XCD's L2
    const unsigned lblk = xcd_local_id(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z),
                                       gridDim.x * gridDim.y * gridDim.z);
    const int sp = (int)(lblk % gridDim.x), hb = (int)((lblk / gridDim.x) % gridDim.y);
    const int64_t bq = lblk / (gridDim.x * gridDim.y);
    const int b = (int)(bq / a.Tq);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, col = lane & 15;
    const int hg = wv & 3, team = wv >> 2, tt = tid & (F8_TNT - 1);
    // the query's position: a scalar load, issued first, whose wait below does not wait
    // for the LDS-DMA copies of Q
    const int64_t t = ld_uniform<int32_t>(a.q_pos + bq);
    // Q of the block's 64 heads -> LDS by copies (slot k: piece k % QP of head k / QP; the
    // pads and heads past H read the zero row; copies past the last segment repeat it);
    // they complete with the first tile's rows
    {
        const int64_t q0 = (bq * a.H + (int64_t)hb * 64) * D * 2;
#pragma unroll
        for (int i = 0; i < L::NQ; ++i) {
            int seg = wv + (MQ_NT / 64) * i;
            seg = seg < L::QSEG ? seg : L::QSEG - 1;
            const int kq = 64 * seg + lane;
            const int hh = kq / L::QP, pc = kq - hh * L::QP;
            const bool data = pc < D / 8 && hb * 64 + hh < a.H;
            const uint8_t* src = data ? a.q + q0 + ((int64_t)hh * D + 8 * pc) * 2 : f8_zero_row;
            copy16_to_lds(src, __builtin_amdgcn_readfirstlane(lds_addr(lds + 1024 * seg)));
        }
    }
    // the split's slice of the index list (CSA), staged once: the row resolution then
    // makes no global loads inside the tile loop (these loads complete after the Q
    // copies, issued first, so the wait for them overlaps the Q latency)
    if (a.idx) {
        const int64_t vb = (int64_t)sp * a.rps;
        const int64_t e_end = vb + a.rps < a.k ? vb + a.rps : (int64_t)a.k;
        for (int64_t v = vb + tid; v < e_end; v += MQ_NT) sidx[v - vb] = a.idx[bq * a.k + v];
    }
    const int64_t n_ent = a.idx ? (int64_t)a.k : att_n_visible(t, a.m, a.n_cap);
    const int64_t n_win = (t >= 0 && a.W > 0) ? (t + 1 < a.W ? t + 1 : a.W) : 0;
    const int64_t w0 = t - n_win + 1;
    const int64_t L_all = n_ent + n_win;
    const int64_t v_begin = (int64_t)sp * a.rps;
    int64_t v_end = v_begin + a.rps;
    if (v_end > L_all) v_end = L_all;
    const int ntiles = v_end > v_begin ? (int)((v_end - v_begin + T - 1) / T) : 0;

    // Row pointers and validity masks of the RCH tiles of chunk c -> table c & 1, one
    // row per thread of the calling team; an absent row reads the zero row.
    auto resolve_chunk = [&](int c) {
        for (int rr = tt; rr < RCH * T; rr += F8_TNT) {
            const uint8_t* p = nullptr;
            {
                const int64_t v = v_begin + (int64_t)(c * RCH) * T + rr;
                if (v < v_end) {
                    if (v < n_ent) {
                        const int64_t s = a.idx ? (int64_t)sidx[v - v_begin] : v;
                        if (s >= 0 && s < a.n_cap) p = att_entry_row(a, b, s, RB);
                    } else {
                        const int64_t pos = w0 + (v - n_ent);
                        int64_t slot = (pos - a.kvw_pos0) % a.kvw_rows;
                        if (slot < 0) slot += a.kvw_rows;
                        p = a.kvw + (int64_t)b * a.kvw_bstride + slot * RB;
                    }
                }
                rowptr[c & 1][rr] = p ? p : f8_zero_row;
            }
            const uint64_t m = __ballot(p != nullptr);       // lanes 0..31: one tile, 32..63: the next
            if ((rr & (T - 1)) == 0) rowmask[c & 1][rr / T] = (uint32_t)(m >> (lane & 32));
        }
    };
    // Copy i of this wave for tile v -> stage v % NST: the 1 KB segment wv + 8 i (the
    // last segment ends at the stage's end; copies past it repeat it); the lane's
    // 16-byte slot k holds piece k % P of row k / P (rows 0..15), then four gap slots,
    // then rows 16..31 the same way; pads, gaps and absent rows read the zero row.
    // Every wave issues the same number of copies for every tile (the vmcnt waits count
    // them), past the split's rows too.
    auto issue_one = [&](int v, int i) {
        const uint8_t* const* rp = rowptr[(v / RCH) & 1] + (v % RCH) * T;
        uint8_t* st = stages + (v % NST) * L::STAGE;
        const int seg = wv + (MQ_NT / 64) * i;
        const int k0 = seg < L::NSEG - 1 ? 64 * seg : L::SLOTS - 64;
        const int k = k0 + lane;
        const int k2 = k < 16 * P ? k : k - 4;              // slot index with the gap removed
        const int row = k2 / P, pc = k2 - row * P;
        const bool data = (k < 16 * P || k >= 16 * P + 4) && pc < P - 1;
        const uint8_t* src = data ? rp[row] + 16 * pc : f8_zero_row;
        copy16_to_lds(src, __builtin_amdgcn_readfirstlane(lds_addr(st + 16 * k0)));
    };
    auto issue_copies = [&](int v) {
#pragma unroll
        for (int i = 0; i < NI; ++i) issue_one(v, i);
    };

    // Softmax with a fixed reference per head and team: m_ref = ATT_REF_LIFT above the
    // largest logit (base 2) of the team's first tile that has a valid row; every
    // probability is exp2(x - m_ref) and is never rescaled, so the O^T accumulators stay
    // in place.  fp32 / bf16 hold x - m_ref <= ATT_HEADROOM with room to spare; if a
    // later logit goes beyond, the block recomputes its split once with m_ref = the
    // largest logit each wave saw.
    v4f o[NDB];                                         // O^T: dims 16 db + 4g + i, heads 16 hg + col
    float m_ref, l_lane, m_seen = -INFINITY;
    const float sl2 = a.scale * CSL_LOG2E;
    bool ovf = false;
    u32x4 pb, pl;                                       // P^T of the wave's current tile, hi + lo

    // per-lane LDS offsets within a stage
    const int kofs0 = f8_row_off(8 * (col >> 2) + (col & 3), RS);       // S^T block 0: rows 8(x/4) + x%4
    const int kofs1 = f8_row_off(8 * (col >> 2) + 4 + (col & 3), RS);   // block 1: the same + 4
    const int v8ofs = f8_row_off(8 * g + (col >> 1), RS) + R + 8 * (col & 1);
    const int v16ofs0 = f8_row_off(8 * g + (col >> 2), RS) + 8 * (col & 3);
    const int v16ofs1 = f8_row_off(8 * g + 4 + (col >> 2), RS) + 8 * (col & 3);
    const uint16_t* const qp = q_s + (16 * hg + col) * L::QSTR + 8 * g;

    auto pv = [&](const uint8_t* st, int db) {
        u32x4 va;
        if (db < RV) {
            const u32x2 t0 = lds_read_tr16((const uint16_t*)(st + v16ofs0 + 32 * db));
            const u32x2 t1 = lds_read_tr16((const uint16_t*)(st + v16ofs1 + 32 * db));
            va = u32x4{t0[0], t0[1], t1[0], t1[1]};
        } else {
            va = f8_widen(lds_read_tr8(st + v8ofs + 16 * db));   // fp8 dim d at byte R + d
        }
        o[db] = mfma_bf16(va, pb, o[db]);
        o[db] = mfma_bf16(va, pl, o[db]);
    };
    // first step of tile u (stage u % NST): S^T, probabilities, output blocks 0..NA-1;
    // the wave's copies of tile cv are spread over the work (a burst of copies from every
    // wave at once stalls on the memory pipeline)
    auto step_a = [&](int u, int cv) {
        const uint32_t rmask = __builtin_amdgcn_readfirstlane(rowmask[(u / RCH) & 1][u % RCH]);   // block-uniform
        const bool full = rmask == 0xffffffffu;         // wave-uniform
        const uint8_t* st = stages + (u % NST) * L::STAGE;
        v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        // groups of SG k-steps: every fragment of a group is read before the group's
        // conversions and products, so the LDS latency is paid once per group
        constexpr int SG = 4;
#pragma unroll
        for (int k0s = 0; k0s < QK; k0s += SG) {
            if (k0s / SG < NI) issue_one(cv, k0s / SG);
            u32x4 qf[SG], kb0[SG], kb1[SG];
            u32x2 kr0[SG], kr1[SG];
#pragma unroll
            for (int j = 0; j < SG; ++j) {
                const int ks = k0s + j;
                qf[j] = *(const u32x4*)(qp + 32 * ks);
                if (ks < RK) {                          // two 8-byte reads: the row stride suits b64
                    const u32x2 x0 = *(const u32x2*)(st + kofs0 + 2 * (32 * ks + 8 * g));
                    const u32x2 x1 = *(const u32x2*)(st + kofs0 + 2 * (32 * ks + 8 * g) + 8);
                    const u32x2 y0 = *(const u32x2*)(st + kofs1 + 2 * (32 * ks + 8 * g));
                    const u32x2 y1 = *(const u32x2*)(st + kofs1 + 2 * (32 * ks + 8 * g) + 8);
                    kb0[j] = u32x4{x0[0], x0[1], x1[0], x1[1]};
                    kb1[j] = u32x4{y0[0], y0[1], y1[0], y1[1]};
                } else {                                // fp8 dim d at byte R + d
                    kr0[j] = *(const u32x2*)(st + kofs0 + R + 32 * ks + 8 * g);
                    kr1[j] = *(const u32x2*)(st + kofs1 + R + 32 * ks + 8 * g);
                }
            }
#pragma unroll
            for (int j = 0; j < SG; ++j) {
                const int ks = k0s + j;
                const u32x4 k0 = ks < RK ? kb0[j] : f8_widen(kr0[j]);
                const u32x4 k1 = ks < RK ? kb1[j] : f8_widen(kr1[j]);
                s0 = mfma_bf16(k0, qf[j], s0);
                s1 = mfma_bf16(k1, qf[j], s1);
            }
        }
#pragma unroll
        for (int i = QK / SG; i < NI; ++i) issue_one(cv, i);
        // ---- probabilities (lane: head col, rows 8g + j), as a bf16 pair hi + lo:
        //      P = hi + lo to ~2^-17 relative, so P.V keeps fp32-level accuracy even
        //      where V has large channels
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = s0[i] * sl2;
            x[4 + i] = s1[i] * sl2;
        }
        if (!full) {
            const uint32_t mine = rmask >> (8 * g);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (!((mine >> j) & 1u)) x[j] = -INFINITY;
        }
        const float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        m_seen = fmaxf(m_seen, mx);
        if (__builtin_amdgcn_read_exec() & __ballot(m_ref == -INFINITY)) {   // no reference yet
            const float tmax = cross4_max(mx);
            if (m_ref == -INFINITY && tmax != -INFINITY) m_ref = tmax + ATT_REF_LIFT;
        }
        ovf |= mx > m_ref + ATT_HEADROOM;
        const float mr = m_ref == -INFINITY ? 0.f : m_ref;   // no reference: every x is -inf
        float ls = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            x[j] = __builtin_amdgcn_exp2f(x[j] - mr);        // 0 for invalid rows
            ls += x[j];
        }
        l_lane += ls;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a0 = x[2 * e], a1 = x[2 * e + 1];
            const uint32_t h = pack_bf16x2(a0, a1);
            pb[e] = h;
            pl[e] = pack_bf16x2(a0 - __uint_as_float(h << 16), a1 - __uint_as_float(h & 0xffff0000u));
        }
#pragma unroll
        for (int db = 0; db < NA; ++db) pv(st, db);
    };
    // second step of tile u: output blocks NA..NDB-1
    auto step_b = [&](int u, int cv) {
        const uint8_t* st = stages + (u % NST) * L::STAGE;
        constexpr int GAP = (NDB - NA + NI - 1) / NI;   // output blocks between two copies
#pragma unroll
        for (int db = NA; db < NDB; ++db) {
            if ((db - NA) % GAP == 0 && (db - NA) / GAP < NI) issue_one(cv, (db - NA) / GAP);
            pv(st, db);
        }
    };

    if constexpr (PRE) {
        // the entry e this token completes is row e of the list when it is visible
        const int64_t e = (t + 1) / a.m - 1;
        if (t >= 0 && (t + 1) % a.m == 0 && e < a.n_cap && hb == 0 && e / a.rps == sp) {
            for (int z = wv; z < pre.gz; z += MQ_NT / 64) compress_dec_body<KV_PACKED>(pre.kv, 0, b, z, pre.gz);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
    }

    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] = v4f{0.f, 0.f, 0.f, 0.f};
        m_ref = pass == 0 ? -INFINITY : cross4_max(m_seen);
        l_lane = 0.f;
        ovf = false;
        pb = pl = u32x4{0, 0, 0, 0};
        if (pass > 0) __syncthreads();                  // stages and tables of the first pass are free
        // ---- prologue: tiles 0 and 1 in flight, Q (first pass) and tile 0 landed
        lds_barrier();                                  // the index slice in LDS
        if (team == 0) resolve_chunk(0);
        lds_barrier();
        issue_copies(0);
        issue_copies(1);
        __builtin_amdgcn_s_waitcnt(WAIT_NEXT);          // this wave's copies of Q and tile 0
        lds_barrier();
        // ---- step u: team u&1 starts tile u, the other team finishes tile u-1; tile u+2
        //      goes into the stage tile u-2 freed
        for (int u = 0; u <= ntiles; ++u) {
            if (team == (u & 1)) {
                if (u < ntiles)
                    step_a(u, u + 2);
                else
                    issue_copies(u + 2);
            } else {
                if (u > 0)
                    step_b(u - 1, u + 2);
                else
                    issue_copies(u + 2);
                // the row table of the chunk whose first tile is copied two steps on
                if ((u + 3) % RCH == 0) resolve_chunk((u + 3) / RCH);
            }
            __builtin_amdgcn_s_waitcnt(WAIT_NEXT);      // this wave's copies of tile u+1
            lds_barrier();                              // tile u+1 visible, stage of tile u-1 free
        }
        __builtin_amdgcn_s_waitcnt(WAIT_ALL);           // the copies past the split have landed
        // the whole block redoes the split only if some wave overflowed
        if (!__syncthreads_or(ovf ? 1 : 0)) break;
    }

    // ---- merge the teams: team 1 hands (O^T, reference, sum) through LDS to the team-0
    //      wave of the same heads, which normalises and writes the output or the split's
    //      partial, one 16-dim block at a time
    v4f* mo = (v4f*)lds + hg * NDB * 64;                // [hg][NDB][64]
    float* mm = (float*)(lds + L::MERGE) + hg * 128;    // [hg][2][64]: reference, sum
    if (team == 1) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) mo[db * 64 + lane] = o[db];
        mm[lane] = m_ref;
        mm[64 + lane] = l_lane;
    }
    __syncthreads();
    if (team == 1) return;
    const float mB = mm[lane], lB = mm[64 + lane];
    const float M = fmaxf(m_ref, mB);
    const float fA = m_ref == -INFINITY ? 0.f : exp2f(m_ref - M);
    const float fB = mB == -INFINITY ? 0.f : exp2f(mB - M);
    const float l_run = cross4_sum(l_lane * fA + lB * fB);
    const int hh = 16 * hg + col;                       // head within the block
    const int h = hb * 64 + hh;
    float inv, lse;
    if (a.nsplit == 1) {
        att_finish(M, l_run, h < a.H ? a.sink : nullptr, h, inv, lse);
    } else {                                        // a split's partial: no sink (the combine adds it)
        inv = l_run > 0.f ? 1.f / l_run : 0.f;
        lse = l_run > 0.f ? (M + log2f(l_run)) * CSL_LN2 : -INFINITY;
    }
    const float cA = fA * inv, cB = fB * inv;
    const int d0 = 4 * g;
    float* of = nullptr;                                // fp32 output or partial
    uint16_t* ob = nullptr;                             // bf16 output
    uint16_t* op = nullptr;                             // a split's partial in fp16, scaled by ATT_PART_SCALE
    if (a.nsplit > 1) {                                 // fp16 for a bf16 output, else fp32
        const int64_t prow = ((bq * a.nhb + hb) * a.nsplit + sp) * 64 + hh;
        if (a.out_fmt == BF16)
            op = (uint16_t*)a.ws_o + prow * D + d0;
        else
            of = a.ws_o + prow * D + d0;
        if (g == 0) a.ws_lse[prow] = lse;
    } else if (h < a.H) {
        if (a.out_fmt == F32)
            of = (float*)a.out + (bq * a.H + h) * D + d0;
        else
            ob = (uint16_t*)a.out + (bq * a.H + h) * D + d0;
        if (a.lse && g == 0) a.lse[bq * a.H + h] = lse;
    }
    if (!of && !ob && !op) return;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const v4f oB = mo[db * 64 + lane];
        float r[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = o[db][i] * cA + oB[i] * cB;
        if (op)
            *(u32x2*)(op + 16 * db) = u32x2{pack_f16x2(r[0] * ATT_PART_SCALE, r[1] * ATT_PART_SCALE),
                                           pack_f16x2(r[2] * ATT_PART_SCALE, r[3] * ATT_PART_SCALE)};
        else if (of)
            *(float4*)(of + 16 * db) = make_float4(r[0], r[1], r[2], r[3]);
        else
            *(u32x2*)(ob + 16 * db) = u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
    }
}

// Merge of split partials: out = sum_s exp(lse_s - M) o_s / sum_s exp(lse_s - M).
// One block of two waves per (query, head): the 64 heads of a head block spread over 64
// small blocks so that the merge reads its partials with the whole GPU in one round
// (HCA decode at batch 16: 8.1 -> 6.8 us against blocks of 4 heads).  Wave 0 first
// loads the split lse of the head (lane s holds split s), then every thread issues
// the loads of its first CMB_UNR splits; the weights are formed while those are in
// flight (loads complete in issue order, so waiting for the lse does not wait for the
// partials), and the splits are accumulated in split order.
constexpr int CMB_HEADS = 1;
constexpr int CMB_UNR = 16;
constexpr int CMB_NT = 128;

template <int D, bool PH>
__global__ void __launch_bounds__(CMB_NT) k_attend_combine(AttendArgs a) {
    using PT = std::conditional_t<PH, u32x2, float4>;  // four dims of a partial as stored
    extern __shared__ float wts[];   // [CMB_HEADS][nsplit] normalised weights, then lse
    // same XCD assignment of queries as the attention kernel (its partials are in that L2)
    const unsigned lblk = xcd_local_id(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
    const int bx = (int)(lblk % gridDim.x);
    const int hb = bx / (64 / CMB_HEADS);
    const int h0 = (bx % (64 / CMB_HEADS)) * CMB_HEADS;   // first head within the head block
    const int64_t bq = lblk / gridDim.x;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int ns = a.nsplit;
    const int64_t base = (bq * a.nhb + hb) * (int64_t)ns;
    float* lse_o = wts + CMB_HEADS * ns;
    constexpr int C4 = D / 4;
    constexpr int ITEMS = (CMB_HEADS * C4 + CMB_NT - 1) / CMB_NT;   // float4 items per thread
    // ---- the split lse of this wave's head (waves 0..3, lane s: split s), issued before the
    //      partials: loads complete in issue order, so the weights need not wait for them
    const int hw = h0 + (wv < CMB_HEADS ? wv : 0);
    const float l_first = (wv < CMB_HEADS && lane < ns) ? a.ws_lse[(base + lane) * 64 + hw] : -INFINITY;
    // ---- first loads: splits 0 .. CMB_UNR-1 of this thread's items (clamped: every load in bounds)
    PT v[ITEMS][CMB_UNR];
    const PT* const part = (const PT*)a.ws_o;           // [rows][D / 4]
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        int item = tid + it * CMB_NT;
        item = item < CMB_HEADS * C4 ? item : CMB_HEADS * C4 - 1;
        const int j = item / C4, c = (item - j * C4) * 4;
        const PT* src = part + ((base * 64 + h0 + j) * D + c) / 4;
#pragma unroll
        for (int u = 0; u < CMB_UNR; ++u) {
            const int sc = u < ns ? u : ns - 1;
            v[it][u] = src[(int64_t)sc * 64 * (D / 4)];
        }
    }
    if (wv < CMB_HEADS) {
        const int hh = hw;
        float M = l_first;
        if (ns > 64) {                                   // more than one pass of 64 splits (rare)
            for (int s0 = 64; s0 < ns; s0 += 64) {
                const float l = s0 + lane < ns ? a.ws_lse[(base + s0 + lane) * 64 + hh] : -INFINITY;
                M = fmaxf(M, l);
            }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
        // a sink logit joins the denominator (once per query, not per split)
        const bool has_sink = a.sink != nullptr && hb * 64 + hh < a.H;
        const float sk = has_sink ? a.sink[hb * 64 + hh] : -INFINITY;
        M = fmaxf(M, sk);
        float den;
        {
            const float w = M == -INFINITY ? 0.f : expf(l_first - M);
            if (lane < ns) wts[wv * ns + lane] = w;
            den = w;
        }
        if (ns > 64) {
            for (int s0 = 64; s0 < ns; s0 += 64) {
                const float l = s0 + lane < ns ? a.ws_lse[(base + s0 + lane) * 64 + hh] : -INFINITY;
                const float w = M == -INFINITY ? 0.f : expf(l - M);
                if (s0 + lane < ns) wts[wv * ns + s0 + lane] = w;
                den += w;
            }
        }
        // fixed-order sum over the wave (butterfly: every lane gets the same bits)
#pragma unroll
        for (int o = 1; o <= 32; o <<= 1) den += __shfl_xor(den, o, 64);
        if (has_sink) den += expf(sk - M);
        const float inv = den > 0.f ? 1.f / den : 0.f;
        for (int s0 = 0; s0 < ns; s0 += 64)
            if (s0 + lane < ns) wts[wv * ns + s0 + lane] *= inv;
        if (lane == 0) lse_o[wv] = den > 0.f ? M + logf(den) : -INFINITY;
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const int item = tid + it * CMB_NT;
        const bool valid = item < CMB_HEADS * C4;
        const int ic = valid ? item : CMB_HEADS * C4 - 1;
        const int j = ic / C4, c = (ic - j * C4) * 4;
        const int hh = h0 + j;
        const int h = hb * 64 + hh;
        const PT* src = part + ((base * 64 + hh) * D + c) / 4;
        const float* wj = wts + j * ns;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int s0 = 0; s0 < ns; s0 += CMB_UNR) {
            if (s0 > 0) {
#pragma unroll
                for (int u = 0; u < CMB_UNR; ++u) {
                    const int sc = s0 + u < ns ? s0 + u : ns - 1;
                    v[it][u] = src[(int64_t)sc * 64 * (D / 4)];
                }
            }
#pragma unroll
            for (int u = 0; u < CMB_UNR; ++u) {
                float4 x;
                if constexpr (PH) {
                    x = make_float4(f16_lo(v[it][u][0]), f16_hi(v[it][u][0]), f16_lo(v[it][u][1]), f16_hi(v[it][u][1]));
                } else {
                    x = v[it][u];
                }
                const float w = s0 + u < ns ? wj[s0 + u] * (PH ? 1.f / ATT_PART_SCALE : 1.f) : 0.f;
                acc.x = fmaf(w, x.x, acc.x); acc.y = fmaf(w, x.y, acc.y);
                acc.z = fmaf(w, x.z, acc.z); acc.w = fmaf(w, x.w, acc.w);
            }
        }
        if (!valid || h >= a.H) continue;
        if (a.out_fmt == F32) {
            *(float4*)((float*)a.out + (bq * a.H + h) * D + c) = acc;
        } else {
            uint2 pk;
            pk.x = pack_bf16x2(acc.x, acc.y);
            pk.y = pack_bf16x2(acc.z, acc.w);
            *(uint2*)((uint16_t*)a.out + (bq * a.H + h) * D + c) = pk;
        }
    }
    if (a.lse && tid < CMB_HEADS && hb * 64 + h0 + tid < a.H) a.lse[bq * a.H + hb * 64 + h0 + tid] = lse_o[tid];
}

template <int D, int FMT>
static hipError_t launch_att2(const AttendArgs& a, hipStream_t s, const AttendPre* pre) {
    dim3 grid((unsigned)a.nsplit, (unsigned)a.nhb, (unsigned)((int64_t)a.B * a.Tq));
    if (a.idx && a.rps > ATT_MAX_SIDX) return hipErrorInvalidValue;
    if constexpr (FMT == F32) {
        hipLaunchKernelGGL((k_attend<D>), grid, dim3(ATT_NT), 0, s, a);
    } else if constexpr (FMT == KV_PACKED && (D == 256 || D == 512)) {
        if (a.r == F8_R && pre)
            hipLaunchKernelGGL((k_attend_f8<D, true>), grid, dim3(MQ_NT), 0, s, a, *pre);
        else if (a.r == F8_R)
            hipLaunchKernelGGL((k_attend_f8<D, false>), grid, dim3(MQ_NT), 0, s, a, AttendPre{});
        else
            hipLaunchKernelGGL((k_attend_mq<D, FMT>), grid, dim3(MQ_NT), 0, s, a);
    } else {
        hipLaunchKernelGGL((k_attend_mq<D, FMT>), grid, dim3(MQ_NT), 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    const size_t lds2 = sizeof(float) * ((size_t)a.nsplit * CMB_HEADS + CMB_HEADS);
    const dim3 cgrid((unsigned)(a.nhb * (64 / CMB_HEADS)), (unsigned)((int64_t)a.B * a.Tq));
    if (FMT == KV_PACKED && (D == 256 || D == 512) && a.r == F8_R && a.out_fmt == BF16)   // k_attend_f8, fp16 partials
        hipLaunchKernelGGL((k_attend_combine<D, true>), cgrid, dim3(CMB_NT), lds2, s, a);
    else
        hipLaunchKernelGGL((k_attend_combine<D, false>), cgrid, dim3(CMB_NT), lds2, s, a);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_att1(const AttendArgs& a, hipStream_t s, const AttendPre* pre) {
    switch (a.kv_fmt) {
    case F32: return launch_att2<D, F32>(a, s, nullptr);
    case BF16: return launch_att2<D, BF16>(a, s, nullptr);
    default: return launch_att2<D, KV_PACKED>(a, s, pre);
    }
}

// the calls whose kernel can compress the layer's new entry first: packed rows with the
// bf16 RoPE part the packed-row kernel takes, one query per sequence
bool attend_takes_pre(const AttendArgs& a) {
    return a.kv_fmt == KV_PACKED && (a.d == 256 || a.d == 512) && a.r == F8_R && a.Tq == 1;
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t s, const AttendPre* pre) {
    if (a.B <= 0 || a.Tq <= 0) return hipSuccess;
    if (pre && !attend_takes_pre(a)) return hipErrorInvalidValue;
    switch (a.d) {
    case 64: return launch_att1<64>(a, s, nullptr);
    case 128: return launch_att1<128>(a, s, nullptr);
    case 256: return launch_att1<256>(a, s, pre);
    default: return launch_att1<512>(a, s, pre);
    }
}

}  // namespace csl
