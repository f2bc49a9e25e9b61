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
// (deterministic, no atomics).
#include <type_traits>

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

template <int D, int FMT>
struct AttLds {
    static constexpr bool F32P = FMT == F32;
    static constexpr int KSTR = F32P ? D + 4 : D + 8;          // elements per K-tile row (bank padding)
    static constexpr int KL_ELEMS = ATT_TILE * KSTR;
    // 16-byte chunks of the longest stored row (packed rows: r <= D/4 RoPE dims)
    static constexpr int CPR_MAX = F32P ? D / 4 : (FMT == BF16 ? D / 8 : (D + D / 4) / 16);
    static constexpr int NJ = (ATT_TILE * CPR_MAX + ATT_NT - 1) / ATT_NT;   // chunks per thread per tile
};
constexpr int ATT_MAX_SIDX = 1536;   // CSA split lengths are capped to this (host plan)

constexpr float ATT_TAU = 8.0f;   // lazy rescale: keep the reference max until it trails by 2^8
constexpr float ATT_HEADROOM = 64.0f;   // largest x - m_ref (base 2) accepted without a rescale
constexpr float ATT_REF_LIFT = 32.0f;   // m_ref starts this far above the first tile's largest logit

// 16x16x16 bf16 MFMA: A lane l = row l%16, k 4*(l/16)..+4; B lane l = col l%16, same k.
__device__ __forceinline__ v4f mfma_bf16_k16(const u32x2& a, const u32x2& b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4s, a), __builtin_bit_cast(v4s, b), c, 0, 0, 0);
}

template <int D, int FMT>
__global__ void __launch_bounds__(ATT_NT, 2) k_attend(AttendArgs a) {
    using L = AttLds<D, FMT>;
    constexpr bool F32P = L::F32P;
    constexpr int KSTR = L::KSTR;
    using KT = typename std::conditional<F32P, float, uint16_t>::type;
    __shared__ __attribute__((aligned(16))) KT kl_s[L::KL_ELEMS];
    __shared__ const uint8_t* rowptr[2 * ATT_TILE];
    __shared__ uint32_t rowmask[2];
    __shared__ int sidx[ATT_MAX_SIDX];
    uint8_t* kl = (uint8_t*)kl_s;
    const int64_t rb = FMT == F32 ? 4 * (int64_t)D : (FMT == BF16 ? 2 * (int64_t)D : 2 * (int64_t)a.r + (D - a.r));

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
    const int cpr = (int)(rb / 16);                     // 16-byte chunks per stored row
    const int nch = ATT_TILE * cpr;

    // ---- the split's slice of the index list, staged once (CSA)
    if (a.idx) {
        const int64_t e_end = v_end < n_ent ? v_end : n_ent;
        for (int64_t v = v_begin + tid; v < e_end; v += ATT_NT) sidx[v - v_begin] = a.idx[bq * a.k + v];
    }

    // ---- Q fragments (B operand of S^T = K Q^T): head h = hb*64 + wv*16 + col.  The
    //      first QR k-steps live in registers; for d = 512 the last QL k-steps are
    //      read from LDS, which keeps the kernel inside 256 registers (two blocks/CU).
    const int h_a = hb * 64 + wv * 16 + col;
    constexpr int QKS = F32P ? D / 4 : D / 32;
    constexpr int QL = (!F32P && D == 512) ? (FMT == BF16 ? 12 : 8) : 0;
    constexpr int QR = QKS - QL;
    constexpr int QSTR = QL * 32 + 8;                   // bf16 per head row in LDS (16-byte pad)
    __shared__ __attribute__((aligned(16))) uint16_t ql_s[QL > 0 ? 64 * QSTR : 8];
    u32x4 qb[F32P ? 1 : QR];
    float qf[F32P ? QKS : 1];
    if constexpr (F32P) {
        const float* qrow = (const float*)a.q + (bq * a.H + h_a) * D;
#pragma unroll
        for (int ks = 0; ks < QKS; ++ks) qf[ks] = h_a < a.H ? qrow[4 * ks + g] : 0.f;
    } else {
        const uint8_t* qrow = a.q + (bq * a.H + h_a) * (int64_t)D * 2;
#pragma unroll
        for (int ks = 0; ks < QR; ++ks)
            qb[ks] = h_a < a.H ? *(const u32x4*)(qrow + (32 * ks + 8 * g) * 2) : u32x4{0, 0, 0, 0};
        if constexpr (QL > 0) {
            for (int c = tid; c < 64 * QL * 4; c += ATT_NT) {
                const int hq = c / (QL * 4), pc = c - hq * (QL * 4);
                const int hg = hb * 64 + hq;
                const u32x4 v = hg < a.H ? *(const u32x4*)(a.q + ((bq * a.H + hg) * (int64_t)D + 32 * QR + 8 * pc) * 2)
                                         : u32x4{0, 0, 0, 0};
                *(u32x4*)(ql_s + hq * QSTR + 8 * pc) = v;
            }
        }
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
                        if (s >= 0 && s < a.n_cap) p = a.kvc + (int64_t)b * a.kvc_bstride + s * rb;
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
    // tile (row c / cpr, 16-byte piece c % cpr), the same for every tile.  The loads
    // of tile it+1 are issued right after tile it reaches LDS and are consumed at the
    // top of the next iteration, so a whole tile of MFMA work hides their latency.
    // Every load is issued (an empty row re-reads the query row and is zeroed), which
    // keeps the load stream branch-free.
    constexpr int NJ = L::NJ;
    u32x4 R[NJ];
    uint32_t okm = 0;
    auto load_regs = [&](int it) {
        const uint8_t** rp = rowptr + (it & 1) * ATT_TILE;
        okm = 0;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int c = tid + ATT_NT * j;
            const int rr = c / cpr;
            const uint8_t* p = c < nch ? rp[rr] : nullptr;
            const bool okc = p != nullptr;
            R[j] = ld_global<u32x4>(okc ? p + 16 * (c - rr * cpr) : a.q);
            okm |= okc ? 1u << j : 0u;
        }
    };

    constexpr int NDB = D / 16;
    v4f o[NDB];          // O^T: lane holds dims 16*db + 4g + i of head col
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = v4f{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const float sl2 = a.scale * CSL_LOG2E;
    const int nch_bf = FMT == KV_PACKED ? a.r / 8 : cpr;    // chunks stored as bf16

    if (ntiles > 0) {
        resolve(0);
        __syncthreads();
        load_regs(0);
    }
    for (int it = 0; it < ntiles; ++it) {
        lds_barrier();                                  // the previous tile's K/V reads are done
        // ---- the prefetched chunks -> the padded compute-dtype K tile
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int c = tid + ATT_NT * j;
            if (c >= nch) continue;
            const int rr = c / cpr, pc = c - rr * cpr;
            const u32x4 v = ((okm >> j) & 1u) ? R[j] : u32x4{0, 0, 0, 0};
            if constexpr (F32P) {
                *(u32x4*)(kl + ((size_t)rr * KSTR + 4 * pc) * 4) = v;
            } else if (FMT == BF16 || pc < nch_bf) {
                *(u32x4*)(kl + ((size_t)rr * KSTR + 8 * pc) * 2) = v;
            } else {
                const int c8 = pc - nch_bf;
                uint32_t c0, c1, c2, c3, c4, c5, c6, c7;
                e4m3x4_to_bf16x4(v[0], c0, c1);
                e4m3x4_to_bf16x4(v[1], c2, c3);
                e4m3x4_to_bf16x4(v[2], c4, c5);
                e4m3x4_to_bf16x4(v[3], c6, c7);
                uint8_t* dst = kl + ((size_t)rr * KSTR + a.r + 16 * c8) * 2;
                *(u32x4*)dst = u32x4{c0, c1, c2, c3};
                *(u32x4*)(dst + 16) = u32x4{c4, c5, c6, c7};
            }
        }
        if (it + 1 < ntiles) resolve(it + 1);
        lds_barrier();                                  // K tile and the next rows' pointers visible
        if (it + 1 < ntiles) load_regs(it + 1);         // in flight during the MFMA work below
        const uint32_t rmask = rowmask[it & 1];
        // ---- S^T = K Q^T: rows 16*r2 + 4g + i of head col, two independent MFMA chains
        v4f s[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
        if constexpr (F32P) {
            const float* k0 = (const float*)kl + (size_t)col * KSTR + g;
            const float* k1 = k0 + 16 * KSTR;
#pragma unroll
            for (int ks = 0; ks < QKS; ++ks) {
                s[0] = mfma_f32(k0[4 * ks], qf[ks], s[0]);
                s[1] = mfma_f32(k1[4 * ks], qf[ks], s[1]);
            }
        } else {
            const uint8_t* k0 = kl + ((size_t)col * KSTR + 8 * g) * 2;
            const uint8_t* k1 = k0 + (size_t)16 * KSTR * 2;
#pragma unroll
            for (int ks = 0; ks < QR; ++ks) {
                s[0] = mfma_bf16(*(const u32x4*)(k0 + 64 * ks), qb[ks], s[0]);
                s[1] = mfma_bf16(*(const u32x4*)(k1 + 64 * ks), qb[ks], s[1]);
            }
            const uint16_t* qlp = ql_s + (wv * 16 + col) * QSTR + 8 * g;
#pragma unroll
            for (int ks = QR; ks < QKS; ++ks) {
                const u32x4 qv = *(const u32x4*)(qlp + 32 * (ks - QR));
                s[0] = mfma_bf16(*(const u32x4*)(k0 + 64 * ks), qv, s[0]);
                s[1] = mfma_bf16(*(const u32x4*)(k1 + 64 * ks), qv, s[1]);
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
        u32x2 pb[2];
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[r2][i] = m_run == -INFINITY ? 0.f : exp2f(x[r2][i] - m_run);
                rs += x[r2][i];
            }
            pb[r2] = u32x2{f32_to_bf16_rne(x[r2][0]) | (f32_to_bf16_rne(x[r2][1]) << 16),
                           f32_to_bf16_rne(x[r2][2]) | (f32_to_bf16_rne(x[r2][3]) << 16)};
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
        if constexpr (F32P) {
            const float* kf = (const float*)kl;
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float* vr = kf + (size_t)(16 * r2 + 4 * g + i) * KSTR + col;
#pragma unroll
                    for (int db = 0; db < NDB; ++db) o[db] = mfma_f32(vr[16 * db], x[r2][i], o[db]);
                }
        } else {
            // V^T fragments by the LDS transpose read: source lane 16g + s reads the four
            // dims 16*db + 4*(s%4).. of row 16*r2 + 4g + s/4, so lane (g, col) receives
            // dim 16*db + col of rows 16*r2 + 4g + 0..3
            const uint16_t* kb = (const uint16_t*)kl;
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2) {
                const uint16_t* vp = kb + (size_t)(16 * r2 + 4 * g + (col >> 2)) * KSTR + 4 * (col & 3);
#pragma unroll
                for (int db = 0; db < NDB; ++db) o[db] = mfma_bf16_k16(lds_read_tr16(vp + 16 * db), pb[r2], o[db]);
            }
        }
        // the next iteration starts with a barrier before the K tile is rewritten
    }

    // ---- finish: normalise, write output or the split's partial
    const int hh = wv * 16 + col;                  // head within the block
    const int h = hb * 64 + hh;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const float lse = l_run > 0.f ? (m_run + log2f(l_run)) * CSL_LN2 : -INFINITY;
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
                        if (s >= 0 && s < a.n_cap) p = a.kvc + (int64_t)b * a.kvc_bstride + s * rb;
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
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        const float lse = l_run > 0.f ? (m_run + log2f(l_run)) * CSL_LN2 : -INFINITY;
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

// Merge of split partials: out = sum_s exp(lse_s - M) o_s / sum_s exp(lse_s - M).
// One block per (query, 4 heads): the 64 heads of a head block spread over 16
// blocks so that the merge reads its partials with the whole GPU.  Waves 0..3 first
// load the split lse of heads h0..h0+3 (lane s holds split s), then every thread
// issues the loads of its first CMB_UNR splits; the weights are formed while those
// are in flight (loads complete in issue order, so waiting for the lse does not wait
// for the partials), and the splits are accumulated in split order.
constexpr int CMB_HEADS = 4;
constexpr int CMB_UNR = 16;
constexpr int CMB_NT = 512;

template <int D>
__global__ void __launch_bounds__(CMB_NT) k_attend_combine(AttendArgs a) {
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
    float4 v[ITEMS][CMB_UNR];
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        int item = tid + it * CMB_NT;
        item = item < CMB_HEADS * C4 ? item : CMB_HEADS * C4 - 1;
        const int j = item / C4, c = (item - j * C4) * 4;
        const float* src = a.ws_o + (base * 64 + h0 + j) * D + c;
#pragma unroll
        for (int u = 0; u < CMB_UNR; ++u) {
            const int sc = u < ns ? u : ns - 1;
            v[it][u] = *(const float4*)(src + (int64_t)sc * 64 * D);
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
        const float* src = a.ws_o + (base * 64 + hh) * D + c;
        const float* wj = wts + j * ns;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int s0 = 0; s0 < ns; s0 += CMB_UNR) {
            if (s0 > 0) {
#pragma unroll
                for (int u = 0; u < CMB_UNR; ++u) {
                    const int sc = s0 + u < ns ? s0 + u : ns - 1;
                    v[it][u] = *(const float4*)(src + (int64_t)sc * 64 * D);
                }
            }
#pragma unroll
            for (int u = 0; u < CMB_UNR; ++u) {
                const float w = s0 + u < ns ? wj[s0 + u] : 0.f;
                acc.x = fmaf(w, v[it][u].x, acc.x); acc.y = fmaf(w, v[it][u].y, acc.y);
                acc.z = fmaf(w, v[it][u].z, acc.z); acc.w = fmaf(w, v[it][u].w, acc.w);
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
static hipError_t launch_att2(const AttendArgs& a, hipStream_t s) {
    dim3 grid((unsigned)a.nsplit, (unsigned)a.nhb, (unsigned)((int64_t)a.B * a.Tq));
    if (a.idx && a.rps > ATT_MAX_SIDX) return hipErrorInvalidValue;
    if constexpr (FMT == F32) {
        hipLaunchKernelGGL((k_attend<D, FMT>), grid, dim3(ATT_NT), 0, s, a);
    } else {
        hipLaunchKernelGGL((k_attend_mq<D, FMT>), grid, dim3(MQ_NT), 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    const size_t lds2 = sizeof(float) * ((size_t)a.nsplit * CMB_HEADS + CMB_HEADS);
    hipLaunchKernelGGL((k_attend_combine<D>), dim3((unsigned)(a.nhb * (64 / CMB_HEADS)), (unsigned)((int64_t)a.B * a.Tq)),
                       dim3(CMB_NT), lds2, s, a);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_att1(const AttendArgs& a, hipStream_t s) {
    switch (a.kv_fmt) {
    case F32: return launch_att2<D, F32>(a, s);
    case BF16: return launch_att2<D, BF16>(a, s);
    default: return launch_att2<D, KV_PACKED>(a, s);
    }
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
    if (a.B <= 0 || a.Tq <= 0) return hipSuccess;
    switch (a.d) {
    case 64: return launch_att1<64>(a, s);
    case 128: return launch_att1<128>(a, s);
    case 256: return launch_att1<256>(a, s);
    default: return launch_att1<512>(a, s);
    }
}

}  // namespace csl
