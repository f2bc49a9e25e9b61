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
// 0..n(t)-1 then the window).  Rows are gathered 32 at a time with the direct
// global->LDS loads of gfx950 (no staging registers), one tile ahead of the
// compute, then converted once into a padded bf16 tile (fp8 -> bf16 with the
// hardware OCP conversion).  Each of the 4 waves owns 16 heads: S = Q.K^T with
// 16x16x32 bf16 MFMA (Q in registers, K fragments from LDS), an online softmax
// on the accumulators with a lazy rescale, P staged through LDS, then O += P.V
// with V fragments read from the same row-major tile by the gfx950 LDS transpose
// read, so no transposed copy of V is ever written.  fp32 rows take the same path
// with 16x16x4 f32 MFMA.  Splits write (o, lse) partials that k_attend_combine
// merges in a fixed order (deterministic, no atomics).
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace csl {

constexpr int ATT_NT = 256;
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
    static constexpr int PSTR = F32P ? ATT_TILE + 4 : ATT_TILE + 8;
    static constexpr int ESZ = F32P ? 4 : 2;
    static constexpr int KL_ELEMS = ATT_TILE * KSTR;
    static constexpr int RAW_BYTES = ATT_TILE * D * (F32P ? 4 : 2);   // largest stored row: bf16 / fp32
    static constexpr int PL_ELEMS = 4 * 16 * PSTR;
};
constexpr int ATT_MAX_SIDX = 1536;   // CSA split lengths are capped to this (host plan)

// Position of key e (0..7) of an 8-key group inside P's LDS row: even keys first,
// then odd ones, matching the row order of the transposed V reads below.
__device__ __forceinline__ int p_perm(int key) { return (key & ~7) + ((key & 1) ? 4 + ((key & 7) >> 1) : ((key & 7) >> 1)); }

constexpr float ATT_TAU = 8.0f;   // lazy rescale: keep the reference max until it trails by 2^8

template <int D, int FMT>
__global__ void __launch_bounds__(ATT_NT, 2) k_attend(AttendArgs a) {
    using L = AttLds<D, FMT>;
    constexpr bool F32P = L::F32P;
    constexpr int KSTR = L::KSTR, PSTR = L::PSTR;
    using KT = typename std::conditional<F32P, float, uint16_t>::type;
    // separate LDS objects: the asynchronous global->LDS loads only ever write `raw`,
    // which lets the compiler see that reads of the K tile and P do not alias them
    __shared__ __attribute__((aligned(16))) KT kl_s[L::KL_ELEMS];
    __shared__ __attribute__((aligned(16))) uint8_t raw[L::RAW_BYTES];
    __shared__ __attribute__((aligned(16))) KT pl_s[L::PL_ELEMS];
    __shared__ const uint8_t* rowptr[2 * ATT_TILE];
    __shared__ int rowok[2 * ATT_TILE];
    __shared__ int sidx[ATT_MAX_SIDX];
    uint8_t* kl = (uint8_t*)kl_s;
    uint8_t* pl = (uint8_t*)pl_s;
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

    // ---- Q fragments (A operand): head h = hb*64 + wv*16 + col
    const int h_a = hb * 64 + wv * 16 + col;
    constexpr int QKS = F32P ? D / 4 : D / 32;
    u32x4 qb[F32P ? 1 : QKS];
    float qf[F32P ? QKS : 1];
    if constexpr (F32P) {
        const float* qrow = (const float*)a.q + (bq * a.H + h_a) * D;
#pragma unroll
        for (int ks = 0; ks < QKS; ++ks) qf[ks] = h_a < a.H ? qrow[4 * ks + g] : 0.f;
    } else {
        const uint8_t* qrow = a.q + (bq * a.H + h_a) * (int64_t)D * 2;
#pragma unroll
        for (int ks = 0; ks < QKS; ++ks)
            qb[ks] = h_a < a.H ? *(const u32x4*)(qrow + (32 * ks + 8 * g) * 2) : u32x4{0, 0, 0, 0};
    }
    __syncthreads();

    // rows of tile `it` -> rowptr/rowok slot it&1 (threads 0..TILE-1)
    auto resolve = [&](int it) {
        if (tid < ATT_TILE) {
            const int64_t v = v_begin + (int64_t)it * ATT_TILE + tid;
            const uint8_t* p = nullptr;
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
            rowok[(it & 1) * ATT_TILE + tid] = p != nullptr;
        }
    };
    // asynchronous gather of tile `it` into the raw LDS tile: lane l of a wave writes
    // chunk 64*wc + l at raw + 1024*wc + 16*l (direct global -> LDS loads)
    auto gather = [&](int it) {
        const uint8_t** rp = rowptr + (it & 1) * ATT_TILE;
        for (int wc = wv; wc * 64 < nch; wc += ATT_NT / 64) {
            const int c = wc * 64 + lane;
            if (c < nch) {
                const int rr = c / cpr, pc = c - rr * cpr;
                const uint8_t* p = rp[rr];
                if (p)
                    __builtin_amdgcn_global_load_lds((const void*)(p + 16 * pc),
                                                     (__attribute__((address_space(3))) void*)(raw + 1024 * wc), 16, 0, 0);
            }
        }
    };

    constexpr int NDB = D / 16;
    v4f o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = v4f{0.f, 0.f, 0.f, 0.f};
    float m_run[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    float l_run[4] = {0.f, 0.f, 0.f, 0.f};
    const float sl2 = a.scale * CSL_LOG2E;
    const int nch_bf = FMT == KV_PACKED ? a.r / 8 : cpr;    // chunks stored as bf16

    if (ntiles > 0) {
        resolve(0);
        __syncthreads();
        gather(0);
    }
    for (int it = 0; it < ntiles; ++it) {
        const int* ok = rowok + (it & 1) * ATT_TILE;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        // ---- convert the raw tile into the padded compute-dtype K tile
        for (int c = tid; c < nch; c += ATT_NT) {
            const int rr = c / cpr, pc = c - rr * cpr;
            u32x4 v = *(const u32x4*)(raw + 16 * c);
            if (!ok[rr]) v = u32x4{0, 0, 0, 0};
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
        lds_barrier();
        if (it + 1 < ntiles) gather(it + 1);          // overlaps the MFMA work below
        // ---- S = Q K^T for this wave's 16 heads x 32 rows: two independent MFMA
        //      chains (rows 0-15, 16-31), operands read one k-step ahead
        v4f s[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
        if constexpr (F32P) {
            const float* k0 = (const float*)kl + (size_t)col * KSTR + g;
            const float* k1 = k0 + 16 * KSTR;
            float b0 = k0[0], b1 = k1[0];
#pragma unroll
            for (int ks = 0; ks < QKS; ++ks) {
                float n0 = 0.f, n1 = 0.f;
                if (ks + 1 < QKS) { n0 = k0[4 * (ks + 1)]; n1 = k1[4 * (ks + 1)]; }
                s[0] = mfma_f32(qf[ks], b0, s[0]);
                s[1] = mfma_f32(qf[ks], b1, s[1]);
                b0 = n0; b1 = n1;
            }
        } else {
            const uint8_t* k0 = kl + ((size_t)col * KSTR + 8 * g) * 2;
            const uint8_t* k1 = k0 + (size_t)16 * KSTR * 2;
            u32x4 b0 = *(const u32x4*)k0, b1 = *(const u32x4*)k1;
#pragma unroll
            for (int ks = 0; ks < QKS; ++ks) {
                u32x4 n0 = b0, n1 = b1;
                if (ks + 1 < QKS) { n0 = *(const u32x4*)(k0 + 64 * (ks + 1)); n1 = *(const u32x4*)(k1 + 64 * (ks + 1)); }
                s[0] = mfma_bf16(qb[ks], b0, s[0]);
                s[1] = mfma_bf16(qb[ks], b1, s[1]);
                b0 = n0; b1 = n1;
            }
        }
        // ---- online softmax (base 2), lazy rescale; lane holds heads 4g+i of rows nb*16+col
        const bool ok0 = ok[col] != 0, ok1 = ok[16 + col] != 0;
        float p0[4], p1[4], corr[4];
        bool need = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float x0 = ok0 ? s[0][i] * sl2 : -INFINITY;
            const float x1 = ok1 ? s[1][i] * sl2 : -INFINITY;
            float mx = fmaxf(x0, x1);
            mx = fmaxf(mx, shfl_xor(mx, 1));
            mx = fmaxf(mx, shfl_xor(mx, 2));
            mx = fmaxf(mx, shfl_xor(mx, 4));
            mx = fmaxf(mx, shfl_xor(mx, 8));
            corr[i] = 1.f;
            if (mx > m_run[i] + ATT_TAU) {           // the reference max moves up
                corr[i] = exp2f(m_run[i] - mx);      // 0 on the first valid tile
                m_run[i] = mx;
                need = true;
            }
            const float e0 = m_run[i] == -INFINITY ? 0.f : exp2f(x0 - m_run[i]);
            const float e1 = m_run[i] == -INFINITY ? 0.f : exp2f(x1 - m_run[i]);
            float rs = e0 + e1;
            rs += shfl_xor(rs, 1);
            rs += shfl_xor(rs, 2);
            rs += shfl_xor(rs, 4);
            rs += shfl_xor(rs, 8);
            l_run[i] = l_run[i] * corr[i] + rs;
            p0[i] = e0;
            p1[i] = e1;
        }
        if (__builtin_amdgcn_read_exec() & __ballot(need)) {   // wave-uniform: some head rescaled
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[db][i] *= corr[i];
        }
        // ---- P -> LDS: pl[wave][head 4g+i][row position]
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int hh = 4 * g + i;
            if constexpr (F32P) {
                float* pr = (float*)pl + ((size_t)wv * 16 + hh) * PSTR;
                pr[col] = p0[i];
                pr[16 + col] = p1[i];
            } else {
                uint16_t* pr = (uint16_t*)pl + ((size_t)wv * 16 + hh) * PSTR;
                pr[p_perm(col)] = (uint16_t)f32_to_bf16_rne(p0[i]);
                pr[p_perm(16 + col)] = (uint16_t)f32_to_bf16_rne(p1[i]);
            }
        }
        lds_barrier();
        // ---- O += P V
        if constexpr (F32P) {
            const float* pr = (const float*)pl + ((size_t)wv * 16 + col) * PSTR;
            const float* kf = (const float*)kl;
#pragma unroll
            for (int ks = 0; ks < ATT_TILE / 4; ++ks) {
                const float pa = pr[4 * ks + g];
                const float* vr = kf + (size_t)(4 * ks + g) * KSTR + col;
#pragma unroll
                for (int db = 0; db < NDB; ++db) o[db] = mfma_f32(pa, vr[16 * db], o[db]);
            }
        } else {
            // k slot j of lane group g holds key 8g + 2j (j < 4) or 8g + 2(j-4) + 1: the
            // source rows of one transposed read are 2 apart, which spreads them over
            // all 32 banks (row stride = 4 banks mod 32)
            const u32x4 pa = *(const u32x4*)((const uint16_t*)pl + ((size_t)wv * 16 + col) * PSTR + 8 * g);
            const uint16_t* kb = (const uint16_t*)kl;
            const uint16_t* v0p = kb + (size_t)(8 * g + 2 * (col >> 2)) * KSTR + 4 * (col & 3);
            const uint16_t* v1p = v0p + KSTR;
            u32x2 r0 = lds_read_tr16(v0p), r1 = lds_read_tr16(v1p);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                u32x2 n0 = r0, n1 = r1;
                if (db + 1 < NDB) { n0 = lds_read_tr16(v0p + 16 * (db + 1)); n1 = lds_read_tr16(v1p + 16 * (db + 1)); }
                const u32x4 vb = {r0[0], r0[1], r1[0], r1[1]};
                o[db] = mfma_bf16(pa, vb, o[db]);
                r0 = n0; r1 = n1;
            }
        }
        // the next iteration starts with a full barrier before the K tile is rewritten
    }

    // ---- finish: normalise, write output or the split's partial
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int hh = wv * 16 + 4 * g + i;       // head within the block
        const int h = hb * 64 + hh;
        const float inv = l_run[i] > 0.f ? 1.f / l_run[i] : 0.f;
        const float lse = l_run[i] > 0.f ? (m_run[i] + log2f(l_run[i])) * CSL_LN2 : -INFINITY;
        if (a.nsplit == 1) {
            if (h < a.H) {
                if (a.out_fmt == F32) {
                    float* orow = (float*)a.out + (bq * a.H + h) * D;
#pragma unroll
                    for (int db = 0; db < NDB; ++db) orow[16 * db + col] = o[db][i] * inv;
                } else {
                    uint16_t* orow = (uint16_t*)a.out + (bq * a.H + h) * D;
#pragma unroll
                    for (int db = 0; db < NDB; ++db) orow[16 * db + col] = (uint16_t)f32_to_bf16_rne(o[db][i] * inv);
                }
                if (a.lse && col == 0) a.lse[bq * a.H + h] = lse;
            }
        } else {
            const int64_t prow = ((bq * a.nhb + hb) * a.nsplit + sp) * 64 + hh;
            float* orow = a.ws_o + prow * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db) orow[16 * db + col] = o[db][i] * inv;
            if (col == 0) a.ws_lse[prow] = lse;
        }
    }
}

// Merge of split partials: out = sum_s exp(lse_s - M) o_s / sum_s exp(lse_s - M).
// One block per (query, 4 heads): the 64 heads of a head block spread over 16
// blocks so that the merge reads its partials with the whole GPU.
constexpr int CMB_HEADS = 4;

template <int D>
__global__ void __launch_bounds__(256) k_attend_combine(AttendArgs a) {
    extern __shared__ float wts[];   // [nsplit][CMB_HEADS] weights, then 1/den, lse
    const int hb = blockIdx.x / (64 / CMB_HEADS);
    const int h0 = (blockIdx.x % (64 / CMB_HEADS)) * CMB_HEADS;   // first head within the head block
    const int64_t bq = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t base = (bq * a.nhb + hb) * (int64_t)a.nsplit;
    float* inv = wts + a.nsplit * CMB_HEADS;
    float* lse_o = inv + CMB_HEADS;
    if (tid < CMB_HEADS) {
        const int hh = h0 + tid;
        float M = -INFINITY;
        for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.ws_lse[(base + s) * 64 + hh]);
        float den = 0.f;
        for (int s = 0; s < a.nsplit; ++s) {
            const float w = M == -INFINITY ? 0.f : expf(a.ws_lse[(base + s) * 64 + hh] - M);
            wts[s * CMB_HEADS + tid] = w;
            den += w;
        }
        inv[tid] = den > 0.f ? 1.f / den : 0.f;
        lse_o[tid] = den > 0.f ? M + logf(den) : -INFINITY;
    }
    __syncthreads();
    constexpr int C4 = D / 4;
    for (int item = tid; item < CMB_HEADS * C4; item += 256) {
        const int j = item / C4, c = (item - j * C4) * 4;
        const int hh = h0 + j;
        const int h = hb * 64 + hh;
        if (h >= a.H) continue;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int s = 0; s < a.nsplit; ++s) {
            const float w = wts[s * CMB_HEADS + j];
            const float4 v = *(const float4*)(a.ws_o + ((base + s) * 64 + hh) * D + c);
            acc.x = fmaf(w, v.x, acc.x); acc.y = fmaf(w, v.y, acc.y);
            acc.z = fmaf(w, v.z, acc.z); acc.w = fmaf(w, v.w, acc.w);
        }
        const float iv = inv[j];
        acc.x *= iv; acc.y *= iv; acc.z *= iv; acc.w *= iv;
        if (a.out_fmt == F32) {
            *(float4*)((float*)a.out + (bq * a.H + h) * D + c) = acc;
        } else {
            uint2 pk;
            pk.x = f32_to_bf16_rne(acc.x) | (f32_to_bf16_rne(acc.y) << 16);
            pk.y = f32_to_bf16_rne(acc.z) | (f32_to_bf16_rne(acc.w) << 16);
            *(uint2*)((uint16_t*)a.out + (bq * a.H + h) * D + c) = pk;
        }
    }
    if (a.lse && tid < CMB_HEADS && hb * 64 + h0 + tid < a.H) a.lse[bq * a.H + hb * 64 + h0 + tid] = lse_o[tid];
}

template <int D, int FMT>
static hipError_t launch_att2(const AttendArgs& a, hipStream_t s) {
    dim3 grid((unsigned)a.nsplit, (unsigned)a.nhb, (unsigned)((int64_t)a.B * a.Tq));
    const int64_t rb = FMT == F32 ? 4 * (int64_t)D : (FMT == BF16 ? 2 * (int64_t)D : 2 * (int64_t)a.r + (D - a.r));
    if (a.idx && a.rps > ATT_MAX_SIDX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_attend<D, FMT>), grid, dim3(ATT_NT), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    const size_t lds2 = sizeof(float) * ((size_t)a.nsplit * CMB_HEADS + 2 * CMB_HEADS);
    hipLaunchKernelGGL((k_attend_combine<D>), dim3((unsigned)(a.nhb * (64 / CMB_HEADS)), (unsigned)((int64_t)a.B * a.Tq)),
                       dim3(256), lds2, s, a);
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
