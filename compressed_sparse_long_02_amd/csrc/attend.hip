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
// 0..n(t)-1 then the window).  Rows are gathered 32 at a time into LDS as bf16
// (fp8 -> bf16 with the hardware OCP conversion).  Each of the 4 waves owns 16
// heads: S = Q.K^T with 16x16x32 bf16 MFMA (Q in registers, K fragments from LDS),
// an online softmax on the accumulators, P staged through LDS, then O += P.V with
// V fragments read from the same row-major tile by the gfx950 LDS transpose read,
// so no transposed copy of V is ever written.  fp32 rows take the same path with
// 16x16x4 f32 MFMA.  Splits write (o, lse) partials that k_attend_combine merges
// in a fixed order (deterministic, no atomics).
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
    static constexpr int KSTR = F32P ? D + 4 : D + 8;          // elements per LDS row
    static constexpr int PSTR = F32P ? ATT_TILE + 4 : ATT_TILE + 8;
    static constexpr int ESZ = F32P ? 4 : 2;
    static constexpr size_t KL_BYTES = (size_t)ATT_TILE * KSTR * ESZ;
    static constexpr size_t PL_BYTES = (size_t)4 * 16 * PSTR * ESZ;
    static constexpr size_t BYTES = KL_BYTES + PL_BYTES + ATT_TILE * (8 + 4);
};

template <int D, int FMT>
__global__ void __launch_bounds__(ATT_NT, 2) k_attend(AttendArgs a) {
    using L = AttLds<D, FMT>;
    constexpr bool F32P = L::F32P;
    constexpr int KSTR = L::KSTR, PSTR = L::PSTR;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t* kl = smem;
    uint8_t* pl = smem + L::KL_BYTES;
    const uint8_t** rowptr = (const uint8_t**)(smem + L::KL_BYTES + L::PL_BYTES);
    int* rowok = (int*)(smem + L::KL_BYTES + L::PL_BYTES + ATT_TILE * 8);

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
    const int64_t rb = FMT == F32 ? 4 * (int64_t)D : (FMT == BF16 ? 2 * (int64_t)D : 2 * (int64_t)a.r + (D - a.r));

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

    constexpr int NDB = D / 16;
    v4f o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = v4f{0.f, 0.f, 0.f, 0.f};
    float m_run[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    float l_run[4] = {0.f, 0.f, 0.f, 0.f};
    const float sl2 = a.scale * CSL_LOG2E;

    const int nch_bf = FMT == KV_PACKED ? a.r / 8 : (FMT == BF16 ? D / 8 : 0);
    const int nch = FMT == F32 ? D / 4 : (FMT == BF16 ? D / 8 : a.r / 8 + (D - a.r) / 16);

    for (int64_t v0 = v_begin; v0 < v_end; v0 += ATT_TILE) {
        // ---- resolve the tile's rows
        if (tid < ATT_TILE) {
            const int64_t v = v0 + tid;
            const uint8_t* p = nullptr;
            int ok = 0;
            if (v < v_end) {
                if (v < n_ent) {
                    int64_t s = v;
                    if (a.idx) s = a.idx[bq * a.k + v];
                    if (s >= 0 && s < a.n_cap) { p = a.kvc + (int64_t)b * a.kvc_bstride + s * rb; ok = 1; }
                } else {
                    const int64_t pos = w0 + (v - n_ent);
                    int64_t slot = (pos - a.kvw_pos0) % a.kvw_rows;
                    if (slot < 0) slot += a.kvw_rows;
                    p = a.kvw + (int64_t)b * a.kvw_bstride + slot * rb;
                    ok = 1;
                }
            }
            rowptr[tid] = p;
            rowok[tid] = ok;
        }
        __syncthreads();
        // ---- gather + convert the tile into LDS (row-major, compute dtype)
        for (int job = tid; job < ATT_TILE * nch; job += ATT_NT) {
            const int rr = job / nch, c = job - rr * nch;
            const uint8_t* p = rowptr[rr];
            if constexpr (F32P) {
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                if (p) v = *(const float4*)(p + 16 * c);
                *(float4*)(kl + ((size_t)rr * KSTR + 4 * c) * 4) = v;
            } else if (FMT == BF16 || c < nch_bf) {
                u32x4 v = {0, 0, 0, 0};
                if (p) v = *(const u32x4*)(p + 16 * c);
                *(u32x4*)(kl + ((size_t)rr * KSTR + 8 * c) * 2) = v;
            } else {
                const int c8 = c - nch_bf;
                u32x4 v = {0, 0, 0, 0};
                if (p) v = *(const u32x4*)(p + 2 * a.r + 16 * c8);
                uint32_t c0, c1, c2, c3, c4, c5, c6, c7;
                e4m3x4_to_bf16x4(v[0], c0, c1);
                e4m3x4_to_bf16x4(v[1], c2, c3);
                e4m3x4_to_bf16x4(v[2], c4, c5);
                e4m3x4_to_bf16x4(v[3], c6, c7);
                const u32x4 lo = {c0, c1, c2, c3}, hi = {c4, c5, c6, c7};
                uint8_t* dst = kl + ((size_t)rr * KSTR + a.r + 16 * c8) * 2;
                *(u32x4*)dst = lo;
                *(u32x4*)(dst + 16) = hi;
            }
        }
        __syncthreads();
        // ---- S = Q K^T for this wave's 16 heads x 32 rows
        v4f s[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            v4f c = {0.f, 0.f, 0.f, 0.f};
            const int row = nb * 16 + col;
            if constexpr (F32P) {
                const float* kr = (const float*)kl + (size_t)row * KSTR;
#pragma unroll
                for (int ks = 0; ks < QKS; ++ks) c = mfma_f32(qf[ks], kr[4 * ks + g], c);
            } else {
                const uint8_t* kr = kl + (size_t)row * KSTR * 2;
#pragma unroll
                for (int ks = 0; ks < QKS; ++ks) c = mfma_bf16(qb[ks], *(const u32x4*)(kr + (32 * ks + 8 * g) * 2), c);
            }
            s[nb] = c;
        }
        // ---- online softmax (base 2); lane holds heads 4g+i of rows nb*16+col
        const bool ok0 = rowok[col] != 0, ok1 = rowok[16 + col] != 0;
        float p0[4], p1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float x0 = ok0 ? s[0][i] * sl2 : -INFINITY;
            const float x1 = ok1 ? s[1][i] * sl2 : -INFINITY;
            float mx = fmaxf(x0, x1);
            mx = fmaxf(mx, shfl_xor(mx, 1));
            mx = fmaxf(mx, shfl_xor(mx, 2));
            mx = fmaxf(mx, shfl_xor(mx, 4));
            mx = fmaxf(mx, shfl_xor(mx, 8));
            const float mnew = fmaxf(m_run[i], mx);
            float corr, e0, e1;
            if (mnew == -INFINITY) {
                corr = 1.f; e0 = 0.f; e1 = 0.f;
            } else {
                corr = exp2f(m_run[i] - mnew);
                e0 = exp2f(x0 - mnew);
                e1 = exp2f(x1 - mnew);
            }
            float rs = e0 + e1;
            rs += shfl_xor(rs, 1);
            rs += shfl_xor(rs, 2);
            rs += shfl_xor(rs, 4);
            rs += shfl_xor(rs, 8);
            l_run[i] = l_run[i] * corr + rs;
            m_run[i] = mnew;
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[db][i] *= corr;
            p0[i] = e0;
            p1[i] = e1;
        }
        // ---- P -> LDS: pl[wave][head 4g+i][row]
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int hh = 4 * g + i;
            if constexpr (F32P) {
                float* pr = (float*)pl + ((size_t)wv * 16 + hh) * PSTR;
                pr[col] = p0[i];
                pr[16 + col] = p1[i];
            } else {
                uint16_t* pr = (uint16_t*)pl + ((size_t)wv * 16 + hh) * PSTR;
                pr[col] = (uint16_t)f32_to_bf16_rne(p0[i]);
                pr[16 + col] = (uint16_t)f32_to_bf16_rne(p1[i]);
            }
        }
        __syncthreads();
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
            const u32x4 pa = *(const u32x4*)((const uint16_t*)pl + ((size_t)wv * 16 + col) * PSTR + 8 * g);
            const uint16_t* kb = (const uint16_t*)kl;
            const uint16_t* v0p = kb + (size_t)(8 * g + (col >> 2)) * KSTR + 4 * (col & 3);
            const uint16_t* v1p = v0p + 4 * KSTR;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const u32x2 r0 = lds_read_tr16(v0p + 16 * db);
                const u32x2 r1 = lds_read_tr16(v1p + 16 * db);
                const u32x4 vb = {r0[0], r0[1], r1[0], r1[1]};
                o[db] = mfma_bf16(pa, vb, o[db]);
            }
        }
        __syncthreads();
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
template <int D>
__global__ void __launch_bounds__(256) k_attend_combine(AttendArgs a) {
    extern __shared__ float wts[];   // [nsplit][64] weights, then [64] 1/den, [64] lse
    const int hb = blockIdx.x;
    const int64_t bq = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t base = (bq * a.nhb + hb) * (int64_t)a.nsplit;
    float* inv = wts + a.nsplit * 64;
    float* lse_o = inv + 64;
    if (tid < 64) {
        float M = -INFINITY;
        for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.ws_lse[(base + s) * 64 + tid]);
        float den = 0.f;
        for (int s = 0; s < a.nsplit; ++s) {
            const float w = M == -INFINITY ? 0.f : expf(a.ws_lse[(base + s) * 64 + tid] - M);
            wts[s * 64 + tid] = w;
            den += w;
        }
        inv[tid] = den > 0.f ? 1.f / den : 0.f;
        lse_o[tid] = den > 0.f ? M + logf(den) : -INFINITY;
    }
    __syncthreads();
    constexpr int C4 = D / 4;
    for (int item = tid; item < 64 * C4; item += 256) {
        const int hh = item / C4, c = (item - hh * C4) * 4;
        const int h = hb * 64 + hh;
        if (h >= a.H) continue;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int s = 0; s < a.nsplit; ++s) {
            const float w = wts[s * 64 + hh];
            const float4 v = *(const float4*)(a.ws_o + ((base + s) * 64 + hh) * D + c);
            acc.x = fmaf(w, v.x, acc.x); acc.y = fmaf(w, v.y, acc.y);
            acc.z = fmaf(w, v.z, acc.z); acc.w = fmaf(w, v.w, acc.w);
        }
        const float iv = inv[hh];
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
    if (a.lse && tid < 64 && hb * 64 + tid < a.H) a.lse[bq * a.H + hb * 64 + tid] = lse_o[tid];
}

template <int D, int FMT>
static hipError_t launch_att2(const AttendArgs& a, hipStream_t s) {
    dim3 grid((unsigned)a.nsplit, (unsigned)a.nhb, (unsigned)((int64_t)a.B * a.Tq));
    const size_t lds = AttLds<D, FMT>::BYTES;
    hipLaunchKernelGGL((k_attend<D, FMT>), grid, dim3(ATT_NT), lds, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    const size_t lds2 = sizeof(float) * ((size_t)a.nsplit * 64 + 128);
    hipLaunchKernelGGL((k_attend_combine<D>), dim3((unsigned)a.nhb, (unsigned)((int64_t)a.B * a.Tq)), dim3(256),
                       lds2, s, a);
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
