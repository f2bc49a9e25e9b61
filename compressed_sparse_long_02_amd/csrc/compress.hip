// compress.hip -- token compression of raw KV rows into compressed entries.
//
// Method: x-techcon article on DeepSeek-V4, section 2, CSA step 1 -- every m raw
// tokens become one entry: a learned weight per raw token plus a position bias,
// normalised by a softmax, then a weighted sum; adjacent blocks overlap.  The HCA
// subsection applies the same operator at m' = 128.  Window geometry (a reading):
// entry i pools raw positions (i+1)m-win .. (i+1)m-1, win = 2m with overlap, m
// without; positions < 0 are left out of the softmax.
//
// Streaming, HBM-bound kernel.  A thread owns 8 consecutive channels (one 16-byte
// bf16 load per row); d/8 adjacent threads cover a row, and RG such groups split
// the window's rows between them, each running an online softmax over its rows.
// The RG partial (max, sum, weighted sum) triples are merged -- each rescaled to the
// entry's maximum, then summed in a pairwise tree over the row groups (lane shuffles
// within a wave, LDS across waves) -- and the entry is stored in its format: fp32, bf16, packed bf16 + e4m3fn, or MXFP4 (one
// e8m0 scale per 32 channels, taken over 4 adjacent threads).  Splitting the rows
// keeps a 128-row HCA window from becoming a 128-deep dependent loop per thread.
// With few entries (decode: one per sequence) the channels are also split over
// gridDim.z blocks of d / gridDim.z channels each, so that the launch still spans
// a good part of the chip; each block recomputes the (cheap) window softmax.
// Decode steps with one logit per token take a one-wave kernel instead
// (k_compress_dec): the block returns at once when its token completes no entry;
// otherwise every lane loads its share of the window's logits and the wave reduces
// their maximum and sum with lane moves, each lane sums its rows with their final
// weights, and the row groups are added with lane moves as well -- no LDS and no
// barrier between the row loads and the store.
#include <type_traits>

#include "compress_dec.h"
#include "device.h"
#include "launch.h"

namespace csl {

struct CmpGeom {
    int TPR;  // threads per row (d / 8)
    int RG;   // row groups per entry
    int EPB;  // entries per block
};

__host__ __device__ inline int pow2_at_least(int v) {
    int w = 1;
    while (w < v) w <<= 1;
    return w;
}

// Long windows over wide rows (HCA's 128 rows of 512 channels) get 1024-thread
// blocks so that each row group walks only a few rows; otherwise 256 threads (the
// maximum step of the merge loops over the groups, so they stay at most 32).
__host__ __device__ inline int cmp_threads(int d, int win) {
    return d >= 256 && (d / 8) * pow2_at_least(win) >= 1024 ? 1024 : 256;
}

__host__ __device__ inline CmpGeom cmp_geom(int d, int win, int nt) {
    CmpGeom g;
    g.TPR = d / 8;
    int rg = nt / g.TPR;
    const int w2 = pow2_at_least(win);
    if (rg > w2) rg = w2;
    if (rg > 32) rg = 32;                  // the merge's maximum walks the groups one by one
    if (rg < 1) rg = 1;
    g.RG = rg;
    g.EPB = nt / (g.TPR * g.RG);
    if (g.EPB < 1) g.EPB = 1;
    return g;
}

template <int XF>
__device__ __forceinline__ void load8(const uint8_t* row, int c0, float* v) {
    if (XF == F32) {
        const float4 a = *(const float4*)(row + (int64_t)c0 * 4);
        const float4 b = *(const float4*)(row + (int64_t)c0 * 4 + 16);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        const u32x4 u = *(const u32x4*)(row + (int64_t)c0 * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_to_f32(u[i] & 0xffffu);
            v[2 * i + 1] = bf16_to_f32(u[i] >> 16);
        }
    }
}

// One block's share of a compression: channel part zi of gz (the grid's z index and
// extent for a single job; a fused launch of two jobs splits its z range between them).
template <int XF, int OF, bool ZC1, int CMP_NT>
__device__ __forceinline__ void compress_body(const CompressArgs& a, int zi, int gz) {
    const int win = a.overlap ? 2 * a.m : a.m;
    const int dt = a.d / gz;                            // channels of this block
    const CmpGeom G = cmp_geom(dt, win, CMP_NT);
    const int per_entry = G.TPR * G.RG;
    const int ep = threadIdx.x / per_entry;
    const int rg = (threadIdx.x / G.TPR) % G.RG;
    const int tr = threadIdx.x % G.TPR;
    const int c0 = zi * dt + tr * 8;
    const int b = blockIdx.y;
    const int64_t q = (int64_t)blockIdx.x * G.EPB + ep;
    bool active = ep < G.EPB && q < a.n_e;
    int64_t i;
    if (a.pos) {                                         // decode-time step: the entry token q completes
        const int64_t p = active ? a.pos[(int64_t)b * a.n_e + q] : -1;
        active = active && p >= 0 && (p + 1) % a.m == 0;
        i = active ? (p + 1) / a.m - 1 : 0;
    } else {
        i = a.e_begin + (active ? q : 0);
    }
    const int64_t p0 = (i + 1) * a.m - win;
    const int64_t xrb = (XF == F32 ? 4 * (int64_t)a.d : 2 * (int64_t)a.d) * a.x_roles;
    // raw row of window slot j: linear buffer or ring; a two-role row's current half
    // (slots j >= m) starts d values in
    auto xrow = [&](int jc) {
        int64_t row = p0 + jc - a.x_pos0;
        if (a.x_rows > 0) { row %= a.x_rows; if (row < 0) row += a.x_rows; }
        return row;
    };
    const int role_off = a.x_roles == 2 ? a.d : 0;
    constexpr int NC = ZC1 ? 1 : 8;   // softmax channels carried per thread

    float acc[8], mx[NC], den[NC];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) { mx[c] = -INFINITY; den[c] = 0.f; }

    if (active) {
        const uint8_t* xb = a.x + (int64_t)b * a.x_bstride;
        const float* zb = (const float*)((const uint8_t*)a.z + (int64_t)b * a.z_bstride);
        const int j0 = p0 < 0 ? (int)(-p0) : 0;
        const int jf = j0 + ((rg - j0) % G.RG + G.RG) % G.RG;   // this thread's first row
        // Rows in batches of CMP_RB: every load of a batch is issued before the first
        // softmax update (a row past the window re-reads the batch's first row and is
        // skipped), so a long window costs one memory round trip per batch rather than
        // per row; the updates run in the same row order as one row at a time.
        // (CMP_RB = 1 when no thread has a second row: the short CSA windows)
        auto rows = [&](auto rb_tag) {
        constexpr int CMP_RB = decltype(rb_tag)::value;
        for (int jb = jf; jb < win; jb += CMP_RB * G.RG) {
            float xv[CMP_RB][8], lg[CMP_RB][NC];
            bool ok[CMP_RB];
#pragma unroll
            for (int u = 0; u < CMP_RB; ++u) {
                const int jw = jb + u * G.RG;
                ok[u] = jw < win;
                const int jc = ok[u] ? jw : jb;
                const int64_t row = xrow(jc);
                load8<XF>(xb + row * xrb, c0 + (jc >= a.m ? role_off : 0), xv[u]);
                if constexpr (ZC1) {
                    lg[u][0] = zb[row] + a.bias[jc];
                } else {
                    const float* zr = zb + row * a.z_ch + c0;
                    const float* br = a.bias + (int64_t)jc * a.z_ch + c0;
#pragma unroll
                    for (int c = 0; c < 8; ++c) lg[u][c] = zr[c] + br[c];
                }
            }
#pragma unroll
            for (int u = 0; u < CMP_RB; ++u) {
                if (!ok[u]) continue;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    if (lg[u][c] > mx[c]) {
                        const float s = expf(mx[c] - lg[u][c]);
                        den[c] *= s;
                        if constexpr (ZC1) {
#pragma unroll
                            for (int cc = 0; cc < 8; ++cc) acc[cc] *= s;
                        } else {
                            acc[c] *= s;
                        }
                        mx[c] = lg[u][c];
                    }
                    const float e = expf(lg[u][c] - mx[c]);
                    den[c] += e;
                    if constexpr (ZC1) {
#pragma unroll
                        for (int cc = 0; cc < 8; ++cc) acc[cc] = fmaf(e, xv[u][cc], acc[cc]);
                    } else {
                        acc[c] = fmaf(e, xv[u][c], acc[c]);
                    }
                }
            }
        }
        };
        if (win <= G.RG) rows(std::integral_constant<int, 1>{});
        else rows(std::integral_constant<int, 4>{});
    }

    // ---- merge the RG row-group partials: every group rescales its (sum, weighted
    // sum) to the entry's maximum logit, then a pairwise tree over rg adds them (level
    // st joins group rg with rg + st).  The tree depends on RG only, so the result is
    // deterministic and independent of the channel split; row group 0 ends with the
    // entry's sums.  A level whose partner is in the same wave reads it by a lane
    // shuffle, otherwise through LDS.
    __shared__ float s_acc[CMP_NT * 8];
    __shared__ float s_den[CMP_NT * NC];
    float v[8];
    if (G.RG > 1) {
        float* s_mx = s_acc;                             // the maxima first, then the sums
        const int base = ep * per_entry + tr;            // row group 0 of this entry and channels
        const int ng = ep < G.EPB ? G.RG : 0;
#pragma unroll
        for (int c = 0; c < NC; ++c) s_mx[threadIdx.x * NC + c] = mx[c];
        __syncthreads();
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            float M = -INFINITY;
            for (int g = 0; g < ng; ++g) M = fmaxf(M, s_mx[(base + g * G.TPR) * NC + c]);
            const float f = mx[c] == -INFINITY ? 0.f : expf(mx[c] - M);
            den[c] *= f;
            if constexpr (ZC1) {
#pragma unroll
                for (int cc = 0; cc < 8; ++cc) acc[cc] *= f;
            } else {
                acc[c] *= f;
            }
        }
        __syncthreads();                                 // maxima read: s_acc reused below
        const bool tpr_pow2 = (G.TPR & (G.TPR - 1)) == 0;
        const int lane = (int)(threadIdx.x & 63);
        for (int st = 1; st < G.RG; st <<= 1) {          // block-uniform trip count
            const bool joins = ep < G.EPB && (rg & (2 * st - 1)) == 0 && rg + st < G.RG;
            float d2[NC], a2[8];
            if (tpr_pow2 && st * G.TPR < 64) {           // partner lane + st * TPR, same wave
                const int src = (lane + st * G.TPR) & 63;
#pragma unroll
                for (int c = 0; c < NC; ++c) d2[c] = __shfl(den[c], src, 64);
#pragma unroll
                for (int c = 0; c < 8; ++c) a2[c] = __shfl(acc[c], src, 64);
            } else {
#pragma unroll
                for (int c = 0; c < 8; ++c) s_acc[threadIdx.x * 8 + c] = acc[c];
#pragma unroll
                for (int c = 0; c < NC; ++c) s_den[threadIdx.x * NC + c] = den[c];
                __syncthreads();
                const int pt = joins ? threadIdx.x + st * G.TPR : threadIdx.x;   // group rg + st
#pragma unroll
                for (int c = 0; c < NC; ++c) d2[c] = s_den[pt * NC + c];
#pragma unroll
                for (int c = 0; c < 8; ++c) a2[c] = s_acc[pt * 8 + c];
                __syncthreads();                         // slots free for the next level
            }
            if (joins) {
#pragma unroll
                for (int c = 0; c < NC; ++c) den[c] += d2[c];
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[c] += a2[c];
            }
        }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = active ? acc[c] / den[ZC1 ? 0 : c] : 0.f;   // final in row group 0
    bool writer = active && rg == 0;

    // this entry's output row (and MXFP4 scale row)
    const int64_t orb = OF == F32 ? 4 * (int64_t)a.d : (OF == BF16 ? 2 * (int64_t)a.d :
                        (OF == KV_PACKED ? 2 * (int64_t)a.r + (a.d - a.r) : (int64_t)a.d / 2));
    uint8_t* orow = nullptr;
    uint8_t* osc = nullptr;
    if (!a.pos) {
        orow = a.out + (int64_t)b * a.out_bstride + q * orb;
        if (OF == MXFP4) osc = a.out_scales + (int64_t)b * a.sc_bstride + q * (a.d / 32);
    } else if (!a.bt) {
        writer = writer && i < a.n_cap;
        orow = a.out + (int64_t)b * a.out_bstride + i * orb;
        if (OF == MXFP4) osc = a.out_scales + (int64_t)b * a.sc_bstride + i * (a.d / 32);
    } else {
        const int64_t lb = i / a.epb;
        const int32_t blk = (writer && lb < a.bt_stride) ? a.bt[(int64_t)b * a.bt_stride + lb] : -1;
        writer = writer && blk >= 0 && blk < a.n_blocks;
        const int64_t off = i - lb * a.epb;
        orow = a.out + (int64_t)blk * a.blk_bytes + off * orb;
        if (OF == MXFP4) osc = a.out_scales + (int64_t)blk * a.sblk_bytes + off * (a.d / 32);
    }

    if (OF == F32) {
        if (writer) {
            float* o = (float*)orow + c0;
            *(float4*)o = make_float4(v[0], v[1], v[2], v[3]);
            *(float4*)(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
        }
    } else if (OF == BF16) {
        if (writer) {
            u32x4 o;
#pragma unroll
            for (int k2 = 0; k2 < 4; ++k2) o[k2] = f32_to_bf16_rne(v[2 * k2]) | (f32_to_bf16_rne(v[2 * k2 + 1]) << 16);
            *(u32x4*)(orow + (int64_t)c0 * 2) = o;
        }
    } else if (OF == KV_PACKED) {
        if (writer) {
            uint8_t* row = orow;
            if (c0 < a.r) {
                u32x4 o;
#pragma unroll
                for (int k2 = 0; k2 < 4; ++k2)
                    o[k2] = f32_to_bf16_rne(v[2 * k2]) | (f32_to_bf16_rne(v[2 * k2 + 1]) << 16);
                *(u32x4*)(row + 2 * c0) = o;
            } else {
                u32x2 o;
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2)
                    o[k2] = f32_to_e4m3_rne_sat(v[4 * k2]) | (f32_to_e4m3_rne_sat(v[4 * k2 + 1]) << 8) |
                            (f32_to_e4m3_rne_sat(v[4 * k2 + 2]) << 16) | (f32_to_e4m3_rne_sat(v[4 * k2 + 3]) << 24);
                *(u32x2*)(row + 2 * a.r + (c0 - a.r)) = o;
            }
        }
    } else {  // MXFP4: 4 adjacent threads hold one 32-channel block
        float am = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) am = fmaxf(am, fabsf(v[c]));
        am = fmaxf(am, shfl_xor(am, 1));
        am = fmaxf(am, shfl_xor(am, 2));
        const int e = mx_block_exponent(am);
        uint32_t w = 0;
#pragma unroll
        for (int c = 0; c < 8; ++c) w |= f32_to_e2m1_rne_sat(ldexpf(v[c], -e)) << (4 * c);
        if (writer) {
            *(uint32_t*)(orow + c0 / 2) = w;
            if ((c0 & 31) == 0) osc[c0 / 32] = (uint8_t)(e + 127);
        }
    }
}

template <int XF, int OF, bool ZC1, int CMP_NT>
__global__ void __launch_bounds__(CMP_NT) k_compress(CompressArgs a) {
    compress_body<XF, OF, ZC1, CMP_NT>(a, (int)blockIdx.z, (int)gridDim.z);
}

// Two compressions of the same new tokens in one launch (a CSA layer's KV entry and its
// indexer key): z indices [0, gz0) run the first job, [gz0, gz0 + gz1) the second.
template <int OF0, int OF1>
__global__ void __launch_bounds__(256) k_compress_pair(CompressArgs a0, CompressArgs a1, int gz0, int gz1) {
    if ((int)blockIdx.z < gz0) compress_body<BF16, OF0, true, 256>(a0, (int)blockIdx.z, gz0);
    else compress_body<BF16, OF1, true, 256>(a1, (int)blockIdx.z - gz0, gz1);
}

// ---- decode-time compression, one logit per token: one wave per block ----------------
template <int OF>
__global__ void __launch_bounds__(64) k_compress_dec(CompressArgs a) {
    compress_dec_body<OF>(a, blockIdx.x, (int)blockIdx.y, (int)blockIdx.z, (int)gridDim.z);
}

template <int OF0, int OF1>
__global__ void __launch_bounds__(64) k_compress_dec_pair(CompressArgs a0, CompressArgs a1, int gz0, int gz1) {
    if ((int)blockIdx.z < gz0) compress_dec_body<OF0>(a0, blockIdx.x, (int)blockIdx.y, (int)blockIdx.z, gz0);
    else compress_dec_body<OF1>(a1, blockIdx.x, (int)blockIdx.y, (int)blockIdx.z - gz0, gz1);
}

// the decode kernel's shape: bf16 rows, one logit per token, a window of at most 256
// slots, and a channel split into parts of 32 .. 512 channels
static bool dec_shape(const CompressArgs& a, int gz) {
    const int win = a.overlap ? 2 * a.m : a.m;
    const int dt = a.d / gz;
    return a.pos && a.x_fmt == BF16 && a.z_ch == 1 && win <= 256 && a.out_fmt != F32 && dt >= 32 && dt <= 512 &&
           (dt & (dt - 1)) == 0;
}

// channel splits: halve the block's channels (keeping whole 32-channel groups)
// while the launch has fewer than 256 entry blocks
static int cmp_splits(const CompressArgs& a) {
    int gz = 1;
    while (a.n_e * (int64_t)a.B * gz < 256 && a.d / (2 * gz) >= 32 && (a.d / (2 * gz)) % 32 == 0) gz *= 2;
    return gz;
}

template <int XF, int OF, int NT>
static hipError_t launch_c3(const CompressArgs& a, hipStream_t s, int gz) {
    const CmpGeom G = cmp_geom(a.d / gz, a.overlap ? 2 * a.m : a.m, NT);
    dim3 grid((unsigned)((a.n_e + G.EPB - 1) / G.EPB), (unsigned)a.B, (unsigned)gz);
    if (a.z_ch == 1)
        hipLaunchKernelGGL((k_compress<XF, OF, true, NT>), grid, dim3(NT), 0, s, a);
    else
        hipLaunchKernelGGL((k_compress<XF, OF, false, NT>), grid, dim3(NT), 0, s, a);
    return hipGetLastError();
}

template <int XF, int OF>
static hipError_t launch_c2(const CompressArgs& a, hipStream_t s) {
    const int gz = cmp_splits(a);
    if constexpr (XF == BF16 && OF != F32) {
        if (dec_shape(a, gz)) {
            hipLaunchKernelGGL((k_compress_dec<OF>), dim3((unsigned)a.n_e, (unsigned)a.B, (unsigned)gz), dim3(64), 0, s, a);
            return hipGetLastError();
        }
    }
    return cmp_threads(a.d / gz, a.overlap ? 2 * a.m : a.m) == 1024 ? launch_c3<XF, OF, 1024>(a, s, gz)
                                                                    : launch_c3<XF, OF, 256>(a, s, gz);
}

template <int XF>
static hipError_t launch_c1(const CompressArgs& a, hipStream_t s) {
    switch (a.out_fmt) {
    case F32: return launch_c2<XF, F32>(a, s);
    case BF16: return launch_c2<XF, BF16>(a, s);
    case KV_PACKED: return launch_c2<XF, KV_PACKED>(a, s);
    default: return launch_c2<XF, MXFP4>(a, s);
    }
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t s) {
    if (a.n_e <= 0 || a.B <= 0) return hipSuccess;
    return a.x_fmt == F32 ? launch_c1<F32>(a, s) : launch_c1<BF16>(a, s);
}

// The decode pair the indexer's scoring kernel can compress before it scores: one-wave
// shapes for both jobs, a packed KV entry then an MXFP4 or bf16 key.  Sets each job's
// channel split.
bool compress_pair_in_index(const CompressArgs& kv, const CompressArgs& key, int& gz_kv, int& gz_key) {
    gz_kv = cmp_splits(kv);
    gz_key = cmp_splits(key);
    return kv.B == key.B && kv.n_e == key.n_e && dec_shape(kv, gz_kv) && dec_shape(key, gz_key) &&
           kv.out_fmt == KV_PACKED && (key.out_fmt == MXFP4 || key.out_fmt == BF16);
}

// The decode job the packed-row attention kernel can compress before it attends: the
// one-wave shape, a packed KV entry.  Sets the channel split.
bool compress_in_attend(const CompressArgs& kv, int& gz) {
    gz = cmp_splits(kv);
    return dec_shape(kv, gz) && kv.out_fmt == KV_PACKED;
}

// Both jobs in one launch when they take a fused kernel's shape (bf16 raw rows, one
// logit per token, a packed KV entry plus an MXFP4 or bf16 key): the one-wave decode
// kernel, else the general one with 256-thread blocks; otherwise one launch after the
// other.
hipError_t launch_compress_pair(const CompressArgs& a0, const CompressArgs& a1, hipStream_t s) {
    if (a0.B <= 0 || a0.n_e <= 0) return hipSuccess;
    const int gz0 = cmp_splits(a0), gz1 = cmp_splits(a1);
    const int w0 = a0.overlap ? 2 * a0.m : a0.m, w1 = a1.overlap ? 2 * a1.m : a1.m;
    if (a0.B == a1.B && a0.n_e == a1.n_e && dec_shape(a0, gz0) && dec_shape(a1, gz1) && a0.out_fmt == KV_PACKED &&
        (a1.out_fmt == MXFP4 || a1.out_fmt == BF16)) {
        const dim3 grid((unsigned)a0.n_e, (unsigned)a0.B, (unsigned)(gz0 + gz1));
        if (a1.out_fmt == MXFP4)
            hipLaunchKernelGGL((k_compress_dec_pair<KV_PACKED, MXFP4>), grid, dim3(64), 0, s, a0, a1, gz0, gz1);
        else
            hipLaunchKernelGGL((k_compress_dec_pair<KV_PACKED, BF16>), grid, dim3(64), 0, s, a0, a1, gz0, gz1);
        return hipGetLastError();
    }
    const bool shape = a0.B == a1.B && a0.n_e == a1.n_e && a0.x_fmt == BF16 && a1.x_fmt == BF16 && a0.z_ch == 1 &&
                       a1.z_ch == 1 && cmp_threads(a0.d / gz0, w0) == 256 && cmp_threads(a1.d / gz1, w1) == 256 &&
                       a0.out_fmt == KV_PACKED && (a1.out_fmt == MXFP4 || a1.out_fmt == BF16);
    if (!shape) {
        hipError_t e = launch_compress(a0, s);
        return e != hipSuccess ? e : launch_compress(a1, s);
    }
    const CmpGeom G0 = cmp_geom(a0.d / gz0, w0, 256), G1 = cmp_geom(a1.d / gz1, w1, 256);
    const int64_t x0 = (a0.n_e + G0.EPB - 1) / G0.EPB, x1 = (a1.n_e + G1.EPB - 1) / G1.EPB;
    const dim3 grid((unsigned)(x0 > x1 ? x0 : x1), (unsigned)a0.B, (unsigned)(gz0 + gz1));
    if (a1.out_fmt == MXFP4)
        hipLaunchKernelGGL((k_compress_pair<KV_PACKED, MXFP4>), grid, dim3(256), 0, s, a0, a1, gz0, gz1);
    else
        hipLaunchKernelGGL((k_compress_pair<KV_PACKED, BF16>), grid, dim3(256), 0, s, a0, a1, gz0, gz1);
    return hipGetLastError();
}

}  // namespace csl
