// compress_dec.h -- one wave's decode-time compression of a completed entry.
//
// Method: x-techcon article on DeepSeek-V4, section 2, CSA step 1 (a learned weight per
// raw token plus a position bias, a softmax over the overlapping window, the weighted
// sum) and the HCA subsection (the same at m' = 128).  Shared by the compression
// kernels (one wave per block) and the indexer's scoring kernel, whose waves compress a
// CSA layer's new entry and indexer key before they score.
#pragma once

#include "device.h"
#include "launch.h"

namespace csl {

// One wave: the entry token q of sequence b completes (if any), channels zi*dt .. +dt.
// Every lane of the wave takes window slots l, l+64, .. for the softmax maximum and sum
// (wave reductions, no LDS); lane (g, tr) then sums rows g, g+RG, .. of its 8 channels
// with their final weights, and the RG row groups are added by lane moves.
template <int OF>
__device__ __forceinline__ void compress_dec_body(const CompressArgs& a, int64_t q, int b, int zi, int gz) {
    const int win = a.overlap ? 2 * a.m : a.m;
    const int dt = a.d / gz;
    const int TPR = dt / 8;                       // 4 .. 64, a power of two
    const int RG = 64 / TPR;
    const int lane = (int)(threadIdx.x & 63);
    const int tr = lane & (TPR - 1), g = lane / TPR;
    const int c0 = zi * dt + tr * 8;
    const int p = a.pos[(int64_t)b * a.n_e + q];
    if (p < 0 || (p + 1) % a.m != 0) return;      // no entry completes (uniform)
    const int64_t i = (p + 1) / a.m - 1;
    const int64_t p0 = (i + 1) * a.m - win;
    const int j0 = p0 < 0 ? (int)(-p0) : 0;
    const uint8_t* xb = a.x + (int64_t)b * a.x_bstride;
    const float* zb = (const float*)((const uint8_t*)a.z + (int64_t)b * a.z_bstride);
    const int64_t xrb = 2 * (int64_t)a.d * a.x_roles;
    const int role_off = a.x_roles == 2 ? a.d : 0;
    // raw row of window slot j: a ring holds at least win rows, so one reduction of the
    // window's first row suffices
    int64_t rbase = p0 - a.x_pos0;
    if (a.x_rows > 0) { rbase %= a.x_rows; if (rbase < 0) rbase += a.x_rows; }
    auto xrow = [&](int j) {
        const int64_t row = rbase + j;
        return (a.x_rows > 0 && row >= a.x_rows) ? row - a.x_rows : row;
    };
    // the window's logits (slots l, l+64, ..), then this lane's first eight rows (all of its
    // rows when win <= 8 RG) -- issued before the reductions need the logits, so that the
    // logits and the rows are one memory round trip
    // (every load from a clamped slot, and a slot outside the window masked by adding -inf
    // rather than by a select: the compiler turns a select of a load into a branch around
    // the load and waits for it inside the branch, one round trip after another)
    float lgw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int j = lane + 64 * u;
        const int jc = j < j0 ? j0 : (j < win ? j : win - 1);
        lgw[u] = (zb[xrow(jc)] + a.bias[jc]) + ((j >= j0 && j < win) ? 0.f : -INFINITY);
    }
    const int jf = g + ((j0 - g + RG - 1) / RG) * RG * (j0 > g);
    u32x4 xr[8];                                        // raw bf16 rows, widened at their FMAs
    float e[8];
    auto load_rows = [&](int jb) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = jb + u * RG;
            const bool ok = j < win;
            const int jc = ok ? j : jb;
            const int64_t row = xrow(jc);
            xr[u] = *(const u32x4*)(xb + row * xrb + 2 * (int64_t)(c0 + (jc >= a.m ? role_off : 0)));
            e[u] = (zb[row] + a.bias[jc]) + (ok ? 0.f : -INFINITY);
        }
    };
    if (jf < win) load_rows(jf);
    float M = fmaxf(fmaxf(lgw[0], lgw[1]), fmaxf(lgw[2], lgw[3]));
    M = cross4_max(row16_max(M));
    float S = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) S += lgw[u] == -INFINITY ? 0.f : expf(lgw[u] - M);
    S = cross4_sum(row16_sum(S));
    // this lane's rows with their final weights, eight loads in flight at a time
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.f;
    for (int jb = jf; jb < win; jb += 8 * RG) {
        if (jb > jf) load_rows(jb);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float w = e[u] == -INFINITY ? 0.f : expf(e[u] - M);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] = fmaf(w, bf16_to_f32(xr[u][i] & 0xffffu), acc[2 * i]);
                acc[2 * i + 1] = fmaf(w, bf16_to_f32(xr[u][i] >> 16), acc[2 * i + 1]);
            }
        }
    }
    // add the row groups: rotations within 16-lane rows, then the row swaps
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        float x = acc[c];
        if (TPR <= 4) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));
        if (TPR <= 8) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
        if (TPR <= 16) {
            const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
            x = __uint_as_float(s[0]) + __uint_as_float(s[1]);
        }
        if (TPR <= 32) {
            const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
            x = __uint_as_float(s[0]) + __uint_as_float(s[1]);
        }
        acc[c] = x;
    }
    float v[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = acc[c] / S;
    bool writer = g == 0;
    const int64_t orb = OF == BF16 ? 2 * (int64_t)a.d :
                        (OF == KV_PACKED ? 2 * (int64_t)a.r + (a.d - a.r) : (int64_t)a.d / 2);
    uint8_t* orow;
    uint8_t* osc = nullptr;
    if (!a.bt) {
        writer = writer && i < a.n_cap;
        orow = a.out + (int64_t)b * a.out_bstride + i * orb;
        if (OF == MXFP4) osc = a.out_scales + (int64_t)b * a.sc_bstride + i * (a.d / 32);
    } else {
        const int64_t lb = i / a.epb;
        const int32_t blk = lb < a.bt_stride ? a.bt[(int64_t)b * a.bt_stride + lb] : -1;
        writer = writer && blk >= 0 && blk < a.n_blocks;
        const int64_t off = i - lb * a.epb;
        orow = a.out + (int64_t)blk * a.blk_bytes + off * orb;
        if (OF == MXFP4) osc = a.out_scales + (int64_t)blk * a.sblk_bytes + off * (a.d / 32);
    }
    if (OF == BF16) {
        if (writer) {
            u32x4 o;
#pragma unroll
            for (int k2 = 0; k2 < 4; ++k2) o[k2] = f32_to_bf16_rne(v[2 * k2]) | (f32_to_bf16_rne(v[2 * k2 + 1]) << 16);
            *(u32x4*)(orow + (int64_t)c0 * 2) = o;
        }
    } else if (OF == KV_PACKED) {
        if (writer) {
            if (c0 < a.r) {
                u32x4 o;
#pragma unroll
                for (int k2 = 0; k2 < 4; ++k2)
                    o[k2] = f32_to_bf16_rne(v[2 * k2]) | (f32_to_bf16_rne(v[2 * k2 + 1]) << 16);
                *(u32x4*)(orow + 2 * c0) = o;
            } else {
                u32x2 o;
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2)
                    o[k2] = f32_to_e4m3_rne_sat(v[4 * k2]) | (f32_to_e4m3_rne_sat(v[4 * k2 + 1]) << 8) |
                            (f32_to_e4m3_rne_sat(v[4 * k2 + 2]) << 16) | (f32_to_e4m3_rne_sat(v[4 * k2 + 3]) << 24);
                *(u32x2*)(orow + 2 * a.r + (c0 - a.r)) = o;
            }
        }
    } else {  // MXFP4: lanes tr .. tr+3 (aligned) hold one 32-channel block
        float am = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) am = fmaxf(am, fabsf(v[c]));
        am = fmaxf(am, shfl_xor(am, 1));
        am = fmaxf(am, shfl_xor(am, 2));
        const int ex = mx_block_exponent(am);
        uint32_t w = 0;
#pragma unroll
        for (int c = 0; c < 8; ++c) w |= f32_to_e2m1_rne_sat(ldexpf(v[c], -ex)) << (4 * c);
        if (writer) {
            *(uint32_t*)(orow + c0 / 2) = w;
            if ((c0 & 31) == 0) osc[c0 / 32] = (uint8_t)(ex + 127);
        }
    }
}

}  // namespace csl
