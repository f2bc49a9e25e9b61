// compress.hip -- token compression of raw KV rows into compressed entries.
//
// Method: x-techcon article on DeepSeek-V4, section 2, CSA step 1 -- every m raw
// tokens become one entry: a learned weight per raw token plus a position bias,
// normalised by a softmax, then a weighted sum; adjacent blocks overlap.  The HCA
// subsection applies the same operator at m' = 128.  Window geometry (a reading):
// entry i pools raw positions (i+1)m-win .. (i+1)m-1, win = 2m with overlap, m
// without; positions < 0 are left out of the softmax.
//
// Streaming, HBM-bound kernel: one thread owns 4 consecutive channels of one entry,
// walks the window once with an online softmax (no second pass over the rows), and
// stores the entry in its storage format (fp32, bf16, packed bf16+e4m3fn, or MXFP4
// with one e8m0 scale per 32 channels).  d/4 consecutive threads form one entry, so
// each raw row is read as contiguous 8- or 16-byte pieces by adjacent lanes.
#include "device.h"
#include "launch.h"

namespace csl {

template <int XF, int OF, bool ZC1>
__global__ void __launch_bounds__(256) k_compress(CompressArgs a) {
    const int TPE = a.d >> 2;                 // threads per entry
    const int EPB = 256 / TPE;                // entries per block
    const int eg = threadIdx.x / TPE;
    const int c0 = (threadIdx.x - eg * TPE) * 4;
    const int b = blockIdx.y;
    const int64_t q = (int64_t)blockIdx.x * EPB + eg;
    const bool active = eg < EPB && q < a.n_e;
    const int64_t i = a.e_begin + (active ? q : 0);
    const int win = a.overlap ? 2 * a.m : a.m;
    const int64_t p0 = (i + 1) * a.m - win;
    const int64_t xrb = XF == F32 ? 4 * (int64_t)a.d : 2 * (int64_t)a.d;

    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    float den[4] = {0.f, 0.f, 0.f, 0.f};
    if (active) {
        const uint8_t* xb = a.x + (int64_t)b * a.x_bstride;
        const float* zb = (const float*)((const uint8_t*)a.z + (int64_t)b * a.z_bstride);
        for (int jw = p0 < 0 ? (int)(-p0) : 0; jw < win; ++jw) {
            const int64_t row = p0 + jw - a.x_pos0;
            float lg[4];
            if (ZC1) {
                const float v = zb[row] + a.bias[jw];
                lg[0] = lg[1] = lg[2] = lg[3] = v;
            } else {
                const float4 zz = *(const float4*)(zb + row * a.z_ch + c0);
                const float4 bb = *(const float4*)(a.bias + (int64_t)jw * a.z_ch + c0);
                lg[0] = zz.x + bb.x; lg[1] = zz.y + bb.y; lg[2] = zz.z + bb.z; lg[3] = zz.w + bb.w;
            }
            float xv[4];
            if (XF == F32) {
                const float4 v = *(const float4*)(xb + row * xrb + (int64_t)c0 * 4);
                xv[0] = v.x; xv[1] = v.y; xv[2] = v.z; xv[3] = v.w;
            } else {
                const uint2 v = *(const uint2*)(xb + row * xrb + (int64_t)c0 * 2);
                xv[0] = bf16_to_f32(v.x & 0xffffu); xv[1] = bf16_to_f32(v.x >> 16);
                xv[2] = bf16_to_f32(v.y & 0xffffu); xv[3] = bf16_to_f32(v.y >> 16);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (lg[c] > mx[c]) {
                    const float s = expf(mx[c] - lg[c]);
                    den[c] *= s;
                    acc[c] *= s;
                    mx[c] = lg[c];
                }
                const float e = expf(lg[c] - mx[c]);
                den[c] += e;
                acc[c] = fmaf(e, xv[c], acc[c]);
            }
        }
    }
    float v[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = active ? acc[c] / den[c] : 0.0f;

    uint8_t* ob = a.out + (int64_t)b * a.out_bstride;
    if (OF == F32) {
        if (active) *(float4*)(ob + q * 4 * (int64_t)a.d + (int64_t)c0 * 4) = make_float4(v[0], v[1], v[2], v[3]);
    } else if (OF == BF16) {
        if (active) {
            uint2 o;
            o.x = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
            o.y = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
            *(uint2*)(ob + q * 2 * (int64_t)a.d + (int64_t)c0 * 2) = o;
        }
    } else if (OF == KV_PACKED) {
        if (active) {
            const int64_t rb = 2 * (int64_t)a.r + (a.d - a.r);
            uint8_t* row = ob + q * rb;
            if (c0 < a.r) {
                uint2 o;
                o.x = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
                o.y = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
                *(uint2*)(row + 2 * c0) = o;
            } else {
                const uint32_t o = f32_to_e4m3_rne_sat(v[0]) | (f32_to_e4m3_rne_sat(v[1]) << 8) |
                                   (f32_to_e4m3_rne_sat(v[2]) << 16) | (f32_to_e4m3_rne_sat(v[3]) << 24);
                *(uint32_t*)(row + 2 * a.r + (c0 - a.r)) = o;
            }
        }
    } else {  // MXFP4: 8 adjacent threads hold one 32-channel block
        float am = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
        am = fmaxf(am, shfl_xor(am, 1));
        am = fmaxf(am, shfl_xor(am, 2));
        am = fmaxf(am, shfl_xor(am, 4));
        const int e = mx_block_exponent(am);
        uint32_t cd[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) cd[c] = f32_to_e2m1_rne_sat(ldexpf(v[c], -e));
        if (active) {
            uint8_t* row = ob + q * (int64_t)(a.d / 2);
            *(uint16_t*)(row + c0 / 2) = (uint16_t)(cd[0] | (cd[1] << 4) | (cd[2] << 8) | (cd[3] << 12));
            if ((c0 & 31) == 0) a.out_scales[(int64_t)b * a.sc_bstride + q * (a.d / 32) + c0 / 32] = (uint8_t)(e + 127);
        }
    }
}

template <int XF, int OF>
static hipError_t launch_c2(const CompressArgs& a, hipStream_t s) {
    const int TPE = a.d / 4, EPB = 256 / TPE;
    dim3 grid((unsigned)((a.n_e + EPB - 1) / EPB), (unsigned)a.B);
    if (a.z_ch == 1)
        hipLaunchKernelGGL((k_compress<XF, OF, true>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((k_compress<XF, OF, false>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
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

}  // namespace csl
