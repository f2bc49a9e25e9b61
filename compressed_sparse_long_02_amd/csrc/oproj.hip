// oproj.hip -- grouped output projection after the attention.
//
// Method: x-techcon article on DeepSeek-V4, section 2, HCA subsection (both
// branches project their outputs group by group to cut the cost of the output
// projection); CSDN explainer, table of attention details ("Grouped Output
// Projection": the heads' outputs are first compressed per group, then combined).
// Group g of G maps the concatenated outputs of its H/G heads (K = (H/G) * d values
// per token, contiguous in the [token][head][dim] attention output) through its own
// R x K matrix:  y[t][g*R + n] = sum_k x[t][g*K + k] * w[g][n][k].  The one common
// projection that follows is the same operation with G = 1.
//
// Design (gfx950), bf16 operands, fp32 accumulation (16x16x32 bf16 MFMA):
//  * few tokens (decode, M <= 64): the weights are the traffic.  A block owns 32
//    output columns of one group and every token; its 8 waves (4 when K is not a
//    multiple of 256) split K and stream their part of the 32 weight rows straight
//    from HBM into MFMA B fragments (each lane 16 contiguous bytes of one row, up to
//    eight k-steps in flight), the token rows come from L2; the parts' partial sums
//    are added through LDS in a fixed order.
//  * many tokens (prefill): a classic LDS-tiled GEMM, 128 x 128 output tiles, K in
//    steps of 64 through double-buffered LDS, 4 waves of 64 x 64.
#include "device.h"
#include "launch.h"

namespace csl {

constexpr int GP_NT = 256;

template <int OUTF>
__device__ __forceinline__ void gp_store(uint8_t* out, int64_t ld, int64_t row, int64_t col, float v) {
    if (OUTF == F32) ((float*)out)[row * ld + col] = v;
    else ((uint16_t*)out)[row * ld + col] = (uint16_t)f32_to_bf16_rne(v);
}

// ---- few tokens: MT row tiles of 16 (M <= 16 * MT), 32 columns per block, NW waves ----
// each taking 1/NW of K, KU k-steps of loads in flight per wave
template <int OUTF, int MT, int NW>
__global__ void __launch_bounds__(64 * NW) k_gproj_skinny(GprojArgs a) {
    constexpr int KU = MT == 1 ? 8 : (MT == 2 ? 4 : 2);
    __shared__ v4f part[NW][MT * 2][64];
    const int n0 = blockIdx.x * 32, g = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, gq = lane >> 4, col = lane & 15;
    const int kq = a.K / NW;                             // this wave's K range [wv*kq, (wv+1)*kq)
    const int64_t xld = (int64_t)a.G * a.K;
    const uint16_t* xg = (const uint16_t*)a.x + (int64_t)g * a.K + wv * kq + 8 * gq;
    const uint16_t* wg = (const uint16_t*)a.w + ((int64_t)g * a.R + n0) * a.K + wv * kq + 8 * gq;
    const uint16_t* xr[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int row = mt * 16 + col;
        xr[mt] = xg + (int64_t)(row < a.M ? row : a.M - 1) * xld;
    }
    const uint16_t* wr0 = wg + (int64_t)col * a.K;
    const uint16_t* wr1 = wr0 + (int64_t)16 * a.K;
    v4f acc[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt][0] = acc[mt][1] = v4f{0.f, 0.f, 0.f, 0.f};
    const int nks = kq / 32;
    for (int ks = 0; ks < nks; ks += KU) {
        u32x4 A[KU][MT], B0[KU], B1[KU];
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int kk = (ks + u < nks ? ks + u : nks - 1) * 32;   // past the end: re-read the last step
            B0[u] = ld_global<u32x4>(wr0 + kk);
            B1[u] = ld_global<u32x4>(wr1 + kk);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) A[u][mt] = ld_global<u32x4>(xr[mt] + kk);
        }
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            if (ks + u >= nks) break;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                acc[mt][0] = mfma_bf16(A[u][mt], B0[u], acc[mt][0]);
                acc[mt][1] = mfma_bf16(A[u][mt], B1[u], acc[mt][1]);
            }
        }
    }
    // the NW K ranges, added in wave order
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        part[wv][2 * mt][lane] = acc[mt][0];
        part[wv][2 * mt + 1][lane] = acc[mt][1];
    }
    __syncthreads();
    // C layout: lane (gq, col) holds rows 4*gq + i of the 16-row tile, column col
    for (int t = wv; t < MT * 2; t += NW) {
        v4f s = part[0][t][lane];
#pragma unroll
        for (int x = 1; x < NW; ++x) s += part[x][t][lane];
        const int mt = t >> 1, nt = t & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = mt * 16 + 4 * gq + i;
            if (row < a.M) gp_store<OUTF>(a.out, (int64_t)a.G * a.R, row, (int64_t)g * a.R + n0 + 16 * nt + col, s[i]);
        }
    }
}

// ---- many tokens: 128 x 128 tiles, K steps of 64 through double-buffered LDS -------
constexpr int GT_BM = 128, GT_BN = 128, GT_BK = 64, GT_STR = GT_BK + 8;   // LDS row: 64 bf16 + 16 B pad

template <int OUTF>
__global__ void __launch_bounds__(GP_NT, 2) k_gproj_tiled(GprojArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][GT_BM * GT_STR];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][GT_BN * GT_STR];
    const int n0 = blockIdx.x * GT_BN, m0 = blockIdx.y * GT_BM, g = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, gq = lane >> 4, col = lane & 15;
    const int wm = (wv >> 1) * 64, wn = (wv & 1) * 64;   // this wave's 64 x 64 quadrant
    const int64_t xld = (int64_t)a.G * a.K;
    const uint16_t* xg = (const uint16_t*)a.x + (int64_t)g * a.K;
    const uint16_t* wg = (const uint16_t*)a.w + ((int64_t)g * a.R + n0) * a.K;
    // global -> registers: 16-byte chunk c = tid + 256 j of a tile: row c / 8, piece c % 8
    u32x4 ra[4], rb[4];
    auto load = [&](int kt) {
        const int k0 = kt * GT_BK;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = tid + GP_NT * j, rr = c >> 3, pc = c & 7;
            const int row = m0 + rr < a.M ? m0 + rr : a.M - 1;    // rows past M re-read the last one
            ra[j] = ld_global<u32x4>(xg + (int64_t)row * xld + k0 + 8 * pc);
            rb[j] = ld_global<u32x4>(wg + (int64_t)rr * a.K + k0 + 8 * pc);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = tid + GP_NT * j, rr = c >> 3, pc = c & 7;
            *(u32x4*)(&As[buf][rr * GT_STR + 8 * pc]) = ra[j];
            *(u32x4*)(&Bs[buf][rr * GT_STR + 8 * pc]) = rb[j];
        }
    };
    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    const int nkt = a.K / GT_BK;
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nkt) load(kt + 1);                  // in flight during this tile's MFMAs
#pragma unroll
        for (int ks = 0; ks < GT_BK / 32; ++ks) {
            u32x4 fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                fa[i] = *(const u32x4*)(&As[buf][(wm + 16 * i + col) * GT_STR + ks * 32 + 8 * gq]);
                fb[i] = *(const u32x4*)(&Bs[buf][(wn + 16 * i + col) * GT_STR + ks * 32 + 8 * gq]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(fa[i], fb[j], acc[i][j]);
        }
        if (kt + 1 < nkt) {
            store(buf ^ 1);                              // the other buffer: its readers finished last step
            __syncthreads();
        }
    }
    const int64_t ld = (int64_t)a.G * a.R;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = m0 + wm + 16 * i + 4 * gq + e;
                if (row < a.M) gp_store<OUTF>(a.out, ld, row, (int64_t)g * a.R + n0 + wn + 16 * j + col, acc[i][j][e]);
            }
}

template <int OUTF>
static hipError_t launch_gp(const GprojArgs& a, hipStream_t s) {
    if (a.M <= 64) {
        const dim3 grid((unsigned)(a.R / 32), (unsigned)a.G);
        if (a.K % 256 == 0) {                            // 8 waves, K / 8 each
            if (a.M <= 16) hipLaunchKernelGGL((k_gproj_skinny<OUTF, 1, 8>), grid, dim3(512), 0, s, a);
            else if (a.M <= 32) hipLaunchKernelGGL((k_gproj_skinny<OUTF, 2, 8>), grid, dim3(512), 0, s, a);
            else hipLaunchKernelGGL((k_gproj_skinny<OUTF, 4, 8>), grid, dim3(512), 0, s, a);
        } else {
            if (a.M <= 16) hipLaunchKernelGGL((k_gproj_skinny<OUTF, 1, 4>), grid, dim3(256), 0, s, a);
            else if (a.M <= 32) hipLaunchKernelGGL((k_gproj_skinny<OUTF, 2, 4>), grid, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((k_gproj_skinny<OUTF, 4, 4>), grid, dim3(256), 0, s, a);
        }
    } else {
        const dim3 grid((unsigned)(a.R / GT_BN), (unsigned)((a.M + GT_BM - 1) / GT_BM), (unsigned)a.G);
        hipLaunchKernelGGL((k_gproj_tiled<OUTF>), grid, dim3(GP_NT), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_grouped_out_proj(const GprojArgs& a, hipStream_t s) {
    if (a.M <= 0) return hipSuccess;
    return a.out_fmt == F32 ? launch_gp<F32>(a, s) : launch_gp<BF16>(a, s);
}

}  // namespace csl
