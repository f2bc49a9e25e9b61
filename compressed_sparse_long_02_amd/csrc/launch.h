// launch.h -- argument blocks and launchers of the HIP kernels (internal; the
// public C ABI in include/csl.h validates arguments and calls these).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csl {

constexpr int IDX_SLOT_W = 2048 + 8;   // words per slice histogram list: count, then <= 2048 entries

struct CompressArgs {
    const uint8_t* x; int x_fmt; int64_t x_bstride; int64_t x_pos0; int64_t n_tok;
    const float* z; int z_ch; int64_t z_bstride;
    const float* bias;
    int B, d, r, m, overlap; int64_t e_begin, n_e;
    uint8_t* out; int out_fmt; uint8_t* out_scales; int64_t out_bstride, sc_bstride;
};

struct IndexArgs {
    const uint8_t* qi; int qi_fmt; const uint8_t* qi_scales; const float* w;
    const uint8_t* ki; int ki_fmt; const uint8_t* ki_scales; int64_t ki_bstride, ks_bstride;
    const int32_t* q_pos;
    int B, Tq, H_I, d_I, m; int64_t n_cap; int k;
    int32_t* out_idx; float* out_score;
    // plan
    int S;          // keys per slice (power of two in [512, 16384])
    int nslices;    // slices per query (<= 1024)
    int spb;        // split path: slices per filter block
    // rows of the split (nslices > 1) and dense paths, in the workspace
    int64_t sstride;     // row stride (n_cap rounded up to a multiple of 4)
    uint32_t* scores;    // order-preserving score keys: split [B*Tq][sstride], dense [B][Tc][sstride]
    uint32_t* hist;      // dense: [B][Tc][2048] histograms of the keys' top 11 bits;
                         // split: [B*Tq][nslices][IDX_SLOT_W] per-slice lists of nonzero bins
    uint32_t* cand_key;  // split: [B*Tq][sstride], filter block f's kept keys at [f*spb*S, ..)
    int32_t* cand_idx;   // split: [B*Tq][sstride], their entry indices
    int32_t* seg_cnt;    // split: [B*Tq][nslices] keys kept per filter block
    uint32_t* row_bin;   // split: [B*Tq][4] threshold bin of each row, keys above it, keys in it
    // dense path (many queries): queries qc0 .. qc0+Tc-1 per pass
    int dense;           // 1: score every (query, key) pair to HBM, then select per query
    int Tc;              // rows per pass
    int qc0;             // first query of the pass (set by the launcher)
};

struct AttendArgs {
    const uint8_t* q; int q_fmt;
    const uint8_t* kvc; int kv_fmt; int64_t kvc_bstride; int64_t n_cap;
    const int32_t* idx; int k;   // CSA: selected entries (idx != nullptr)
    int m;                       // HCA: entries visible at t are s < floor((t+1)/m)
    const uint8_t* kvw; int64_t kvw_bstride, kvw_pos0, kvw_rows;
    const int32_t* q_pos; int W, B, Tq, H, d, r; float scale;
    uint8_t* out; int out_fmt; float* lse;
    // plan
    int nhb;        // head blocks of 64
    int nsplit;     // splits of the attended row list
    int rps;        // rows per split (multiple of the row tile)
    float* ws_o;    // [B*Tq][nhb][nsplit][64][d]
    float* ws_lse;  // [B*Tq][nhb][nsplit][64]
};

hipError_t launch_compress(const CompressArgs& a, hipStream_t s);
hipError_t launch_index_topk(const IndexArgs& a, hipStream_t s);
hipError_t launch_attend(const AttendArgs& a, hipStream_t s);

}  // namespace csl
