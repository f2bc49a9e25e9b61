// launch.h -- argument blocks and launchers of the HIP kernels (internal; the
// public C ABI in include/csl.h validates arguments and calls these).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csl {

constexpr int IDX_SLOT_W = 2048 + 8;   // words per slice histogram list: count, then <= 2048 entries

struct CompressArgs {
    const uint8_t* x; int x_fmt; int64_t x_bstride; int64_t x_pos0; int64_t n_tok;
    int64_t x_rows;              // > 0: x and z are rings (position p in row (p - x_pos0) mod x_rows)
    int x_roles;                 // 2: a raw row holds a look-back value, then a current value
    const float* z; int z_ch; int64_t z_bstride;
    const float* bias;
    int B, d, r, m, overlap; int64_t e_begin, n_e;
    uint8_t* out; int out_fmt; uint8_t* out_scales; int64_t out_bstride, sc_bstride;
    // decode-time step (pos != nullptr): token q of sequence b at pos[b*n_e + q] compresses
    // entry (pos+1)/m - 1 when (pos+1) % m == 0, written at its absolute index in the cache:
    // out + b*out_bstride + e*row (e < n_cap), or, with a block table, row e % epb of block
    // bt[b*bt_stride + e/epb] (blocks blk_bytes apart; scales sblk_bytes apart)
    const int32_t* pos; int64_t n_cap;
    const int32_t* bt; int64_t bt_stride; int epb; int64_t blk_bytes, sblk_bytes, n_blocks;
};

struct IndexArgs {
    const uint8_t* qi; int qi_fmt; const uint8_t* qi_scales; const float* w;
    const uint8_t* ki; int ki_fmt; const uint8_t* ki_scales; int64_t ki_bstride, ks_bstride;
    // paged keys (bt != nullptr): key s of sequence b is row s % epb of block bt[b * bt_stride
    // + s / epb], blocks blk_bytes apart from ki (its scales: sblk_bytes apart from ki_scales);
    // ids outside [0, n_blocks) are absent blocks (their keys score -inf); epb % 16 == 0
    const int32_t* bt; int64_t bt_stride; int epb; int64_t blk_bytes, sblk_bytes, n_blocks;
    const int32_t* q_pos;
    int B, Tq, H_I, d_I, m; int64_t n_cap; int k;
    int32_t* out_idx; float* out_score;
    // plan
    int S;          // keys per slice (power of two in [512, 16384])
    int nslices;    // slices per query (<= 1024)
    // rows of the split (nslices > 1) and dense paths, in the workspace
    int64_t sstride;     // row stride (n_cap rounded up to a multiple of 4)
    uint32_t* scores;    // order-preserving score keys: dense [B][Tc][sstride]; split: [B*Tq][sstride],
                         // the keys at or above the query's threshold bin when too many for LDS
    uint32_t* hist;      // dense: [B][Tc][2048] histograms of the keys' top 11 bits;
                         // split: [B*Tq][nslices][IDX_SLOT_W] per-slice lists of nonzero bins
    uint32_t* cand_key;  // split: [B*Tq][sstride], slice s's kept keys at [s*S, ..), in entry order
    int32_t* cand_idx;   // split: [B*Tq][sstride], their entry indices
    int32_t* seg_cnt;    // split: [B*Tq][nslices] keys kept per slice
    int32_t* fb_idx;     // split: [B*Tq][sstride], entry indices of the `scores` keys (when used)
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
    const float* sink;           // [H] sink logits, or nullptr
    // paged entries (bt != nullptr): entry s of sequence b is row s % epb of block
    // bt[b * bt_stride + s / epb], blocks blk_bytes apart from kvc; ids outside
    // [0, n_blocks) are absent blocks
    const int32_t* bt; int64_t bt_stride; int epb; int64_t blk_bytes, n_blocks;
    const int32_t* q_pos; int W, B, Tq, H, d, r; float scale;
    uint8_t* out; int out_fmt; float* lse;
    // plan
    int nhb;        // head blocks of 64
    int nsplit;     // splits of the attended row list
    int rps;        // rows per split (multiple of the row tile)
    float* ws_o;    // [B*Tq][nhb][nsplit][64][d]
    float* ws_lse;  // [B*Tq][nhb][nsplit][64]
};

struct GprojArgs {
    const uint8_t* x;   // bf16 [M][G*K]
    const uint8_t* w;   // bf16 [G][R][K]
    int M, G, K, R;
    uint8_t* out; int out_fmt;   // [M][G*R], F32 or BF16
};

// A CSA layer's decode-time compression jobs (its KV entry, its indexer key) run by the
// indexer's scoring kernel before it scores (channel splits gz_kv, gz_key).
struct IndexPre {
    CompressArgs kv, key;
    int gz_kv, gz_key;
};

hipError_t launch_compress(const CompressArgs& a, hipStream_t s);
hipError_t launch_compress_pair(const CompressArgs& a0, const CompressArgs& a1, hipStream_t s);
bool compress_pair_in_index(const CompressArgs& kv, const CompressArgs& key, int& gz_kv, int& gz_key);
hipError_t launch_index_topk(const IndexArgs& a, hipStream_t s, const IndexPre* pre = nullptr);
// An HCA layer's decode-time compression job run by the attention kernel (channel split gz).
struct AttendPre {
    CompressArgs kv;
    int gz;
};
bool compress_in_attend(const CompressArgs& kv, int& gz);
bool attend_takes_pre(const AttendArgs& a);
hipError_t launch_attend(const AttendArgs& a, hipStream_t s, const AttendPre* pre = nullptr);
hipError_t launch_grouped_out_proj(const GprojArgs& a, hipStream_t s);

}  // namespace csl
