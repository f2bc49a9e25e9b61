/*
 * csl.h -- C ABI of the MI355X (gfx950) hybrid compressed attention library
 * (libcsl.so): the hot path of the CSA + HCA attention layer described for
 * DeepSeek-V4.
 *
 * Sources: the pages are commentary on the DeepSeek-V4 technical report --
 *   [X] m.x-techcon.com article 133366, section 2 (hybrid compressed attention:
 *       CSA steps 1-3, the HCA subsection, the mixed-precision KV paragraph) and
 *       section 4 (FP4 QAT paragraph; KV-cache management paragraph);
 *   [C] deepseek.csdn.net explainer, sections on CSA, HCA, SWA and the KV cache;
 *   [B] chenxutan.com article, section 4.5 (mixed KV storage).
 *
 * Conventions shared by every call
 *  - All tensor arguments are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or synchronises.  Work is enqueued on `stream` (a
 *    hipStream_t; NULL = the default stream) and returns at once.
 *  - Positions are absolute token positions (int64 on the host, int32 in device
 *    arrays).  A query at position t sees compressed entries s < floor((t+1)/m)
 *    (the entries whose raw tokens are all <= t) and the window t-W+1 .. t.
 *  - Byte strides (`*_bstride`) step from one sequence of the batch to the next.
 *    Rows inside a sequence are dense, `csl_row_bytes(fmt, d, r)` bytes each.
 *  - Alignment: every base pointer and every byte stride must be a multiple of
 *    16 bytes, except q_pos/idx/w (4 bytes) and MXFP4 scale arrays (1 byte).
 *  - Errors: calls return CSL_OK (0) or a negative code.  Arguments are checked
 *    on the host before anything is enqueued; on error nothing is launched and
 *    no output is touched.  csl_last_error() gives the reason as text
 *    (thread-local).  Values inside device arrays (positions, indices) cannot be
 *    checked on the host: out-of-range indices are skipped, never dereferenced.
 *  - Results are deterministic: identical inputs give identical bytes (no
 *    floating-point atomics; fixed reduction orders).
 *  - Calls on different streams may run concurrently if their outputs and
 *    workspaces do not overlap.
 */
#ifndef CSL_H
#define CSL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage formats of a row of d values.
 *  CSL_F32        d x fp32.
 *  CSL_BF16       d x bf16.
 *  CSL_KV_PACKED  the r RoPE dims as bf16, then the other d-r dims as OCP fp8
 *                 e4m3fn (unit scale) -- the mixed-precision KV entry ([X]
 *                 mixed-precision paragraph; [B] section 4.5): 576 bytes for
 *                 d = 512, r = 64.
 *  CSL_MXFP4      d/2 bytes of OCP e2m1 codes (element 2i in the low nibble of
 *                 byte i) plus, in a SEPARATE scale array, d/32 e8m0 scales per
 *                 row (one per 32 consecutive elements; value 2^(code-127)).
 */
typedef enum {
    CSL_F32 = 0,
    CSL_BF16 = 1,
    CSL_KV_PACKED = 2,
    CSL_MXFP4 = 3
} csl_fmt;

enum {
    CSL_OK = 0,
    CSL_EINVAL = -1,        /* null pointer, bad size, stride or alignment */
    CSL_EUNSUPPORTED = -2,  /* valid but not built: head dim, format combination, k, device */
    CSL_EWORKSPACE = -3,    /* workspace missing or smaller than csl_*_workspace() */
    CSL_ELAUNCH = -4,       /* the HIP runtime refused the launch */
    CSL_EDEVICE = -5        /* no usable gfx950 device is current */
};

/* Bytes of one stored row; -1 for an unknown format. */
int64_t csl_row_bytes(int fmt, int d, int r);

/*
 * kv_compress -- token compression ([X] section 2, CSA step 1; HCA subsection).
 * Entry i of each sequence pools raw rows with a softmax over learned per-token
 * logits plus a per-slot position bias:
 *   win = overlap ? 2m : m;   p_j = (i+1)*m - win + j,  j = 0..win-1 (p_j >= 0 only)
 *   w_j,c = softmax_j(z[p_j, c] + bias[j, c]),  e_i[c'] = sum_j w_{j,c(c')} v_j[c']
 *   (c(c') = 0 when z_ch == 1, c' when z_ch == d).
 * CSA uses overlap = 1 (adjacent blocks overlap), HCA overlap = 0.
 *  x          raw rows, x_fmt CSL_F32 or CSL_BF16, x_roles*d values each; row of
 *             position p of sequence b at x + b*x_bstride + (p - x_pos0)*row bytes.
 *             The buffer holds positions x_pos0 .. x_pos0 + n_tok - 1 and must hold
 *             every window position >= 0 of entries e_begin .. e_begin+n_e-1.
 *  x_roles    1: v_j is the row.  2 (overlap only): two-role rows ([B] section 4.2
 *             projects 2*head_dim per token for the compressor): v_j is the row's
 *             first d values in the look-back slots j < m and its last d values in
 *             the current slots j >= m.
 *  z          fp32 logits, z_ch (1 or d) per position, same position indexing:
 *             z + b*z_bstride (bytes) + (p - x_pos0)*z_ch floats.
 *  bias       fp32 [win][z_ch], one bias per window slot (host-checked count).
 *  out        entry e_begin+q of sequence b at out + b*out_bstride +
 *             q*csl_row_bytes(out_fmt, d, r); out_fmt any csl_fmt.  For CSL_MXFP4
 *             the scales go to out_scales + b*sc_bstride + q*(d/32), and the block
 *             scale is the smallest power of two with 6*2^e >= max|block|;
 *             codes are rounded to nearest even.  bf16/e4m3 stores round to
 *             nearest even; e4m3 saturates at +-448.
 *  Limits: d a multiple of 32 with 32 <= d <= 1024; for packed output r a
 *  multiple of 8 with 0 <= r <= d and d + r a multiple of 16 (16-byte rows);
 *  m >= 1; e_begin >= 0.
 */
int kv_compress(const void* x, int x_fmt, int x_roles, int64_t x_bstride, int64_t x_pos0, int64_t n_tok,
                const float* z, int z_ch, int64_t z_bstride, const float* bias,
                int B, int d, int r, int m, int overlap, int64_t e_begin, int64_t n_e,
                void* out, int out_fmt, uint8_t* out_scales, int64_t out_bstride, int64_t sc_bstride,
                void* stream);

/*
 * kv_compress_step -- decode-time compression driven from the state ring, the other
 * half of the two-tier cache ([X] section 4, KV-cache paragraph: a per-request state
 * cache holds the window and the not yet compressed tail; [C] KV-cache section).
 * Each sequence b appended T new tokens at positions pos[b*T + 0 .. T-1] (ragged
 * across the batch).  A token at p with (p + 1) % m == 0 completes entry
 * e = (p + 1)/m - 1, which is pooled as in kv_compress from the raw rows and logits
 * in the rings and written into the cache; other tokens do nothing (one launch serves
 * the whole batch).
 *  x_ring     raw rows (x_fmt, x_roles*d values): position p of sequence b in row
 *             p mod x_rows of x_ring + b*x_bstride; z_ring the logits, same rows.  The
 *             ring must hold the window of every completed entry: x_rows >= win + T - 1
 *             (checked) with the newest x_rows positions resident (the caller's part).
 *  out        the compressed cache: linear (block_table NULL) -- entry e of sequence b
 *             at out + b*out_bstride + e*row bytes, scales out_scales + b*sc_bstride +
 *             e*(d/32), entries e >= n_cap skipped -- or paged: row e % entries_per_block
 *             of block block_table[b*bt_stride + e / entries_per_block] (out +
 *             block*block_bytes; scales out_scales + block*scale_block_bytes); absent
 *             blocks (ids outside [0, n_blocks)) and entries beyond the table are skipped.
 *  Other arguments as in kv_compress.
 */
int kv_compress_step(const void* x_ring, int x_fmt, int x_roles, int64_t x_bstride, int64_t x_rows,
                     const float* z_ring, int z_ch, int64_t z_bstride, const float* bias,
                     const int32_t* pos, int B, int T, int d, int r, int m, int overlap,
                     void* out, int out_fmt, uint8_t* out_scales, int64_t out_bstride, int64_t sc_bstride,
                     int64_t n_cap, const int32_t* block_table, int64_t bt_stride, int entries_per_block,
                     int64_t block_bytes, int64_t scale_block_bytes, int64_t n_blocks, void* stream);

/*
 * kv_compress_step_pair -- two kv_compress_step jobs over the same new tokens (pos, B,
 * T) in one launch: a CSA layer's KV entry and its indexer key, both pooled from their
 * rings when a token completes a block.  Each job's fields mean what kv_compress_step's
 * arguments of the same names mean, and each job is validated as that call would
 * validate it; on any error nothing is launched.  Results are identical to two
 * kv_compress_step calls (jobs whose shapes the fused kernel does not take -- other
 * than bf16 raw rows, one logit per token, a packed KV entry then an MXFP4 or bf16
 * key -- are run as two launches).
 */
typedef struct {
    const void* x_ring; int x_fmt; int x_roles; int64_t x_bstride; int64_t x_rows;
    const float* z_ring; int z_ch; int64_t z_bstride; const float* bias;
    int d; int r; int m; int overlap;
    void* out; int out_fmt; uint8_t* out_scales; int64_t out_bstride; int64_t sc_bstride; int64_t n_cap;
    const int32_t* block_table; int64_t bt_stride; int entries_per_block;
    int64_t block_bytes; int64_t scale_block_bytes; int64_t n_blocks;
} csl_compress_job;

int kv_compress_step_pair(const csl_compress_job* first, const csl_compress_job* second, const int32_t* pos, int B,
                          int T, void* stream);

/*
 * index_topk -- lightning indexer + top-k selection ([X] section 2, CSA step 2;
 * FP4 indexer QK: [X] mixed-precision paragraph and section 4).
 * For query j of sequence b at position t = q_pos[b*Tq + j]:
 *   score(s) = sum_h w[b,j,h] * max(0, qi[b,j,h,:] . ki[b,s,:]),  s < n(t) = min(floor((t+1)/m), n_cap)
 * (the pages give no formula for the indexer score: this ReLU-gated, per-head
 * weighted form is the reading adopted).  Keeps the k best by (score desc,
 * index asc) and writes them ASCENDING by index to out_idx[b,j,0..k-1], padded
 * with -1 when n(t) < k; out_score (nullable) gets their fp32 scores (-inf pads).
 *  qi         dense [B][Tq][H_I] rows of d_I in qi_fmt; qi_scales [B][Tq][H_I][d_I/32]
 *             for CSL_MXFP4 (else NULL).
 *  w          fp32 [B][Tq][H_I] head weights.
 *  ki         entry s of sequence b at ki + b*ki_bstride + s*csl_row_bytes(ki_fmt, d_I, 0);
 *             ki_scales + b*ks_bstride + s*(d_I/32) for CSL_MXFP4.
 *  Formats: qi_fmt == ki_fmt, one of CSL_F32 (d_I 32 or 128), CSL_BF16 (d_I 32, 64
 *  or 128), CSL_MXFP4 (d_I 128; scales applied by the scaled FP4 MFMA).
 *  Limits: H_I <= 128, 1 <= k <= 2048, n_cap <= 2^24 (CSL_EUNSUPPORTED beyond).
 *  ws         device workspace of at least csl_index_topk_workspace(...) bytes
 *             (0 for small calls; a little over 16 * B * Tq * n_cap bytes when a query's
 *             entries span several scoring blocks: the blocks' candidates and, for
 *             queries with many tied keys, their gathered rows are staged there).
 */
int index_topk(const void* qi, int qi_fmt, const uint8_t* qi_scales, const float* w,
               const void* ki, int ki_fmt, const uint8_t* ki_scales, int64_t ki_bstride, int64_t ks_bstride,
               const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int m, int64_t n_cap, int k,
               int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes, void* stream);

size_t csl_index_topk_workspace(int B, int Tq, int64_t n_cap, int k);

/*
 * index_topk_paged -- index_topk over paged indexer keys, the classical half of the
 * two-tier cache ([X] section 4, KV-cache paragraph; [C] KV-cache section: the CSA
 * cache also holds the indexer's keys).  Key s of sequence b is row (s %
 * entries_per_block) of block block_table[b*bt_stride + s / entries_per_block]: its
 * bytes at ki_pool + block*block_bytes + (s % entries_per_block)*row bytes, its MXFP4
 * scales at ki_scale_pool + block*scale_block_bytes + (s % entries_per_block)*(d_I/32).
 * The key rows may share their blocks with the compressed KV entries (one block per
 * lcm(m, m') raw tokens holding both: pass pointers into the block and the block's full
 * stride).  entries_per_block must be a multiple of 16.  Keys of an absent block (id
 * outside [0, n_blocks)) are never read and score -inf.  Other arguments, results and
 * the workspace (csl_index_topk_workspace) as in index_topk.
 */
int index_topk_paged(const void* qi, int qi_fmt, const uint8_t* qi_scales, const float* w,
                     const void* ki_pool, int ki_fmt, const uint8_t* ki_scale_pool,
                     const int32_t* block_table, int64_t bt_stride, int entries_per_block,
                     int64_t block_bytes, int64_t scale_block_bytes, int64_t n_blocks,
                     const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int m, int64_t n_cap, int k,
                     int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes, void* stream);

/*
 * csa_index_step -- a CSA layer's decode step up to the selection: the compression of
 * the entries the new tokens complete ([X] section 2, CSA step 1: the KV entry and, by
 * the indexer's own compressor, its key) followed by the lightning indexer's top-k over
 * every complete key, the new one included ([X] section 2, CSA step 2).  The results
 * are those of kv_compress_step_pair(kv_job, key_job, q_pos, B, Tq) followed by
 * index_topk (block_table NULL: keys at ki + b*ki_bstride, scales at ki_scales +
 * b*ks_bstride) or index_topk_paged (block_table given, with its geometry), on the same
 * stream; every argument means what it means there, q_pos doubling as the jobs' token
 * positions.  The key job should write the keys this call reads; the KV job's output
 * must not overlap the keys or their scales.  With one query per sequence, entries
 * spanning several scoring blocks, d_I = 128 MXFP4 or bf16 keys that the key job writes
 * in place, and the one-wave compression shapes (bf16 rings, one logit per token), the
 * compression runs inside the indexer's scoring kernel (one launch fewer); otherwise it
 * is launched first.  Workspace: csl_index_topk_workspace(B, Tq, n_cap, k).  Both jobs
 * and the index arguments are checked before anything is launched.
 */
int csa_index_step(const csl_compress_job* kv_job, const csl_compress_job* key_job,
                   const void* qi, int qi_fmt, const uint8_t* qi_scales, const float* w,
                   const void* ki, int ki_fmt, const uint8_t* ki_scales, int64_t ki_bstride, int64_t ks_bstride,
                   const int32_t* block_table, int64_t bt_stride, int entries_per_block, int64_t block_bytes,
                   int64_t scale_block_bytes, int64_t n_blocks,
                   const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int m, int64_t n_cap, int k,
                   int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes, void* stream);

/*
 * index_topk_noalloc -- index_topk for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and results as index_topk, without the workspace
 * arguments.  The staging it needs lives in a static device array of the library,
 * csl_noalloc_scratch_bytes() bytes (96 MiB) on every GPU the library runs on, held
 * until the process ends.  A call whose staging would exceed it (the
 * csl_index_topk_workspace figure of the same sizes, e.g. more than about 6 million
 * (query, entry) pairs per call when entries span several scoring blocks, or a
 * many-query prefill call) returns CSL_EWORKSPACE and launches nothing.  No call
 * allocates or frees memory.  All calls on one GPU share that array: calls that may
 * overlap in time on one GPU (different streams, or graphs replayed concurrently) race
 * and must be serialised by the caller.  Nothing in the array has to start at zero.
 */
int index_topk_noalloc(const void* qi, int qi_fmt, const uint8_t* qi_scales, const float* w,
                       const void* ki, int ki_fmt, const uint8_t* ki_scales, int64_t ki_bstride, int64_t ks_bstride,
                       const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int m, int64_t n_cap, int k,
                       int32_t* out_idx, float* out_score, void* stream);

/* Bytes of the static scratch index_topk_noalloc uses on each GPU. */
size_t csl_noalloc_scratch_bytes(void);

/*
 * csa_attend -- CSA attention ([X] section 2, CSA step 3): shared-KV MQA of each
 * query over the selected compressed entries and its sliding window, in ONE
 * softmax:  S(t) = {idx[b,j,u] : 0 <= idx < n_cap} U {window positions
 * max(0,t-W+1) .. t};  o_h = sum_{v in S} softmax(scale * q_h . v) v  (key = value
 * = the stored row);  lse_h = log sum exp(scale * q_h . v).  An empty S gives
 * o = 0, lse = -inf.
 *  q          dense [B][Tq][H][d]: CSL_BF16 when the KV is CSL_BF16/CSL_KV_PACKED,
 *             CSL_F32 when the KV is CSL_F32.
 *  kv_c       compressed entries (kv_fmt) of sequence b at kv_c + b*kvc_bstride,
 *             n_cap rows resident.
 *  idx        int32 [B][Tq][k] (e.g. index_topk's output; -1 = empty slot).
 *  kv_w       window rows (same kv_fmt): position p of sequence b is row
 *             ((p - kvw_pos0) mod kvw_rows) of kv_w + b*kvw_bstride -- a linear
 *             buffer (kvw_pos0 = its first position) or a ring (kvw_pos0 = 0).  The
 *             caller keeps positions t-W+1 .. t resident; kvw_rows >= W is required
 *             (CSL_EINVAL otherwise), so W consecutive positions never share a row.
 *  sink       fp32 [H] attention-sink logits, or NULL for none ([C] table of attention
 *             details, "Attention Sink": a head may attend to nothing).  Head h's
 *             softmax then has the extra logit sink[h] with no value:
 *             o_h = sum_S exp(l) v / (exp(sink[h]) + sum_S exp(l)),
 *             lse_h = log(exp(sink[h]) + sum_S exp(l))  (an empty S: o = 0, lse = sink[h]).
 *  out        [B][Tq][H][d], out_fmt CSL_F32 or CSL_BF16;  out_lse fp32 [B][Tq][H] or NULL.
 *  Limits: d in {64, 128, 256, 512}; packed: r multiple of 8, d-r multiple of 16,
 *  r <= d/4 (CSL_EUNSUPPORTED beyond).
 *  ws         device workspace of at least csl_attend_workspace(...) bytes
 *             (split partials; may be NULL when that size is 0).
 */
int csa_attend(const void* q, int q_fmt, const void* kv_c, int kv_fmt, int64_t kvc_bstride, int64_t n_cap,
               const int32_t* idx, int k,
               const void* kv_w, int64_t kvw_bstride, int64_t kvw_pos0, int64_t kvw_rows, const float* sink,
               const int32_t* q_pos, int W, int B, int Tq, int H, int d, int r, float scale,
               void* out, int out_fmt, float* out_lse, void* ws, size_t ws_bytes, void* stream);

/*
 * hca_attend -- HCA attention ([X] section 2, HCA subsection): as csa_attend, but
 * over EVERY complete entry, S(t) = {s < min(floor((t+1)/m), n_cap)} U window.
 * n_cap = 0 with W > 0 is a sliding-window-only layer.
 */
int hca_attend(const void* q, int q_fmt, const void* kv_c, int kv_fmt, int64_t kvc_bstride, int64_t n_cap, int m,
               const void* kv_w, int64_t kvw_bstride, int64_t kvw_pos0, int64_t kvw_rows, const float* sink,
               const int32_t* q_pos, int W, int B, int Tq, int H, int d, int r, float scale,
               void* out, int out_fmt, float* out_lse, void* ws, size_t ws_bytes, void* stream);

/*
 * csa_attend_paged / hca_attend_paged -- the same attention over a PAGED compressed
 * cache, the classical half of the two-tier cache ([X] section 4, KV-cache paragraph:
 * compressed CSA/HCA entries in blocks, each block covering lcm(m, m') raw tokens;
 * [C] KV-cache section).  Compressed entry s of sequence b is row
 * (s % entries_per_block) of physical block block_table[b*bt_stride + s /
 * entries_per_block] of the pool, blocks block_bytes apart from kv_pool (a block may
 * hold other data after its rows).  For blocks of lcm(4, 128) = 128 raw tokens a CSA
 * layer has entries_per_block = 32 and an HCA layer 1, and both layers can share one
 * block table.  A block id outside [0, n_blocks) is an absent block: its rows are
 * skipped (never read).  Requires bt_stride >= ceil(n_cap / entries_per_block),
 * block_bytes >= entries_per_block * row bytes and a multiple of 16, n_cap < 2^31.
 * The window (the other tier: a ring per sequence) and every other argument as in
 * csa_attend / hca_attend.
 */
int csa_attend_paged(const void* q, int q_fmt, const void* kv_pool, int kv_fmt, const int32_t* block_table,
                     int64_t bt_stride, int entries_per_block, int64_t block_bytes, int64_t n_blocks, int64_t n_cap,
                     const int32_t* idx, int k,
                     const void* kv_w, int64_t kvw_bstride, int64_t kvw_pos0, int64_t kvw_rows, const float* sink,
                     const int32_t* q_pos, int W, int B, int Tq, int H, int d, int r, float scale,
                     void* out, int out_fmt, float* out_lse, void* ws, size_t ws_bytes, void* stream);

int hca_attend_paged(const void* q, int q_fmt, const void* kv_pool, int kv_fmt, const int32_t* block_table,
                     int64_t bt_stride, int entries_per_block, int64_t block_bytes, int64_t n_blocks, int64_t n_cap,
                     int m, const void* kv_w, int64_t kvw_bstride, int64_t kvw_pos0, int64_t kvw_rows,
                     const float* sink, const int32_t* q_pos, int W, int B, int Tq, int H, int d, int r, float scale,
                     void* out, int out_fmt, float* out_lse, void* ws, size_t ws_bytes, void* stream);

/*
 * hca_attend_step -- an HCA layer's decode step: the compression of the entries the new
 * tokens complete ([X] section 2, HCA subsection: the CSA compression at m' = 128, no
 * overlap) followed by the dense attention over every complete entry plus the window.
 * The results are those of kv_compress_step(kv_job's arguments, pos = q_pos, T = Tq)
 * followed by hca_attend (block_table NULL: entries at kv_c + b*kvc_bstride) or
 * hca_attend_paged (block_table given, kv_c the pool), on the same stream; every argument
 * means what it means there.  The job should write the entries this call reads.  With
 * one query per sequence, packed rows of the RoPE width 64 and d 256 or 512, a job that
 * writes those entries in place (same buffer and strides, or the same block table) and
 * the one-wave compression shape (bf16 ring, one logit per token), the compression runs
 * inside the attention kernel, by the split that attends the new entry (one launch
 * fewer); otherwise it is launched first.  Workspace: csl_attend_workspace(B, Tq, H, d,
 * n_cap + W).  The job and the attention arguments are checked before anything is
 * launched.
 */
int hca_attend_step(const csl_compress_job* kv_job, const void* q, int q_fmt, const void* kv_c, int kv_fmt,
                    int64_t kvc_bstride, const int32_t* block_table, int64_t bt_stride, int entries_per_block,
                    int64_t block_bytes, int64_t n_blocks, int64_t n_cap, int m,
                    const void* kv_w, int64_t kvw_bstride, int64_t kvw_pos0, int64_t kvw_rows, const float* sink,
                    const int32_t* q_pos, int W, int B, int Tq, int H, int d, int r, float scale,
                    void* out, int out_fmt, float* out_lse, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for csa_attend[_paged] (rows_max = k + W) or hca_attend[_paged]
 * (rows_max = n_cap + W) with these sizes; 0 when no split partials are needed. */
size_t csl_attend_workspace(int B, int Tq, int H, int d, int64_t rows_max);

/*
 * grouped_out_proj -- grouped output projection after the attention ([X] section 2,
 * HCA subsection: both branches project their outputs group by group; [C] table of
 * attention details, "Grouped Output Projection": compress per group, then combine).
 * With the attention output of M tokens laid out [M][H][d] and G groups of H/G heads,
 * group g's input is the K = (H/G)*d contiguous values g*K .. g*K+K-1 of a token:
 *   out[t][g*R + n] = sum_k x[t][g*K + k] * w[g][n][k]      (fp32 accumulation)
 * G = 1 is a plain projection (the common projection that combines the groups).
 *  x      bf16 [M][G*K] (dense);  w  bf16 [G][R][K] (dense; row n of group g's matrix
 *         is output n's weights, the layout of a [out][in] linear weight).
 *  out    [M][G*R], CSL_F32 or CSL_BF16 (round to nearest even).
 *  Limits: K and R multiples of 128 (CSL_EUNSUPPORTED otherwise); 16-byte aligned
 *  pointers.  The pages give no sizes; the benchmark uses H = 64, d = 512, G = 8,
 *  R = 1024.
 */
int grouped_out_proj(const void* x, int x_fmt, const void* w, int w_fmt, int M, int G, int K, int R,
                     void* out, int out_fmt, void* stream);

/* Text of a status code; text of the calling thread's last error (copied into
 * buf, NUL-terminated; returns the full length); library version (major*10000 +
 * minor*100 + patch). */
const char* csl_status_string(int status);
int csl_last_error(char* buf, size_t n);
int csl_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CSL_H */
