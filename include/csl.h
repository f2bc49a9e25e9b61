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
 *   w_j,c = softmax_j(z[p_j, c] + bias[j, c]),  e_i[c'] = sum_j w_{j,c(c')} x[p_j, c']
 *   (c(c') = 0 when z_ch == 1, c' when z_ch == d).
 * CSA uses overlap = 1 (adjacent blocks overlap), HCA overlap = 0.
 *  x          raw rows, x_fmt CSL_F32 or CSL_BF16; row of position p of sequence b
 *             at x + b*x_bstride + (p - x_pos0)*csl_row_bytes(x_fmt, d, 0).  The
 *             buffer holds positions x_pos0 .. x_pos0 + n_tok - 1 and must hold
 *             every window position >= 0 of entries e_begin .. e_begin+n_e-1.
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
int kv_compress(const void* x, int x_fmt, int64_t x_bstride, int64_t x_pos0, int64_t n_tok,
                const float* z, int z_ch, int64_t z_bstride, const float* bias,
                int B, int d, int r, int m, int overlap, int64_t e_begin, int64_t n_e,
                void* out, int out_fmt, uint8_t* out_scales, int64_t out_bstride, int64_t sc_bstride,
                void* stream);

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
 *             (0 for small calls; a little over 12 * B * Tq * n_cap bytes when a query's
 *             entries span several scoring blocks: score rows and filtered
 *             candidates are staged there).
 */
int index_topk(const void* qi, int qi_fmt, const uint8_t* qi_scales, const float* w,
               const void* ki, int ki_fmt, const uint8_t* ki_scales, int64_t ki_bstride, int64_t ks_bstride,
               const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int m, int64_t n_cap, int k,
               int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes, void* stream);

size_t csl_index_topk_workspace(int B, int Tq, int64_t n_cap, int k);

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
 *             caller keeps positions t-W+1 .. t resident.
 *  out        [B][Tq][H][d], out_fmt CSL_F32 or CSL_BF16;  out_lse fp32 [B][Tq][H] or NULL.
 *  Limits: d in {64, 128, 256, 512}; packed: r multiple of 8, d-r multiple of 16,
 *  r <= d/4 (CSL_EUNSUPPORTED beyond).
 *  ws         device workspace of at least csl_attend_workspace(...) bytes
 *             (split partials; may be NULL when that size is 0).
 */
int csa_attend(const void* q, int q_fmt, const void* kv_c, int kv_fmt, int64_t kvc_bstride, int64_t n_cap,
               const int32_t* idx, int k,
               const void* kv_w, int64_t kvw_bstride, int64_t kvw_pos0, int64_t kvw_rows,
               const int32_t* q_pos, int W, int B, int Tq, int H, int d, int r, float scale,
               void* out, int out_fmt, float* out_lse, void* ws, size_t ws_bytes, void* stream);

/*
 * hca_attend -- HCA attention ([X] section 2, HCA subsection): as csa_attend, but
 * over EVERY complete entry, S(t) = {s < min(floor((t+1)/m), n_cap)} U window.
 */
int hca_attend(const void* q, int q_fmt, const void* kv_c, int kv_fmt, int64_t kvc_bstride, int64_t n_cap, int m,
               const void* kv_w, int64_t kvw_bstride, int64_t kvw_pos0, int64_t kvw_rows,
               const int32_t* q_pos, int W, int B, int Tq, int H, int d, int r, float scale,
               void* out, int out_fmt, float* out_lse, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for csa_attend (rows_max = k + W) or hca_attend (rows_max =
 * n_cap + W) with these sizes; 0 when no split partials are needed. */
size_t csl_attend_workspace(int B, int Tq, int H, int d, int64_t rows_max);

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
