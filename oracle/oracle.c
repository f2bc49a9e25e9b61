/*
 * oracle.c -- plain, slow, fp64 CPU reference of the hybrid compressed attention
 * layer (CSA + HCA) described for DeepSeek-V4.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or load
 * this file; only the test-suite, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no code, header, table or constant generator with
 * the HIP library: it has its own format codecs and its own loops, written from the
 * definitions, in the order the pages describe the method.
 *
 * Sources (cited by page and section; the pages are commentary on the DeepSeek-V4
 * technical report):
 *  [X] m.x-techcon.com article 133366, section 2 (hybrid compressed attention):
 *      subsection on CSA, steps 1-3 (compression with learned weights + position
 *      bias + softmax + overlapping blocks; lightning indexer + top-k; 128-token
 *      window attended together with the selected entries), subsection on HCA
 *      (m' = 128, dense, shared-KV MQA), and the paragraph on mixed-precision KV
 *      (BF16 RoPE dims + FP8 rest, FP4 indexer QK); section 4, FP4 QAT paragraph
 *      (FP4 -> FP8 lossless with block scales).
 *  [C] deepseek.csdn.net explainer, sections on CSA, HCA, SWA and the KV cache.
 *  [B] chenxutan.com article, section 4.5 (mixed KV storage: rope dims first,
 *      e4m3fn for the rest) and section 6.2 (the e2m1 value list).
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *  - compression window: entry i covers raw positions (i+1)m-win .. (i+1)m-1 with
 *    win = 2m when blocks overlap (CSA) and win = m otherwise (HCA); positions < 0
 *    are left out of the softmax so the weights still sum to one;
 *  - one logit per raw token (z_ch = 1) or one per channel (z_ch = d), plus one
 *    learned bias per position inside the window;
 *  - indexer score(t,s) = sum_h w[t,h] * max(0, q[t,h] . k[s]) over entries s that
 *    are complete at t (s < floor((t+1)/m)); top-k by (score desc, index asc);
 *    output ascending by index, padded with -1;  (parity unpinned by the pages:
 *    the pages name a low-rank "lightning indexer" but print no formula)
 *  - attention: one joint softmax over {selected or all entries} U {window rows
 *    t-W+1..t}; key = value = the stored row; logits = scale * q.v;
 *  - MXFP4: e2m1 codes, one e8m0 scale per 32 contiguous elements, scale = the
 *    smallest power of two with 6*2^e >= block max (no clipping), codes by
 *    round-to-nearest-even, low nibble = even element;
 *  - attention sink ([C] table of attention details, "Attention Sink": a head may
 *    attend to nothing): one extra logit per head that joins the softmax's
 *    denominator and carries no value;
 *  - grouped output projection ([X] HCA subsection; [C] "Grouped Output
 *    Projection": heads are projected group by group before one common output
 *    projection): group g of G maps the concatenated outputs of its H/G heads
 *    through its own matrix;
 *  - two-role values (an alternative compressor input suggested by [B] section 4.2,
 *    whose projection emits 2*head_dim per token): with overlapping windows a raw
 *    row may carry two value vectors, the first used when the row sits in the
 *    look-back half of a window, the second in the current half;
 *  - two-tier cache ([X] section 4, KV-cache paragraph; [C] KV-cache section):
 *    raw rows and window rows live in a ring (position p in slot p mod rows),
 *    compressed entries in fixed blocks reached through a per-sequence block
 *    table (entry s in block table[s / entries_per_block], row s % entries_per_block).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#include <float.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_KV_PACKED = 2, ORC_MXFP4 = 3 };

enum { ORC_OK = 0, ORC_EINVAL = -1 };

/* ------------------------------------------------------------------------- */
/* Format codecs, from the format definitions.                                */
/* ------------------------------------------------------------------------- */

/* bf16 is the upper half of an IEEE binary32. */
double orc_bf16_decode(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa; no infinities;
 * S.1111.111 is NaN; exponent field 0 is subnormal m/8 * 2^-6.                 */
double orc_e4m3_decode(uint8_t b)
{
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = (m / 8.0) * ldexp(1.0, -6);
    else v = (1.0 + m / 8.0) * ldexp(1.0, e - 7);
    return s ? -v : v;
}

/* OCP FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa.  Positive values are
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6 (value list of [B] section 6.2).                   */
double orc_e2m1_decode(uint8_t c)
{
    int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double v;
    if (e == 0) v = 0.5 * m;
    else v = (1.0 + 0.5 * m) * ldexp(1.0, e - 1);
    return s ? -v : v;
}

/* E8M0 scale: 2^(code-127); code 255 is NaN. */
double orc_e8m0_decode(uint8_t c)
{
    if (c == 255) return NAN;
    return ldexp(1.0, (int)c - 127);
}

/* Round x to the grid of a binary floating-point format with `mbits` stored
 * mantissa bits, smallest normal exponent `emin`, and largest finite `maxf`,
 * ties to even.  `satur` != 0 clamps overflow to +-maxf, otherwise it returns
 * +-inf.  Works on the value; bit patterns are built by the encoders below.    */
static double round_to_format(double x, int mbits, int emin, double maxf, int satur)
{
    if (x != x) return x;
    if (x == 0.0) return x;
    double a = fabs(x);
    int e;
    frexp(a, &e);           /* a = f * 2^e, f in [0.5,1) => floor(log2 a) = e-1 */
    int ex = e - 1;
    if (ex < emin) ex = emin; /* subnormal range shares the quantum of emin */
    double quantum = ldexp(1.0, ex - mbits);
    double q = nearbyint(a / quantum); /* default rounding mode: nearest, ties even */
    double r = q * quantum;
    if (r > maxf) r = satur ? maxf : INFINITY;
    return x < 0 ? -r : r;
}

uint16_t orc_bf16_encode(double x)
{
    /* bf16: 7 stored mantissa bits, emin = -126, max = (2 - 2^-7) * 2^127 */
    if (x != x) return 0x7FC0;
    double r = round_to_format(x, 7, -126, (2.0 - ldexp(1.0, -7)) * ldexp(1.0, 127), 0);
    float f = (float)r; /* exact: r is on the bf16 grid */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

uint8_t orc_e4m3_encode(double x)
{
    /* e4m3fn: 3 mantissa bits, emin = -6, max 448, saturating */
    if (x != x) return 0x7F;
    double r = round_to_format(x, 3, -6, 448.0, 1);
    uint8_t s = (r < 0 || (r == 0 && signbit(x))) ? 0x80 : 0;
    double a = fabs(r);
    if (a == 0.0) return s;
    int e;
    frexp(a, &e);
    int ex = e - 1;
    if (ex < -6) {                       /* subnormal: a = m/8 * 2^-6 */
        int m = (int)llround(a / ldexp(1.0, -9));
        return s | (uint8_t)m;
    }
    int m = (int)llround((a / ldexp(1.0, ex) - 1.0) * 8.0);
    return s | (uint8_t)((ex + 7) << 3) | (uint8_t)m;
}

uint8_t orc_e2m1_encode(double x)
{
    /* e2m1: 1 mantissa bit, emin = 0, max 6, saturating */
    double r = round_to_format(x, 1, 0, 6.0, 1);
    uint8_t s = (r < 0 || (r == 0 && signbit(x))) ? 0x8 : 0;
    double a = fabs(r);
    if (a == 0.0) return s;
    if (a < 1.0) return s | 1;           /* 0.5 is the only subnormal */
    int e;
    frexp(a, &e);
    int ex = e - 1;                      /* 0, 1 or 2 */
    int m = (int)llround((a / ldexp(1.0, ex) - 1.0) * 2.0);
    return s | (uint8_t)((ex + 1) << 1) | (uint8_t)m;
}

/* Shared exponent of one MXFP4 block: the smallest e with 6 * 2^e >= amax. */
int orc_mx_block_exponent(double amax)
{
    if (!(amax > 0.0)) return -127;
    int E;
    double f = frexp(amax, &E);          /* amax = f * 2^E, f in [0.5, 1) */
    int e = (f <= 0.75) ? E - 3 : E - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* Encode n (multiple of 32) values into MXFP4 codes (n/2 bytes) + scales. */
void orc_mxfp4_encode_row(const double* v, int n, uint8_t* codes, uint8_t* scales)
{
    for (int b = 0; b < n / 32; ++b) {
        double amax = 0.0;
        for (int i = 0; i < 32; ++i) {
            double a = fabs(v[b * 32 + i]);
            if (a > amax) amax = a;
        }
        int e = orc_mx_block_exponent(amax);
        scales[b] = (uint8_t)(e + 127);
        for (int i = 0; i < 32; i += 2) {
            uint8_t lo = orc_e2m1_encode(ldexp(v[b * 32 + i], -e));
            uint8_t hi = orc_e2m1_encode(ldexp(v[b * 32 + i + 1], -e));
            codes[(b * 32 + i) / 2] = (uint8_t)((lo & 15) | ((hi & 15) << 4));
        }
    }
}

/* Bytes of one stored row. */
int64_t orc_row_bytes(int fmt, int d, int r)
{
    switch (fmt) {
    case ORC_F32: return 4 * (int64_t)d;
    case ORC_BF16: return 2 * (int64_t)d;
    case ORC_KV_PACKED: return 2 * (int64_t)r + (int64_t)(d - r);
    case ORC_MXFP4: return (int64_t)d / 2;
    }
    return -1;
}

/* Decode one stored row of d values.  `sc` is the row's scale bytes (MXFP4). */
static void decode_row(const uint8_t* p, const uint8_t* sc, int fmt, int d, int r, double* out)
{
    if (fmt == ORC_F32) {
        for (int i = 0; i < d; ++i) { float f; memcpy(&f, p + 4 * i, 4); out[i] = f; }
    } else if (fmt == ORC_BF16) {
        for (int i = 0; i < d; ++i) { uint16_t h; memcpy(&h, p + 2 * i, 2); out[i] = orc_bf16_decode(h); }
    } else if (fmt == ORC_KV_PACKED) {
        /* RoPE dims first, as bf16; then the other d-r dims as e4m3fn ([B] 4.5) */
        for (int i = 0; i < r; ++i) { uint16_t h; memcpy(&h, p + 2 * i, 2); out[i] = orc_bf16_decode(h); }
        for (int i = r; i < d; ++i) out[i] = orc_e4m3_decode(p[2 * r + (i - r)]);
    } else { /* ORC_MXFP4 */
        for (int i = 0; i < d; ++i) {
            uint8_t byte = p[i / 2];
            uint8_t c = (i & 1) ? (byte >> 4) : (byte & 15);
            out[i] = orc_e2m1_decode(c) * orc_e8m0_decode(sc[i / 32]);
        }
    }
}

/* Encode one row of d values. */
static void encode_row(const double* v, int fmt, int d, int r, uint8_t* p, uint8_t* sc)
{
    if (fmt == ORC_F32) {
        for (int i = 0; i < d; ++i) { float f = (float)v[i]; memcpy(p + 4 * i, &f, 4); }
    } else if (fmt == ORC_BF16) {
        for (int i = 0; i < d; ++i) { uint16_t h = orc_bf16_encode(v[i]); memcpy(p + 2 * i, &h, 2); }
    } else if (fmt == ORC_KV_PACKED) {
        for (int i = 0; i < r; ++i) { uint16_t h = orc_bf16_encode(v[i]); memcpy(p + 2 * i, &h, 2); }
        for (int i = r; i < d; ++i) p[2 * r + (i - r)] = orc_e4m3_encode(v[i]);
    } else {
        orc_mxfp4_encode_row(v, d, p, sc);
    }
}

/* Public wrappers so tests can run the row codecs on their own. */
void orc_decode_rows(const uint8_t* p, const uint8_t* sc, int fmt, int d, int r, int64_t n, double* out)
{
    int64_t rb = orc_row_bytes(fmt, d, r);
    for (int64_t i = 0; i < n; ++i)
        decode_row(p + i * rb, sc ? sc + i * (d / 32) : NULL, fmt, d, r, out + i * d);
}

void orc_encode_rows(const double* v, int fmt, int d, int r, int64_t n, uint8_t* p, uint8_t* sc)
{
    int64_t rb = orc_row_bytes(fmt, d, r);
    for (int64_t i = 0; i < n; ++i)
        encode_row(v + i * d, fmt, d, r, p + i * rb, sc ? sc + i * (d / 32) : NULL);
}

/* ------------------------------------------------------------------------- */
/* Token compression ([X] CSA step 1; same operator at m' for HCA).           */
/* ------------------------------------------------------------------------- */
/*
 * Entry i of sequence b is a softmax-weighted sum of the raw rows in its window:
 *   win = overlap ? 2m : m;  p_j = (i+1)m - win + j,  j = 0..win-1,  valid iff p_j >= 0
 *   a_j,c  = z[p_j, c] + bias[j, c]                (learned weight + position bias)
 *   w_j,c  = exp(a_j,c) / sum_{valid j'} exp(a_j',c)
 *   e_i[c'] = sum_{valid j} w_{j, c(c')} * v_j[c'],  c(c') = 0 if z_ch == 1 else c'
 * v_j is the raw row of position p_j; with x_roles == 2 (overlap only) a raw row holds
 * 2d values and v_j is its first half for the look-back slots j < m, its second half
 * for the current slots j >= m.
 * Raw row p of sequence b: linear buffer (x_rows == 0) at x + b*x_bstride +
 * (p - x_pos0)*rowbytes; ring (x_rows > 0) at slot ((p - x_pos0) mod x_rows).  Its
 * logits sit at the same row of z (z_ch floats per row, z_bstride bytes per sequence).
 */
static const uint8_t* ring_or_linear(const uint8_t* base, int64_t pos0, int64_t rows, int64_t rb, int64_t p)
{
    int64_t s = p - pos0;
    if (rows > 0) { s %= rows; if (s < 0) s += rows; }
    return base + s * rb;
}

static void compress_entry(const void* x, int x_fmt, int64_t x_bstride, int64_t x_pos0, int64_t x_rows, int x_roles,
                           const float* z, int z_ch, int64_t z_bstride, const float* bias,
                           int b, int d, int r, int m, int overlap, int64_t i, int out_fmt, uint8_t* o, uint8_t* sc)
{
    const int win = overlap ? 2 * m : m;
    const int64_t xrb = orc_row_bytes(x_fmt, x_roles * d, 0);
    double* rows = (double*)malloc(sizeof(double) * (size_t)win * x_roles * d);
    double* wgt = (double*)malloc(sizeof(double) * (size_t)win * z_ch);
    int* valid = (int*)malloc(sizeof(int) * (size_t)win);
    double* e = (double*)malloc(sizeof(double) * (size_t)d);
    for (int j = 0; j < win; ++j) {
        int64_t p = (i + 1) * m - win + j;
        valid[j] = p >= 0;
        if (!valid[j]) continue;
        const uint8_t* xr = ring_or_linear((const uint8_t*)x + b * x_bstride, x_pos0, x_rows, xrb, p);
        decode_row(xr, NULL, x_fmt, x_roles * d, r, rows + (size_t)j * x_roles * d);
        const float* zr = (const float*)ring_or_linear((const uint8_t*)z + b * z_bstride, x_pos0, x_rows,
                                                       4 * (int64_t)z_ch, p);
        for (int c = 0; c < z_ch; ++c) wgt[(size_t)j * z_ch + c] = (double)zr[c] + (double)bias[j * z_ch + c];
    }
    /* softmax over the valid window positions, per weight channel */
    for (int c = 0; c < z_ch; ++c) {
        double mx = -INFINITY, den = 0.0;
        for (int j = 0; j < win; ++j) if (valid[j] && wgt[(size_t)j * z_ch + c] > mx) mx = wgt[(size_t)j * z_ch + c];
        for (int j = 0; j < win; ++j) if (valid[j]) den += exp(wgt[(size_t)j * z_ch + c] - mx);
        for (int j = 0; j < win; ++j)
            wgt[(size_t)j * z_ch + c] = valid[j] ? exp(wgt[(size_t)j * z_ch + c] - mx) / den : 0.0;
    }
    for (int cc = 0; cc < d; ++cc) {
        double acc = 0.0;
        int c = (z_ch == 1) ? 0 : cc;
        for (int j = 0; j < win; ++j) {
            if (!valid[j]) continue;
            const int half = (x_roles == 2 && j >= m) ? d : 0;   /* which value of a two-role row */
            acc += wgt[(size_t)j * z_ch + c] * rows[(size_t)j * x_roles * d + half + cc];
        }
        e[cc] = acc;
    }
    encode_row(e, out_fmt, d, r, o, sc);
    free(rows); free(wgt); free(valid); free(e);
}

static int compress_args_ok(int x_fmt, int x_roles, int overlap, int d, int m, int z_ch)
{
    if (d <= 0 || m <= 0 || (z_ch != 1 && z_ch != d)) return 0;
    if (x_fmt != ORC_F32 && x_fmt != ORC_BF16) return 0;
    if (x_roles != 1 && x_roles != 2) return 0;
    if (x_roles == 2 && !overlap) return 0;
    return 1;
}

/* Entries e_begin .. e_begin+n_e-1 of every sequence; entry e_begin+q is written at
 * out + b*out_bstride + q*rowbytes(out_fmt) (scales: out_scales + b*sc_bstride +
 * q*d/32).  A linear raw buffer must hold every valid window position. */
int orc_kv_compress(const void* x, int x_fmt, int64_t x_bstride, int64_t x_pos0, int64_t n_tok, int64_t x_rows,
                    int x_roles, const float* z, int z_ch, int64_t z_bstride, const float* bias,
                    int B, int d, int r, int m, int overlap, int64_t e_begin, int64_t n_e,
                    void* out, int out_fmt, uint8_t* out_scales, int64_t out_bstride, int64_t sc_bstride)
{
    if (B < 0 || n_e < 0 || !compress_args_ok(x_fmt, x_roles, overlap, d, m, z_ch)) return ORC_EINVAL;
    const int win = overlap ? 2 * m : m;
    const int64_t orb = orc_row_bytes(out_fmt, d, r);
    if (x_rows <= 0) {
        /* every valid window position must be present in the linear raw buffer */
        for (int64_t q = 0; q < n_e; ++q) {
            int64_t i = e_begin + q;
            for (int j = 0; j < win; ++j) {
                int64_t p = (i + 1) * m - win + j;
                if (p >= 0 && (p < x_pos0 || p >= x_pos0 + n_tok)) return ORC_EINVAL;
            }
        }
    }
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b) {
        for (int64_t q = 0; q < n_e; ++q) {
            uint8_t* o = (uint8_t*)out + b * out_bstride + q * orb;
            uint8_t* sc = out_scales ? out_scales + b * sc_bstride + q * (d / 32) : NULL;
            compress_entry(x, x_fmt, x_bstride, x_pos0, x_rows, x_roles, z, z_ch, z_bstride, bias, b, d, r, m,
                           overlap, e_begin + q, out_fmt, o, sc);
        }
    }
    return ORC_OK;
}

/*
 * Decode-time compression: for every new token (b, j) at position p = pos[b*T + j]
 * that completes a block ((p + 1) mod m == 0), entry e = (p + 1)/m - 1 is pooled from
 * the ring of raw rows (slot p mod x_rows, x_pos0 = 0) and written at out +
 * (b*T + j)*rowbytes (scales at out_scales + (b*T + j)*d/32); out_entry[b*T + j] = e,
 * or -1 when the token completes no block (nothing written).
 */
int orc_kv_compress_step(const void* x, int x_fmt, int64_t x_bstride, int64_t x_rows, int x_roles,
                         const float* z, int z_ch, int64_t z_bstride, const float* bias,
                         const int32_t* pos, int B, int T, int d, int r, int m, int overlap,
                         void* out, int out_fmt, uint8_t* out_scales, int32_t* out_entry)
{
    if (B < 0 || T < 0 || x_rows <= 0 || !compress_args_ok(x_fmt, x_roles, overlap, d, m, z_ch)) return ORC_EINVAL;
    const int64_t orb = orc_row_bytes(out_fmt, d, r);
    for (int64_t u = 0; u < (int64_t)B * T; ++u) {
        const int64_t p = pos[u];
        const int b = (int)(u / (T > 0 ? T : 1));
        if (p < 0 || (p + 1) % m != 0) { out_entry[u] = -1; continue; }
        const int64_t e = (p + 1) / m - 1;
        out_entry[u] = (int32_t)e;
        compress_entry(x, x_fmt, x_bstride, 0, x_rows, x_roles, z, z_ch, z_bstride, bias, b, d, r, m, overlap, e,
                       out_fmt, (uint8_t*)out + u * orb, out_scales ? out_scales + u * (d / 32) : NULL);
    }
    return ORC_OK;
}

/*
 * Plain paged gather: row s of sequence b, stored in block block_table[b*bt_stride +
 * s / epb] of the pool at byte offset (s % epb)*row_bytes of that block (blocks
 * block_bytes apart), copied to out + b*out_bstride + s*row_bytes for s < n.  A
 * negative block id (no block) gives a zero row.
 */
void orc_paged_gather(const uint8_t* pool, int64_t row_bytes, const int32_t* block_table, int64_t bt_stride,
                      int epb, int64_t block_bytes, int B, int64_t n, uint8_t* out, int64_t out_bstride)
{
    for (int b = 0; b < B; ++b)
        for (int64_t s = 0; s < n; ++s) {
            const int32_t blk = block_table[b * bt_stride + s / epb];
            uint8_t* dst = out + b * out_bstride + s * row_bytes;
            if (blk < 0) memset(dst, 0, (size_t)row_bytes);
            else memcpy(dst, pool + (int64_t)blk * block_bytes + (s % epb) * row_bytes, (size_t)row_bytes);
        }
}

/* ------------------------------------------------------------------------- */
/* Lightning indexer + top-k ([X] CSA step 2).                                */
/* ------------------------------------------------------------------------- */

typedef struct { double score; int64_t idx; } cand_t;

static int cand_cmp(const void* a, const void* b)
{
    const cand_t* x = (const cand_t*)a;
    const cand_t* y = (const cand_t*)b;
    if (x->score > y->score) return -1;   /* higher score first */
    if (x->score < y->score) return 1;
    return (x->idx < y->idx) ? -1 : (x->idx > y->idx); /* ties: smaller index first */
}

static int idx_cmp(const void* a, const void* b)
{
    const cand_t* x = (const cand_t*)a;
    const cand_t* y = (const cand_t*)b;
    return (x->idx < y->idx) ? -1 : (x->idx > y->idx);
}

/* Number of compressed entries complete at query position t. */
static int64_t n_visible(int64_t t, int m, int64_t n_cap)
{
    if (t < 0) return 0;
    int64_t n = (t + 1) / m;
    return n < n_cap ? n : n_cap;
}

/*
 * For each query (b, j) at position t = q_pos[b*Tq + j]:
 *   score(s) = sum_h w[b,j,h] * max(0, sum_i qi[b,j,h,i] * ki[b,s,i]),  s < n_visible(t)
 * keep the k best by (score desc, index asc), write them ascending by index,
 * pad with -1 (and -inf scores).  qi is dense [B][Tq][H_I][d_I] in qi_fmt (scales
 * [B][Tq][H_I][d_I/32] for MXFP4); ki rows of sequence b start at ki + b*ki_bstride
 * (scales at ki_scales + b*ks_bstride).  `out_score` may be NULL.
 */
int orc_index_topk(const void* qi, int qi_fmt, const uint8_t* qi_scales, const float* w,
                   const void* ki, int ki_fmt, const uint8_t* ki_scales, int64_t ki_bstride, int64_t ks_bstride,
                   const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int m, int64_t n_cap, int k,
                   int32_t* out_idx, float* out_score)
{
    if (B < 0 || Tq < 0 || H_I <= 0 || d_I <= 0 || m <= 0 || k <= 0 || n_cap < 0) return ORC_EINVAL;
    const int64_t qrb = orc_row_bytes(qi_fmt, d_I, 0), krb = orc_row_bytes(ki_fmt, d_I, 0);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        for (int j = 0; j < Tq; ++j) {
            const int64_t t = q_pos[(int64_t)b * Tq + j];
            const int64_t n = n_visible(t, m, n_cap);
            double* q = (double*)malloc(sizeof(double) * (size_t)H_I * d_I);
            double* kr = (double*)malloc(sizeof(double) * (size_t)d_I);
            cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)(n > 0 ? n : 1));
            const int64_t qrow0 = ((int64_t)b * Tq + j) * H_I;
            for (int h = 0; h < H_I; ++h)
                decode_row((const uint8_t*)qi + (qrow0 + h) * qrb,
                           qi_scales ? qi_scales + (qrow0 + h) * (d_I / 32) : NULL, qi_fmt, d_I, 0, q + (size_t)h * d_I);
            const float* wr = w + qrow0;
            for (int64_t s = 0; s < n; ++s) {
                decode_row((const uint8_t*)ki + b * ki_bstride + s * krb,
                           ki_scales ? ki_scales + b * ks_bstride + s * (d_I / 32) : NULL, ki_fmt, d_I, 0, kr);
                double sc = 0.0;
                for (int h = 0; h < H_I; ++h) {
                    double dot = 0.0;
                    for (int i = 0; i < d_I; ++i) dot += q[(size_t)h * d_I + i] * kr[i];
                    sc += (double)wr[h] * (dot > 0.0 ? dot : 0.0);
                }
                c[s].score = sc;
                c[s].idx = s;
            }
            qsort(c, (size_t)n, sizeof(cand_t), cand_cmp);
            int64_t kk = n < k ? n : k;
            qsort(c, (size_t)kk, sizeof(cand_t), idx_cmp);
            int32_t* oi = out_idx + ((int64_t)b * Tq + j) * k;
            float* os = out_score ? out_score + ((int64_t)b * Tq + j) * k : NULL;
            for (int64_t a = 0; a < k; ++a) {
                oi[a] = a < kk ? (int32_t)c[a].idx : -1;
                if (os) os[a] = a < kk ? (float)c[a].score : -INFINITY;
            }
            free(q); free(kr); free(c);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Shared-KV MQA over {entries} U {sliding window} ([X] CSA step 3, HCA).     */
/* ------------------------------------------------------------------------- */

/* Stored row of window position p: slot (p - pos0) mod rows. */
static const uint8_t* window_row(const uint8_t* base, int64_t pos0, int64_t rows, int64_t rb, int64_t p)
{
    int64_t s = (p - pos0) % rows;
    if (s < 0) s += rows;
    return base + s * rb;
}

/*
 * One query (b, j), all heads:  the attended set is a list L of stored rows (K = V),
 * logits l = scale * q_h . v, o_h = sum softmax(l) v, lse_h = log sum exp(l).
 * With a sink (sink != NULL) head h's softmax also has the logit sink[h], which has
 * no value:  o_h = sum exp(l) v / (exp(sink[h]) + sum exp(l)),  lse_h = log(exp(sink[h])
 * + sum exp(l)).  An empty list gives o = 0 and lse = -inf (= sink[h] with a sink).
 */
static void attend_list(const double* q, int H, int d, double scale, double* const* rows, int64_t nrows,
                        const float* sink, float* out_f32, uint16_t* out_bf16, float* lse)
{
    double* l = (double*)malloc(sizeof(double) * (size_t)(nrows > 0 ? nrows : 1));
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
    for (int h = 0; h < H; ++h) {
        double mx = -INFINITY;
        for (int64_t a = 0; a < nrows; ++a) {
            double dot = 0.0;
            for (int i = 0; i < d; ++i) dot += q[(size_t)h * d + i] * rows[a][i];
            l[a] = scale * dot;
            if (l[a] > mx) mx = l[a];
        }
        if (sink && (double)sink[h] > mx) mx = sink[h];
        double den = 0.0;
        for (int64_t a = 0; a < nrows; ++a) den += exp(l[a] - mx);
        if (sink) den += exp((double)sink[h] - mx);
        for (int i = 0; i < d; ++i) o[i] = 0.0;
        for (int64_t a = 0; a < nrows; ++a) {
            double p = exp(l[a] - mx) / den;
            for (int i = 0; i < d; ++i) o[i] += p * rows[a][i];
        }
        for (int i = 0; i < d; ++i) {
            if (out_f32) out_f32[(size_t)h * d + i] = (float)o[i];
            if (out_bf16) out_bf16[(size_t)h * d + i] = orc_bf16_encode(o[i]);
        }
        if (lse) lse[h] = den > 0.0 ? (float)(mx + log(den)) : -INFINITY;
    }
    free(l); free(o);
}

/*
 * Common driver of both attention calls.  For query (b, j) at t = q_pos[b*Tq+j]:
 *   entries:  CSA -- the listed indices idx[b,j,0..k-1] that lie in [0, n_cap)
 *             HCA -- every s < n_visible(t)      (idx == NULL selects this)
 *   window:   positions max(0, t-W+1) .. t, stored as described in window_row.
 * q is dense [B][Tq][H][d] (f32 or bf16), out is [B][Tq][H][d] (f32 or bf16),
 * lse [B][Tq][H] (nullable).
 */
static int attend_common(const void* q, int q_fmt, const void* kv_c, int kv_fmt, int64_t kvc_bstride, int64_t n_cap,
                         const int32_t* idx, int k, int m,
                         const void* kv_w, int64_t kvw_bstride, int64_t kvw_pos0, int64_t kvw_rows,
                         const float* sink, const int32_t* q_pos, int W, int B, int Tq, int H, int d, int r,
                         double scale, void* out, int out_fmt, float* out_lse)
{
    if (B < 0 || Tq < 0 || H <= 0 || d <= 0 || W < 0 || n_cap < 0) return ORC_EINVAL;
    if (W > 0 && kvw_rows <= 0) return ORC_EINVAL;
    if (q_fmt != ORC_F32 && q_fmt != ORC_BF16) return ORC_EINVAL;
    if (out_fmt != ORC_F32 && out_fmt != ORC_BF16) return ORC_EINVAL;
    const int64_t rb = orc_row_bytes(kv_fmt, d, r), qrb = orc_row_bytes(q_fmt, d, r);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        for (int j = 0; j < Tq; ++j) {
            const int64_t t = q_pos[(int64_t)b * Tq + j];
            int64_t ne = 0, nw = 0;
            if (idx) {
                const int32_t* ix = idx + ((int64_t)b * Tq + j) * k;
                for (int a = 0; a < k; ++a) ne += (ix[a] >= 0 && ix[a] < n_cap);
            } else {
                ne = n_visible(t, m, n_cap);
            }
            int64_t w0 = t - W + 1;
            if (w0 < 0) w0 = 0;
            nw = (t >= 0 && W > 0) ? t - w0 + 1 : 0;
            const int64_t nrows = ne + nw;
            double* data = (double*)malloc(sizeof(double) * (size_t)(nrows > 0 ? nrows : 1) * d);
            double** rows = (double**)malloc(sizeof(double*) * (size_t)(nrows > 0 ? nrows : 1));
            int64_t a = 0;
            if (idx) {
                const int32_t* ix = idx + ((int64_t)b * Tq + j) * k;
                for (int u = 0; u < k; ++u) {
                    if (ix[u] < 0 || ix[u] >= n_cap) continue;
                    rows[a] = data + (size_t)a * d;
                    decode_row((const uint8_t*)kv_c + b * kvc_bstride + (int64_t)ix[u] * rb, NULL, kv_fmt, d, r, rows[a]);
                    ++a;
                }
            } else {
                for (int64_t s = 0; s < ne; ++s) {
                    rows[a] = data + (size_t)a * d;
                    decode_row((const uint8_t*)kv_c + b * kvc_bstride + s * rb, NULL, kv_fmt, d, r, rows[a]);
                    ++a;
                }
            }
            for (int64_t p = w0; p < w0 + nw; ++p) {
                rows[a] = data + (size_t)a * d;
                decode_row(window_row((const uint8_t*)kv_w + b * kvw_bstride, kvw_pos0, kvw_rows, rb, p), NULL,
                           kv_fmt, d, r, rows[a]);
                ++a;
            }
            double* qd = (double*)malloc(sizeof(double) * (size_t)H * d);
            const int64_t qrow0 = ((int64_t)b * Tq + j) * H;
            for (int h = 0; h < H; ++h)
                decode_row((const uint8_t*)q + (qrow0 + h) * qrb, NULL, q_fmt, d, r, qd + (size_t)h * d);
            float* of = out_fmt == ORC_F32 ? (float*)out + qrow0 * d : NULL;
            uint16_t* ob = out_fmt == ORC_BF16 ? (uint16_t*)out + qrow0 * d : NULL;
            attend_list(qd, H, d, scale, rows, nrows, sink, of, ob, out_lse ? out_lse + qrow0 : NULL);
            free(qd); free(rows); free(data);
        }
    }
    return ORC_OK;
}

int orc_csa_attend(const void* q, int q_fmt, const void* kv_c, int kv_fmt, int64_t kvc_bstride, int64_t n_cap,
                   const int32_t* idx, int k,
                   const void* kv_w, int64_t kvw_bstride, int64_t kvw_pos0, int64_t kvw_rows, const float* sink,
                   const int32_t* q_pos, int W, int B, int Tq, int H, int d, int r, double scale,
                   void* out, int out_fmt, float* out_lse)
{
    if (!idx || k <= 0) return ORC_EINVAL;
    return attend_common(q, q_fmt, kv_c, kv_fmt, kvc_bstride, n_cap, idx, k, 1, kv_w, kvw_bstride, kvw_pos0,
                         kvw_rows, sink, q_pos, W, B, Tq, H, d, r, scale, out, out_fmt, out_lse);
}

int orc_hca_attend(const void* q, int q_fmt, const void* kv_c, int kv_fmt, int64_t kvc_bstride, int64_t n_cap, int m,
                   const void* kv_w, int64_t kvw_bstride, int64_t kvw_pos0, int64_t kvw_rows, const float* sink,
                   const int32_t* q_pos, int W, int B, int Tq, int H, int d, int r, double scale,
                   void* out, int out_fmt, float* out_lse)
{
    if (m <= 0) return ORC_EINVAL;
    return attend_common(q, q_fmt, kv_c, kv_fmt, kvc_bstride, n_cap, NULL, 0, m, kv_w, kvw_bstride, kvw_pos0,
                         kvw_rows, sink, q_pos, W, B, Tq, H, d, r, scale, out, out_fmt, out_lse);
}

/* ------------------------------------------------------------------------- */
/* Grouped output projection ([X] HCA subsection; [C] attention details).    */
/* ------------------------------------------------------------------------- */
/*
 * x: M rows of G*K values (row t = the outputs of the H heads of token t, head-major,
 * so group g holds values g*K .. g*K+K-1); w: G matrices of R rows of K values (row n
 * of matrix g = the weights of output n of group g).  out[t][g*R + n] =
 * sum_k x[t][g*K + k] * w[g][n][k], in fp64, stored as fp32.  x_fmt / w_fmt: F32 or BF16.
 */
int orc_grouped_out_proj(const void* x, int x_fmt, const void* w, int w_fmt, int M, int G, int K, int R,
                         float* out)
{
    if (M < 0 || G <= 0 || K <= 0 || R <= 0) return ORC_EINVAL;
    if ((x_fmt != ORC_F32 && x_fmt != ORC_BF16) || (w_fmt != ORC_F32 && w_fmt != ORC_BF16)) return ORC_EINVAL;
    const int64_t xrb = orc_row_bytes(x_fmt, G * K, 0), wrb = orc_row_bytes(w_fmt, K, 0);
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < M; ++t) {
        double* xr = (double*)malloc(sizeof(double) * (size_t)G * K);
        double* wr = (double*)malloc(sizeof(double) * (size_t)K);
        decode_row((const uint8_t*)x + (int64_t)t * xrb, NULL, x_fmt, G * K, 0, xr);
        for (int g = 0; g < G; ++g)
            for (int n = 0; n < R; ++n) {
                decode_row((const uint8_t*)w + ((int64_t)g * R + n) * wrb, NULL, w_fmt, K, 0, wr);
                double acc = 0.0;
                for (int k = 0; k < K; ++k) acc += xr[(size_t)g * K + k] * wr[k];
                out[(int64_t)t * G * R + (int64_t)g * R + n] = (float)acc;
            }
        free(xr); free(wr);
    }
    return ORC_OK;
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
