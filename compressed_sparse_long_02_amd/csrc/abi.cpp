// abi.cpp -- the C ABI of libcsl.so (declared in include/csl.h): host-side argument
// validation (before anything touches the GPU), launch planning (slices, splits,
// workspace), device check, and dispatch to the kernel launchers.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "csl.h"
#include "launch.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool al4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// Per-device cache: is the device a gfx950?
std::mutex g_dev_mu;
int g_dev_ok[64];  // 0 unknown, 1 ok, -1 not gfx950

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(CSL_EDEVICE, "no HIP device is current");
    if (dev >= 64) return fail(CSL_EDEVICE, "device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_ok[dev] == 0) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) return fail(CSL_EDEVICE, "cannot query device %d", dev);
        g_dev_ok[dev] = std::strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    }
    if (g_dev_ok[dev] < 0) return fail(CSL_EUNSUPPORTED, "device %d is not a gfx950 (MI355X)", dev);
    return CSL_OK;
}

int launched(hipError_t e) {
    if (e != hipSuccess) return fail(CSL_ELAUNCH, "launch failed: %s", hipGetErrorString(e));
    g_err.clear();
    return CSL_OK;
}

// ---- planning (also used by the workspace queries) -------------------------
constexpr int MAX_SLICES = 1024;        // slices of one query (the row select scans their counts in one pass)
constexpr int MAX_S = 16384;            // keys one scoring block holds in LDS
constexpr int64_t MAX_NCAP = (int64_t)MAX_S * MAX_SLICES;

// Slices of S keys (a power of two in [512, 16384]), about 256 scoring blocks in all
// (one per compute unit: long contiguous streams; the block's waves balance among
// themselves).  One slice per query: the block selects; several: the split path over
// score rows.
void plan_index(int B, int Tq, int64_t n_cap, int& S, int& nslices) {
    const int64_t target_blocks = 256;
    const int64_t work = (n_cap > 0 ? n_cap : 1) * (int64_t)(B > 0 ? B : 1) * (Tq > 0 ? Tq : 1);
    const int64_t need = (work + target_blocks - 1) / target_blocks;
    S = 512;   // at least one key per thread of the 512-thread scoring block
    while (S < need && S < MAX_S) S <<= 1;
    while (n_cap > (int64_t)S * MAX_SLICES && S < MAX_S) S <<= 1;
    nslices = n_cap <= 0 ? 1 : (int)((n_cap + S - 1) / S);
}

int64_t row_stride(int64_t n_cap) { return n_cap < 4 ? 4 : (n_cap + 3) & ~(int64_t)3; }

size_t index_ws(int B, int Tq, int64_t n_cap, int nslices) {
    if (nslices <= 1) return 0;
    const size_t q = (size_t)B * Tq;
    return q * ((size_t)3 * row_stride(n_cap) + (size_t)nslices * (csl::IDX_SLOT_W + 1) + 4) * 4 + 256;
}

// Split path: slices per filter block, about 256 filter blocks (one per compute unit) in all.
int index_spb(int B, int Tq, int nslices) {
    const int64_t q = (int64_t)(B > 0 ? B : 1) * (Tq > 0 ? Tq : 1);
    int64_t spb = ((int64_t)nslices * q + 255) / 256;
    return (int)(spb < 1 ? 1 : (spb > nslices ? nslices : spb));
}

constexpr int ATT_STEP = 32;            // rows a block stages per iteration; split lengths are multiples
constexpr int ATT_TARGET_BLOCKS = 256;  // one block (8 waves, two per SIMD) per compute unit
constexpr int ATT_MIN_RPS = 64;
constexpr int ATT_MAX_SPLIT = 128;

constexpr int ATT_MAX_CSA_RPS = 1536;   // rows of a CSA split whose indices are staged in LDS

void plan_attend(int B, int Tq, int H, int64_t rows_max, bool csa, int& nhb, int& nsplit, int& rps) {
    nhb = (H + 63) / 64;
    const int64_t L = rows_max > 0 ? rows_max : 1;
    const int64_t total_q = (int64_t)B * Tq * nhb;
    int64_t ns = total_q > 0 ? (ATT_TARGET_BLOCKS + total_q - 1) / total_q : 1;
    if (ns < 1) ns = 1;
    if (ns > ATT_MAX_SPLIT) ns = ATT_MAX_SPLIT;
    int64_t r = (L + ns - 1) / ns;
    r = (r + ATT_STEP - 1) / ATT_STEP * ATT_STEP;
    if (r < ATT_MIN_RPS) r = ATT_MIN_RPS;
    if (csa && r > ATT_MAX_CSA_RPS) r = ATT_MAX_CSA_RPS;
    rps = (int)r;
    nsplit = (int)((L + r - 1) / r);
}

size_t attend_ws(int B, int Tq, int d, int nhb, int nsplit) {
    if (nsplit <= 1) return 0;
    const size_t rows = (size_t)B * Tq * nhb * nsplit * 64;
    return rows * (size_t)d * 4 + rows * 4 + 512;
}

int64_t row_bytes(int fmt, int d, int r) {
    switch (fmt) {
    case CSL_F32: return 4 * (int64_t)d;
    case CSL_BF16: return 2 * (int64_t)d;
    case CSL_KV_PACKED: return 2 * (int64_t)r + (d - r);
    case CSL_MXFP4: return (int64_t)d / 2;
    default: return -1;
    }
}

int validate_attend(const char* fn, const void* q, int q_fmt, const void* kv_c, int kv_fmt, int64_t kvc_bstride,
                    int64_t n_cap, const void* kv_w, int64_t kvw_bstride, int64_t kvw_rows, const int32_t* q_pos,
                    int W, int B, int Tq, int H, int d, int r, void* out, int out_fmt) {
    if (B < 0 || Tq < 0) return fail(CSL_EINVAL, "%s: negative B or Tq", fn);
    if ((int64_t)B * Tq > 65535) return fail(CSL_EUNSUPPORTED, "%s: B*Tq = %lld exceeds 65535", fn, (long long)B * Tq);
    if (H < 1 || W < 0 || n_cap < 0) return fail(CSL_EINVAL, "%s: need H >= 1, W >= 0, n_cap >= 0", fn);
    if (d != 64 && d != 128 && d != 256 && d != 512) return fail(CSL_EUNSUPPORTED, "%s: d = %d not in {64,128,256,512}", fn, d);
    if (kv_fmt != CSL_F32 && kv_fmt != CSL_BF16 && kv_fmt != CSL_KV_PACKED)
        return fail(CSL_EUNSUPPORTED, "%s: kv_fmt %d not supported (F32, BF16, KV_PACKED)", fn, kv_fmt);
    if ((kv_fmt == CSL_F32) != (q_fmt == CSL_F32) || (q_fmt != CSL_F32 && q_fmt != CSL_BF16))
        return fail(CSL_EUNSUPPORTED, "%s: q_fmt must be F32 with F32 KV and BF16 with BF16/packed KV", fn);
    if (kv_fmt == CSL_KV_PACKED && (r < 0 || r > d || r % 8 != 0 || (d - r) % 16 != 0 || (d + r) % 16 != 0))
        return fail(CSL_EINVAL, "%s: packed rows need r %% 8 == 0, (d-r) %% 16 == 0, (d+r) %% 16 == 0", fn);
    if (kv_fmt == CSL_KV_PACKED && 4 * r > d)
        return fail(CSL_EUNSUPPORTED, "%s: packed rows with r = %d > d/4 are not built", fn, r);
    if (out_fmt != CSL_F32 && out_fmt != CSL_BF16) return fail(CSL_EINVAL, "%s: out_fmt must be F32 or BF16", fn);
    if (B * (int64_t)Tq == 0) return CSL_OK;
    if (!q || !q_pos || !out) return fail(CSL_EINVAL, "%s: null q, q_pos or out", fn);
    if (n_cap > 0 && !kv_c) return fail(CSL_EINVAL, "%s: null kv_c with n_cap > 0", fn);
    if (W > 0 && (!kv_w || kvw_rows < 1)) return fail(CSL_EINVAL, "%s: W > 0 needs kv_w and kvw_rows >= 1", fn);
    if (!al16(q) || !al16(out) || !al16(kv_c) || !al16(kv_w) || !al4(q_pos))
        return fail(CSL_EINVAL, "%s: q/kv_c/kv_w/out must be 16-byte aligned", fn);
    if ((kvc_bstride & 15) || (kvw_bstride & 15)) return fail(CSL_EINVAL, "%s: byte strides must be multiples of 16", fn);
    (void)row_bytes;
    return CSL_OK;
}

}  // namespace

extern "C" {

int64_t csl_row_bytes(int fmt, int d, int r) { return row_bytes(fmt, d, r); }

const char* csl_status_string(int status) {
    switch (status) {
    case CSL_OK: return "ok";
    case CSL_EINVAL: return "invalid argument";
    case CSL_EUNSUPPORTED: return "unsupported configuration";
    case CSL_EWORKSPACE: return "workspace missing or too small";
    case CSL_ELAUNCH: return "kernel launch failed";
    case CSL_EDEVICE: return "no usable gfx950 device";
    default: return "unknown status";
    }
}

int csl_last_error(char* buf, size_t n) {
    if (buf && n) {
        std::strncpy(buf, g_err.c_str(), n - 1);
        buf[n - 1] = 0;
    }
    return (int)g_err.size();
}

int csl_version(void) { return 100; }

int kv_compress(const void* x, int x_fmt, int64_t x_bstride, int64_t x_pos0, int64_t n_tok,
                const float* z, int z_ch, int64_t z_bstride, const float* bias,
                int B, int d, int r, int m, int overlap, int64_t e_begin, int64_t n_e,
                void* out, int out_fmt, uint8_t* out_scales, int64_t out_bstride, int64_t sc_bstride,
                void* stream) {
    const char* fn = "kv_compress";
    if (B < 0 || n_e < 0 || n_tok < 0 || e_begin < 0) return fail(CSL_EINVAL, "%s: negative size", fn);
    if (B > 65535) return fail(CSL_EUNSUPPORTED, "%s: B > 65535", fn);
    if (m < 1) return fail(CSL_EINVAL, "%s: m must be >= 1", fn);
    if (d < 32 || d > 1024 || d % 32) return fail(CSL_EUNSUPPORTED, "%s: d = %d must be a multiple of 32 in [32, 1024]", fn, d);
    if (x_fmt != CSL_F32 && x_fmt != CSL_BF16) return fail(CSL_EINVAL, "%s: x_fmt must be F32 or BF16", fn);
    if (out_fmt < CSL_F32 || out_fmt > CSL_MXFP4) return fail(CSL_EINVAL, "%s: unknown out_fmt %d", fn, out_fmt);
    if (out_fmt == CSL_KV_PACKED && (r < 0 || r > d || r % 8 || (d + r) % 16))
        return fail(CSL_EINVAL, "%s: packed output needs r %% 8 == 0, (d + r) %% 16 == 0, 0 <= r <= d", fn);
    if (z_ch != 1 && z_ch != d) return fail(CSL_EINVAL, "%s: z_ch must be 1 or d", fn);
    if ((int64_t)n_e * m > ((int64_t)1 << 40)) return fail(CSL_EINVAL, "%s: entry range too large", fn);
    if (B == 0 || n_e == 0) { g_err.clear(); return CSL_OK; }
    if (!x || !z || !bias || !out) return fail(CSL_EINVAL, "%s: null x, z, bias or out", fn);
    if ((out_fmt == CSL_MXFP4) != (out_scales != nullptr)) return fail(CSL_EINVAL, "%s: out_scales must be given exactly for MXFP4", fn);
    if (!al16(x) || (x_bstride & 15) || !al16(out) || (out_bstride & 15))
        return fail(CSL_EINVAL, "%s: x/out and their strides must be 16-byte aligned", fn);
    if (z_ch == d ? (!al16(z) || (z_bstride & 15) || !al16(bias)) : (!al4(z) || (z_bstride & 3) || !al4(bias)))
        return fail(CSL_EINVAL, "%s: z/bias misaligned", fn);
    const int win = overlap ? 2 * m : m;
    int64_t lo = (e_begin + 1) * m - win;
    if (lo < 0) lo = 0;
    const int64_t hi = (e_begin + n_e) * m - 1;
    if (lo < x_pos0 || hi >= x_pos0 + n_tok)
        return fail(CSL_EINVAL, "%s: raw positions %lld..%lld are not all in the buffer [%lld, %lld)", fn,
                    (long long)lo, (long long)hi, (long long)x_pos0, (long long)(x_pos0 + n_tok));
    int rc = check_device();
    if (rc) return rc;
    csl::CompressArgs a{(const uint8_t*)x, x_fmt, x_bstride, x_pos0, n_tok, z, z_ch, z_bstride, bias,
                        B, d, r, m, overlap ? 1 : 0, e_begin, n_e,
                        (uint8_t*)out, out_fmt, out_scales, out_bstride, sc_bstride};
    return launched(csl::launch_compress(a, (hipStream_t)stream));
}

// Many queries per call (prefill): the dense path scores every (query, key) pair into
// the workspace, a pass of at most DENSE_WS_MAX bytes at a time.
constexpr int DENSE_MIN_TQ = 64;
constexpr size_t DENSE_WS_MAX = (size_t)2 << 30;

bool dense_path(int fmt, int d_I, int H_I, int Tq) {
    return fmt == CSL_BF16 && d_I == 128 && (H_I == 16 || H_I == 32 || H_I == 64 || H_I == 128) && Tq >= DENSE_MIN_TQ;
}
int dense_tc(int B, int Tq, int64_t n_cap) {
    // queries per pass: a multiple of 12 (the score kernel's query group), the passes
    // as even as possible, each within DENSE_WS_MAX
    const size_t per_q = (size_t)(B > 0 ? B : 1) * ((size_t)row_stride(n_cap) + 2048) * 4;
    size_t cap = (DENSE_WS_MAX / per_q) / 12 * 12;
    if (cap < 12) cap = 12;
    const size_t tq = Tq > 0 ? (size_t)Tq : 1;
    const size_t passes = (tq + cap - 1) / cap;
    const size_t tc = ((tq + passes - 1) / passes + 11) / 12 * 12;
    return (int)(tc < cap ? tc : cap);
}
size_t dense_ws(int B, int Tq, int64_t n_cap) {
    return (size_t)B * dense_tc(B, Tq, n_cap) * ((size_t)row_stride(n_cap) + 2048) * 4 + 256;
}

size_t csl_index_topk_workspace(int B, int Tq, int64_t n_cap, int k) {
    if (B < 0 || Tq < 0 || k < 1) return 0;
    int S, ns;
    plan_index(B, Tq, n_cap, S, ns);
    size_t ws = index_ws(B, Tq, n_cap, ns);
    if (Tq >= DENSE_MIN_TQ) {                            // the dense path may be taken (fmt, d_I, H_I unknown here)
        const size_t d = dense_ws(B, Tq, n_cap);
        ws = d > ws ? d : ws;
    }
    return ws;
}

int index_topk(const void* qi, int qi_fmt, const uint8_t* qi_scales, const float* w,
               const void* ki, int ki_fmt, const uint8_t* ki_scales, int64_t ki_bstride, int64_t ks_bstride,
               const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int m, int64_t n_cap, int k,
               int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "index_topk";
    if (B < 0 || Tq < 0 || n_cap < 0) return fail(CSL_EINVAL, "%s: negative size", fn);
    if (B > 65535 || Tq > 65535) return fail(CSL_EUNSUPPORTED, "%s: B and Tq must be <= 65535", fn);
    if (m < 1) return fail(CSL_EINVAL, "%s: m must be >= 1", fn);
    if (k < 1 || k > 2048) return fail(CSL_EUNSUPPORTED, "%s: k = %d not in [1, 2048]", fn, k);
    if (H_I < 1 || H_I > 128) return fail(CSL_EUNSUPPORTED, "%s: H_I = %d not in [1, 128]", fn, H_I);
    if (qi_fmt != ki_fmt) return fail(CSL_EUNSUPPORTED, "%s: qi_fmt and ki_fmt must match", fn);
    const bool dok = (ki_fmt == CSL_F32 && (d_I == 32 || d_I == 128)) ||
                     (ki_fmt == CSL_BF16 && (d_I == 32 || d_I == 64 || d_I == 128)) ||
                     (ki_fmt == CSL_MXFP4 && d_I == 128);
    if (!dok) return fail(CSL_EUNSUPPORTED, "%s: (fmt %d, d_I %d) not built", fn, ki_fmt, d_I);
    const bool dense = dense_path(ki_fmt, d_I, H_I, Tq);
    if (n_cap > MAX_NCAP) return fail(CSL_EUNSUPPORTED, "%s: n_cap must be <= 2^24", fn);
    int S = 0, nslices = 1;
    if (!dense) plan_index(B, Tq, n_cap, S, nslices);
    const size_t need = dense ? dense_ws(B, Tq, n_cap) : index_ws(B, Tq, n_cap, nslices);
    if (B * (int64_t)Tq == 0) { g_err.clear(); return CSL_OK; }
    if (!qi || !w || !q_pos || !out_idx || (n_cap > 0 && !ki)) return fail(CSL_EINVAL, "%s: null pointer argument", fn);
    if ((ki_fmt == CSL_MXFP4) != (qi_scales != nullptr) || (ki_fmt == CSL_MXFP4) != (ki_scales != nullptr || n_cap == 0))
        return fail(CSL_EINVAL, "%s: scale arrays must be given exactly for MXFP4", fn);
    if (!al16(qi) || !al16(ki) || (ki_bstride & 15) || !al4(w) || !al4(q_pos) || !al4(out_idx) || !al4(out_score))
        return fail(CSL_EINVAL, "%s: misaligned pointer or stride", fn);
    if (need > 0 && (!ws || ws_bytes < need || !al16(ws)))
        return fail(CSL_EWORKSPACE, "%s: needs %zu bytes of 16-byte aligned workspace", fn, need);
    int rc = check_device();
    if (rc) return rc;
    csl::IndexArgs a{};
    a.qi = (const uint8_t*)qi; a.qi_fmt = qi_fmt; a.qi_scales = qi_scales; a.w = w;
    a.ki = (const uint8_t*)ki; a.ki_fmt = ki_fmt; a.ki_scales = ki_scales; a.ki_bstride = ki_bstride; a.ks_bstride = ks_bstride;
    a.q_pos = q_pos; a.B = B; a.Tq = Tq; a.H_I = H_I; a.d_I = d_I; a.m = m; a.n_cap = n_cap; a.k = k;
    a.out_idx = out_idx; a.out_score = out_score;
    a.S = S; a.nslices = nslices;
    if (dense) {
        a.dense = 1;
        a.Tc = dense_tc(B, Tq, n_cap);
        a.sstride = row_stride(n_cap);
        a.scores = (uint32_t*)ws;
        a.hist = (uint32_t*)((uint8_t*)ws + (size_t)B * a.Tc * a.sstride * 4);
    } else if (nslices > 1) {
        a.spb = index_spb(B, Tq, nslices);
        a.sstride = row_stride(n_cap);
        const size_t q = (size_t)B * Tq;
        const size_t nr = q * a.sstride * 4;           // bytes of one [B*Tq][sstride] array
        a.scores = (uint32_t*)ws;
        a.cand_key = (uint32_t*)((uint8_t*)ws + nr);
        a.cand_idx = (int32_t*)((uint8_t*)ws + 2 * nr);
        a.hist = (uint32_t*)((uint8_t*)ws + 3 * nr);
        a.seg_cnt = (int32_t*)(a.hist + q * nslices * csl::IDX_SLOT_W);
        a.row_bin = (uint32_t*)(a.seg_cnt + q * nslices);
    }
    return launched(csl::launch_index_topk(a, (hipStream_t)stream));
}

size_t csl_attend_workspace(int B, int Tq, int H, int d, int64_t rows_max) {
    if (B < 0 || Tq < 0 || H < 1) return 0;
    int nhb, nsplit, rps;
    plan_attend(B, Tq, H, rows_max, true, nhb, nsplit, rps);   // the CSA cap only adds splits
    return attend_ws(B, Tq, d, nhb, nsplit);
}

static int attend_impl(const char* fn, const void* q, int q_fmt, const void* kv_c, int kv_fmt, int64_t kvc_bstride,
                       int64_t n_cap, const int32_t* idx, int k, int m, const void* kv_w, int64_t kvw_bstride,
                       int64_t kvw_pos0, int64_t kvw_rows, const int32_t* q_pos, int W, int B, int Tq, int H, int d,
                       int r, float scale, void* out, int out_fmt, float* out_lse, void* ws, size_t ws_bytes,
                       void* stream) {
    int rc = validate_attend(fn, q, q_fmt, kv_c, kv_fmt, kvc_bstride, n_cap, kv_w, kvw_bstride, kvw_rows, q_pos, W,
                             B, Tq, H, d, r, out, out_fmt);
    if (rc) return rc;
    const int64_t rows_max = (idx ? (int64_t)k : n_cap) + W;
    int nhb, nsplit, rps;
    plan_attend(B, Tq, H, rows_max, true, nhb, nsplit, rps);
    const size_t need = attend_ws(B, Tq, d, nhb, nsplit);
    if (B * (int64_t)Tq == 0) { g_err.clear(); return CSL_OK; }
    if (out_lse && !al4(out_lse)) return fail(CSL_EINVAL, "%s: out_lse misaligned", fn);
    if (need > 0 && (!ws || ws_bytes < need || !al16(ws)))
        return fail(CSL_EWORKSPACE, "%s: needs %zu bytes of 16-byte aligned workspace", fn, need);
    rc = check_device();
    if (rc) return rc;
    csl::AttendArgs a{};
    a.q = (const uint8_t*)q; a.q_fmt = q_fmt;
    a.kvc = (const uint8_t*)kv_c; a.kv_fmt = kv_fmt; a.kvc_bstride = kvc_bstride; a.n_cap = n_cap;
    a.idx = idx; a.k = k; a.m = m;
    a.kvw = (const uint8_t*)kv_w; a.kvw_bstride = kvw_bstride; a.kvw_pos0 = kvw_pos0; a.kvw_rows = kvw_rows > 0 ? kvw_rows : 1;
    a.q_pos = q_pos; a.W = W; a.B = B; a.Tq = Tq; a.H = H; a.d = d; a.r = r; a.scale = scale;
    a.out = (uint8_t*)out; a.out_fmt = out_fmt; a.lse = out_lse;
    a.nhb = nhb; a.nsplit = nsplit; a.rps = rps;
    if (nsplit > 1) {
        const size_t rows = (size_t)B * Tq * nhb * nsplit * 64;
        a.ws_o = (float*)ws;
        a.ws_lse = (float*)((uint8_t*)ws + ((rows * d * 4 + 255) & ~(size_t)255));
    }
    return launched(csl::launch_attend(a, (hipStream_t)stream));
}

int csa_attend(const void* q, int q_fmt, const void* kv_c, int kv_fmt, int64_t kvc_bstride, int64_t n_cap,
               const int32_t* idx, int k,
               const void* kv_w, int64_t kvw_bstride, int64_t kvw_pos0, int64_t kvw_rows,
               const int32_t* q_pos, int W, int B, int Tq, int H, int d, int r, float scale,
               void* out, int out_fmt, float* out_lse, void* ws, size_t ws_bytes, void* stream) {
    if (k < 1) return fail(CSL_EINVAL, "csa_attend: k must be >= 1");
    if (B * (int64_t)Tq > 0 && (!idx || !al4(idx))) return fail(CSL_EINVAL, "csa_attend: null or misaligned idx");
    return attend_impl("csa_attend", q, q_fmt, kv_c, kv_fmt, kvc_bstride, n_cap, idx, k, 1, kv_w, kvw_bstride,
                       kvw_pos0, kvw_rows, q_pos, W, B, Tq, H, d, r, scale, out, out_fmt, out_lse, ws, ws_bytes, stream);
}

int hca_attend(const void* q, int q_fmt, const void* kv_c, int kv_fmt, int64_t kvc_bstride, int64_t n_cap, int m,
               const void* kv_w, int64_t kvw_bstride, int64_t kvw_pos0, int64_t kvw_rows,
               const int32_t* q_pos, int W, int B, int Tq, int H, int d, int r, float scale,
               void* out, int out_fmt, float* out_lse, void* ws, size_t ws_bytes, void* stream) {
    if (m < 1) return fail(CSL_EINVAL, "hca_attend: m must be >= 1");
    return attend_impl("hca_attend", q, q_fmt, kv_c, kv_fmt, kvc_bstride, n_cap, nullptr, 0, m, kv_w, kvw_bstride,
                       kvw_pos0, kvw_rows, q_pos, W, B, Tq, H, d, r, scale, out, out_fmt, out_lse, ws, ws_bytes, stream);
}

}  // extern "C"
