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

// Scratch of index_topk_noalloc (for callers that cannot allocate): a file-scope device
// array, so each GPU the library runs on holds its own copy from the time the code
// object is loaded there until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in): it looks up each device's
// address once with hipGetSymbolAddress and passes that.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)96 << 20;
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

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

// Device address of `scratch` on the current device, looked up on the first call made
// with that device current and kept per device.
std::mutex g_scr_mu;
void* g_scr_ptr[64];

int scratch_ptr(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fail(CSL_EDEVICE, "no usable HIP device is current");
    std::lock_guard<std::mutex> lk(g_scr_mu);
    if (!g_scr_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(CSL_ELAUNCH, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
        g_scr_ptr[dev] = p;
    }
    *out = g_scr_ptr[dev];
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
    return q * ((size_t)4 * row_stride(n_cap) + (size_t)nslices * (csl::IDX_SLOT_W + 1)) * 4 + 256;
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

// Paged compressed entries (csa_attend_paged / hca_attend_paged, index_topk_paged,
// kv_compress_step): entry s of sequence b is row s % epb of physical block
// bt[b * bt_stride + s / epb]; blocks are blk_bytes apart; the pool holds n_blocks.
struct Paged {
    const int32_t* bt = nullptr;
    int64_t bt_stride = 0;
    int epb = 0;
    int64_t blk_bytes = 0, n_blocks = 0;
    int64_t sblk_bytes = 0;     // index_topk_paged: block stride of the MXFP4 scale rows
};

int validate_paged(const char* fn, const Paged& pg, int64_t n_cap, int64_t rb) {
    if (!pg.bt || !al4(pg.bt)) return fail(CSL_EINVAL, "%s: null or misaligned block table", fn);
    if (pg.epb < 1 || pg.n_blocks < 1 || pg.n_blocks > INT32_MAX)
        return fail(CSL_EINVAL, "%s: need entries_per_block >= 1 and 1 <= n_blocks < 2^31", fn);
    if (pg.bt_stride < (n_cap + pg.epb - 1) / pg.epb)
        return fail(CSL_EINVAL, "%s: block-table rows of %lld ids cannot cover %lld entries of %d per block", fn,
                    (long long)pg.bt_stride, (long long)n_cap, pg.epb);
    if (pg.blk_bytes < pg.epb * rb || (pg.blk_bytes & 15))
        return fail(CSL_EINVAL, "%s: block_bytes must be a multiple of 16 holding entries_per_block rows", fn);
    if (n_cap > INT32_MAX) return fail(CSL_EUNSUPPORTED, "%s: paged n_cap must be < 2^31", fn);
    return CSL_OK;
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
    if (W > 0 && !kv_w) return fail(CSL_EINVAL, "%s: W > 0 needs kv_w", fn);
    if (W > 0 && kvw_rows < W)    // a shorter ring would hand two window positions the same row
        return fail(CSL_EINVAL, "%s: kvw_rows = %lld is below the window W = %d", fn, (long long)kvw_rows, W);
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

// Checks shared by kv_compress and kv_compress_step (everything but the raw-row range).
static int compress_common(const char* fn, const void* x, int x_fmt, int x_roles, int64_t x_bstride, const float* z,
                           int z_ch, int64_t z_bstride, const float* bias, int B, int d, int r, int m, int overlap,
                           const void* out, int out_fmt, const uint8_t* out_scales, int64_t out_bstride) {
    if (B < 0) return fail(CSL_EINVAL, "%s: negative size", fn);
    if (B > 65535) return fail(CSL_EUNSUPPORTED, "%s: B > 65535", fn);
    if (m < 1) return fail(CSL_EINVAL, "%s: m must be >= 1", fn);
    if (d < 32 || d > 1024 || d % 32) return fail(CSL_EUNSUPPORTED, "%s: d = %d must be a multiple of 32 in [32, 1024]", fn, d);
    if (x_fmt != CSL_F32 && x_fmt != CSL_BF16) return fail(CSL_EINVAL, "%s: x_fmt must be F32 or BF16", fn);
    if (x_roles != 1 && x_roles != 2) return fail(CSL_EINVAL, "%s: x_roles must be 1 or 2", fn);
    if (x_roles == 2 && !overlap) return fail(CSL_EINVAL, "%s: two-role rows need overlapping windows", fn);
    if (out_fmt < CSL_F32 || out_fmt > CSL_MXFP4) return fail(CSL_EINVAL, "%s: unknown out_fmt %d", fn, out_fmt);
    if (out_fmt == CSL_KV_PACKED && (r < 0 || r > d || r % 8 || (d + r) % 16))
        return fail(CSL_EINVAL, "%s: packed output needs r %% 8 == 0, (d + r) %% 16 == 0, 0 <= r <= d", fn);
    if (z_ch != 1 && z_ch != d) return fail(CSL_EINVAL, "%s: z_ch must be 1 or d", fn);
    if (B == 0) return CSL_OK;
    if (!x || !z || !bias || !out) return fail(CSL_EINVAL, "%s: null x, z, bias or out", fn);
    if ((out_fmt == CSL_MXFP4) != (out_scales != nullptr)) return fail(CSL_EINVAL, "%s: out_scales must be given exactly for MXFP4", fn);
    if (!al16(x) || (x_bstride & 15) || !al16(out) || (out_bstride & 15))
        return fail(CSL_EINVAL, "%s: x/out and their strides must be 16-byte aligned", fn);
    if (z_ch == d ? (!al16(z) || (z_bstride & 15) || !al16(bias)) : (!al4(z) || (z_bstride & 3) || !al4(bias)))
        return fail(CSL_EINVAL, "%s: z/bias misaligned", fn);
    return CSL_OK;
}

int kv_compress(const void* x, int x_fmt, int x_roles, int64_t x_bstride, int64_t x_pos0, int64_t n_tok,
                const float* z, int z_ch, int64_t z_bstride, const float* bias,
                int B, int d, int r, int m, int overlap, int64_t e_begin, int64_t n_e,
                void* out, int out_fmt, uint8_t* out_scales, int64_t out_bstride, int64_t sc_bstride,
                void* stream) {
    const char* fn = "kv_compress";
    if (n_e < 0 || n_tok < 0 || e_begin < 0) return fail(CSL_EINVAL, "%s: negative size", fn);
    if ((int64_t)n_e * m > ((int64_t)1 << 40)) return fail(CSL_EINVAL, "%s: entry range too large", fn);
    if (B == 0 || n_e == 0) {
        int rc = compress_common(fn, x, x_fmt, x_roles, x_bstride, z, z_ch, z_bstride, bias, 0, d, r, m, overlap, out,
                                 out_fmt, out_scales, out_bstride);
        if (rc) return rc;
        g_err.clear();
        return CSL_OK;
    }
    int rc = compress_common(fn, x, x_fmt, x_roles, x_bstride, z, z_ch, z_bstride, bias, B, d, r, m, overlap, out,
                             out_fmt, out_scales, out_bstride);
    if (rc) return rc;
    const int win = overlap ? 2 * m : m;
    int64_t lo = (e_begin + 1) * m - win;
    if (lo < 0) lo = 0;
    const int64_t hi = (e_begin + n_e) * m - 1;
    if (lo < x_pos0 || hi >= x_pos0 + n_tok)
        return fail(CSL_EINVAL, "%s: raw positions %lld..%lld are not all in the buffer [%lld, %lld)", fn,
                    (long long)lo, (long long)hi, (long long)x_pos0, (long long)(x_pos0 + n_tok));
    rc = check_device();
    if (rc) return rc;
    csl::CompressArgs a{};
    a.x = (const uint8_t*)x; a.x_fmt = x_fmt; a.x_bstride = x_bstride; a.x_pos0 = x_pos0; a.n_tok = n_tok;
    a.x_rows = 0; a.x_roles = x_roles;
    a.z = z; a.z_ch = z_ch; a.z_bstride = z_bstride; a.bias = bias;
    a.B = B; a.d = d; a.r = r; a.m = m; a.overlap = overlap ? 1 : 0; a.e_begin = e_begin; a.n_e = n_e;
    a.out = (uint8_t*)out; a.out_fmt = out_fmt; a.out_scales = out_scales; a.out_bstride = out_bstride;
    a.sc_bstride = sc_bstride;
    return launched(csl::launch_compress(a, (hipStream_t)stream));
}

}  // extern "C"

// Validation and argument block of one decode-time compression job.
static int step_job(const char* fn, const csl_compress_job& j, const int32_t* pos, int B, int T, csl::CompressArgs& a) {
    if (T < 0) return fail(CSL_EINVAL, "%s: negative T", fn);
    if (T > 65535) return fail(CSL_EUNSUPPORTED, "%s: T > 65535", fn);
    int rc = compress_common(fn, j.x_ring, j.x_fmt, j.x_roles, j.x_bstride, j.z_ring, j.z_ch, j.z_bstride, j.bias, B,
                             j.d, j.r, j.m, j.overlap, j.out, j.out_fmt, j.out_scales, j.block_table ? 0 : j.out_bstride);
    if (rc) return rc;
    const int win = j.overlap ? 2 * j.m : j.m;
    if (j.x_rows < win + T - 1)
        return fail(CSL_EINVAL, "%s: a ring of %lld rows cannot hold the %d-row window of T = %d new tokens", fn,
                    (long long)j.x_rows, win, T);
    Paged pg;
    if (j.block_table) {
        pg.bt = j.block_table; pg.bt_stride = j.bt_stride; pg.epb = j.entries_per_block; pg.blk_bytes = j.block_bytes;
        pg.sblk_bytes = j.scale_block_bytes; pg.n_blocks = j.n_blocks;
        if ((rc = validate_paged(fn, pg, (int64_t)j.bt_stride * (j.entries_per_block > 0 ? j.entries_per_block : 1),
                                 row_bytes(j.out_fmt, j.d, j.r))))
            return rc;
        if (j.out_fmt == CSL_MXFP4 && j.scale_block_bytes < (int64_t)j.entries_per_block * (j.d / 32))
            return fail(CSL_EINVAL, "%s: scale_block_bytes cannot hold entries_per_block scale rows", fn);
    } else if (j.n_cap < 0) {
        return fail(CSL_EINVAL, "%s: negative n_cap", fn);
    }
    if (B * (int64_t)T > 0 && (!pos || !al4(pos))) return fail(CSL_EINVAL, "%s: null or misaligned pos", fn);
    a = csl::CompressArgs{};
    a.x = (const uint8_t*)j.x_ring; a.x_fmt = j.x_fmt; a.x_bstride = j.x_bstride; a.x_pos0 = 0; a.n_tok = j.x_rows;
    a.x_rows = j.x_rows; a.x_roles = j.x_roles;
    a.z = j.z_ring; a.z_ch = j.z_ch; a.z_bstride = j.z_bstride; a.bias = j.bias;
    a.B = B; a.d = j.d; a.r = j.r; a.m = j.m; a.overlap = j.overlap ? 1 : 0; a.e_begin = 0; a.n_e = T;
    a.out = (uint8_t*)j.out; a.out_fmt = j.out_fmt; a.out_scales = j.out_scales; a.out_bstride = j.out_bstride;
    a.sc_bstride = j.sc_bstride;
    a.pos = pos; a.n_cap = j.n_cap;
    if (j.block_table) { a.bt = pg.bt; a.bt_stride = pg.bt_stride; a.epb = pg.epb; a.blk_bytes = pg.blk_bytes;
                         a.sblk_bytes = pg.sblk_bytes; a.n_blocks = pg.n_blocks; }
    return CSL_OK;
}

extern "C" {

int kv_compress_step(const void* x_ring, int x_fmt, int x_roles, int64_t x_bstride, int64_t x_rows,
                     const float* z_ring, int z_ch, int64_t z_bstride, const float* bias,
                     const int32_t* pos, int B, int T, int d, int r, int m, int overlap,
                     void* out, int out_fmt, uint8_t* out_scales, int64_t out_bstride, int64_t sc_bstride,
                     int64_t n_cap, const int32_t* block_table, int64_t bt_stride, int entries_per_block,
                     int64_t block_bytes, int64_t scale_block_bytes, int64_t n_blocks, void* stream) {
    const csl_compress_job j{x_ring, x_fmt, x_roles, x_bstride, x_rows, z_ring, z_ch, z_bstride, bias, d, r, m, overlap,
                             out, out_fmt, out_scales, out_bstride, sc_bstride, n_cap, block_table, bt_stride,
                             entries_per_block, block_bytes, scale_block_bytes, n_blocks};
    csl::CompressArgs a;
    int rc = step_job("kv_compress_step", j, pos, B, T, a);
    if (rc) return rc;
    if (B * (int64_t)T == 0) { g_err.clear(); return CSL_OK; }
    rc = check_device();
    if (rc) return rc;
    return launched(csl::launch_compress(a, (hipStream_t)stream));
}

int kv_compress_step_pair(const csl_compress_job* first, const csl_compress_job* second, const int32_t* pos, int B,
                          int T, void* stream) {
    const char* fn = "kv_compress_step_pair";
    if (!first || !second) return fail(CSL_EINVAL, "%s: null job", fn);
    csl::CompressArgs a0, a1;
    int rc = step_job(fn, *first, pos, B, T, a0);
    if (rc) return rc;
    rc = step_job(fn, *second, pos, B, T, a1);
    if (rc) return rc;
    if (B * (int64_t)T == 0) { g_err.clear(); return CSL_OK; }
    rc = check_device();
    if (rc) return rc;
    return launched(csl::launch_compress_pair(a0, a1, (hipStream_t)stream));
}

// Many queries per call (prefill): the dense path scores every (query, key) pair into
// the workspace, a pass of at most DENSE_WS_MAX bytes at a time.
constexpr int DENSE_MIN_TQ = 64;
constexpr size_t DENSE_WS_MAX = (size_t)2 << 30;

bool dense_path(int fmt, int d_I, int H_I, int Tq) {
    return (fmt == CSL_BF16 || fmt == CSL_MXFP4) && d_I == 128 && (H_I == 16 || H_I == 32 || H_I == 64 || H_I == 128) &&
           Tq >= DENSE_MIN_TQ;
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

}  // extern "C"

// index_topk with a caller workspace (use_scratch false) or with the library's static
// scratch (use_scratch true, index_topk_noalloc).
static int index_impl(const char* fn, const void* qi, int qi_fmt, const uint8_t* qi_scales, const float* w,
                      const void* ki, int ki_fmt, const uint8_t* ki_scales, int64_t ki_bstride, int64_t ks_bstride,
                      const Paged* pg,
                      const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int m, int64_t n_cap, int k,
                      int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes, bool use_scratch, void* stream,
                      const csl::CompressArgs* kvj = nullptr, const csl::CompressArgs* keyj = nullptr) {
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
    if (pg) {
        if (int rc = validate_paged(fn, *pg, n_cap, row_bytes(ki_fmt, d_I, 0))) return rc;
        if (pg->epb % 16) return fail(CSL_EUNSUPPORTED, "%s: entries_per_block must be a multiple of 16", fn);
        if (ki_fmt == CSL_MXFP4 && pg->sblk_bytes < (int64_t)pg->epb * (d_I / 32))
            return fail(CSL_EINVAL, "%s: scale_block_bytes cannot hold entries_per_block scale rows", fn);
    }
    if (use_scratch) {
        if (need > NOALLOC_SCRATCH_BYTES)
            return fail(CSL_EWORKSPACE, "%s: this call needs %zu bytes of scratch, more than the %zu bytes the library "
                        "holds (use index_topk with a workspace)", fn, need, NOALLOC_SCRATCH_BYTES);
    } else if (need > 0 && (!ws || ws_bytes < need || !al16(ws))) {
        return fail(CSL_EWORKSPACE, "%s: needs %zu bytes of 16-byte aligned workspace", fn, need);
    }
    int rc = check_device();
    if (rc) return rc;
    if (use_scratch && need > 0) {
        rc = scratch_ptr(&ws);
        if (rc) return rc;
        ws_bytes = NOALLOC_SCRATCH_BYTES;
    }
    csl::IndexArgs a{};
    a.qi = (const uint8_t*)qi; a.qi_fmt = qi_fmt; a.qi_scales = qi_scales; a.w = w;
    a.ki = (const uint8_t*)ki; a.ki_fmt = ki_fmt; a.ki_scales = ki_scales; a.ki_bstride = ki_bstride; a.ks_bstride = ks_bstride;
    if (pg) { a.bt = pg->bt; a.bt_stride = pg->bt_stride; a.epb = pg->epb; a.blk_bytes = pg->blk_bytes;
              a.sblk_bytes = pg->sblk_bytes; a.n_blocks = pg->n_blocks; }
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
        a.sstride = row_stride(n_cap);
        const size_t q = (size_t)B * Tq;
        const size_t nr = q * a.sstride * 4;           // bytes of one [B*Tq][sstride] array
        a.cand_key = (uint32_t*)ws;
        a.cand_idx = (int32_t*)((uint8_t*)ws + nr);
        a.scores = (uint32_t*)((uint8_t*)ws + 2 * nr);
        a.fb_idx = (int32_t*)((uint8_t*)ws + 3 * nr);
        a.hist = (uint32_t*)((uint8_t*)ws + 4 * nr);
        a.seg_cnt = (int32_t*)(a.hist + q * nslices * csl::IDX_SLOT_W);
    }
    const hipStream_t s = (hipStream_t)stream;
    if (kvj) {
        // csa_index_step: the compression runs inside the scoring kernel when the key job
        // writes exactly the keys this call reads and the shapes are the fused ones;
        // otherwise the compression launch, then the index launch
        const csl::CompressArgs& kj = *keyj;
        const bool mx = ki_fmt == CSL_MXFP4;
        const bool same_keys = kj.out == (const uint8_t*)ki && kj.out_fmt == ki_fmt && kj.d == d_I && kj.m == m &&
            (mx ? kj.out_scales == ki_scales : true) &&
            (pg ? (kj.bt == pg->bt && kj.bt_stride == pg->bt_stride && kj.epb == pg->epb &&
                   kj.blk_bytes == pg->blk_bytes && kj.n_blocks == pg->n_blocks && (!mx || kj.sblk_bytes == pg->sblk_bytes))
                : (!kj.bt && kj.out_bstride == ki_bstride && (!mx || kj.sc_bstride == ks_bstride)));
        csl::IndexPre pre{*kvj, kj, 0, 0};
        if (Tq == 1 && !dense && nslices > 1 && d_I == 128 && (mx || ki_fmt == CSL_BF16) && same_keys &&
            csl::compress_pair_in_index(*kvj, kj, pre.gz_kv, pre.gz_key))
            return launched(csl::launch_index_topk(a, s, &pre));
        const hipError_t e = csl::launch_compress_pair(*kvj, kj, s);
        if (e != hipSuccess) return launched(e);
    }
    return launched(csl::launch_index_topk(a, s));
}

extern "C" {

int csa_index_step(const csl_compress_job* kv_job, const csl_compress_job* key_job,
                   const void* qi, int qi_fmt, const uint8_t* qi_scales, const float* w,
                   const void* ki, int ki_fmt, const uint8_t* ki_scales, int64_t ki_bstride, int64_t ks_bstride,
                   const int32_t* block_table, int64_t bt_stride, int entries_per_block, int64_t block_bytes,
                   int64_t scale_block_bytes, int64_t n_blocks,
                   const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int m, int64_t n_cap, int k,
                   int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "csa_index_step";
    if (!kv_job || !key_job) return fail(CSL_EINVAL, "%s: null job", fn);
    csl::CompressArgs a0, a1;
    int rc = step_job(fn, *kv_job, q_pos, B, Tq, a0);
    if (rc) return rc;
    rc = step_job(fn, *key_job, q_pos, B, Tq, a1);
    if (rc) return rc;
    Paged pg;
    if (block_table) {
        pg.bt = block_table; pg.bt_stride = bt_stride; pg.epb = entries_per_block; pg.blk_bytes = block_bytes;
        pg.sblk_bytes = scale_block_bytes; pg.n_blocks = n_blocks;
    }
    return index_impl(fn, qi, qi_fmt, qi_scales, w, ki, ki_fmt, ki_scales, block_table ? 0 : ki_bstride,
                      block_table ? 0 : ks_bstride, block_table ? &pg : nullptr, q_pos, B, Tq, H_I, d_I, m, n_cap, k,
                      out_idx, out_score, ws, ws_bytes, false, stream, &a0, &a1);
}

int index_topk(const void* qi, int qi_fmt, const uint8_t* qi_scales, const float* w,
               const void* ki, int ki_fmt, const uint8_t* ki_scales, int64_t ki_bstride, int64_t ks_bstride,
               const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int m, int64_t n_cap, int k,
               int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes, void* stream) {
    return index_impl("index_topk", qi, qi_fmt, qi_scales, w, ki, ki_fmt, ki_scales, ki_bstride, ks_bstride, nullptr,
                      q_pos, B, Tq, H_I, d_I, m, n_cap, k, out_idx, out_score, ws, ws_bytes, false, stream);
}

int index_topk_paged(const void* qi, int qi_fmt, const uint8_t* qi_scales, const float* w,
                     const void* ki_pool, int ki_fmt, const uint8_t* ki_scale_pool,
                     const int32_t* block_table, int64_t bt_stride, int entries_per_block,
                     int64_t block_bytes, int64_t scale_block_bytes, int64_t n_blocks,
                     const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int m, int64_t n_cap, int k,
                     int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes, void* stream) {
    Paged pg;
    pg.bt = block_table; pg.bt_stride = bt_stride; pg.epb = entries_per_block; pg.blk_bytes = block_bytes;
    pg.sblk_bytes = scale_block_bytes; pg.n_blocks = n_blocks;
    return index_impl("index_topk_paged", qi, qi_fmt, qi_scales, w, ki_pool, ki_fmt, ki_scale_pool, 0, 0, &pg, q_pos,
                      B, Tq, H_I, d_I, m, n_cap, k, out_idx, out_score, ws, ws_bytes, false, stream);
}

int index_topk_noalloc(const void* qi, int qi_fmt, const uint8_t* qi_scales, const float* w,
                       const void* ki, int ki_fmt, const uint8_t* ki_scales, int64_t ki_bstride, int64_t ks_bstride,
                       const int32_t* q_pos, int B, int Tq, int H_I, int d_I, int m, int64_t n_cap, int k,
                       int32_t* out_idx, float* out_score, void* stream) {
    return index_impl("index_topk_noalloc", qi, qi_fmt, qi_scales, w, ki, ki_fmt, ki_scales, ki_bstride, ks_bstride,
                      nullptr, q_pos, B, Tq, H_I, d_I, m, n_cap, k, out_idx, out_score, nullptr, 0, true, stream);
}

size_t csl_noalloc_scratch_bytes(void) { return NOALLOC_SCRATCH_BYTES; }

size_t csl_attend_workspace(int B, int Tq, int H, int d, int64_t rows_max) {
    if (B < 0 || Tq < 0 || H < 1) return 0;
    int nhb, nsplit, rps;
    plan_attend(B, Tq, H, rows_max, true, nhb, nsplit, rps);   // the CSA cap only adds splits
    return attend_ws(B, Tq, d, nhb, nsplit);
}

}  // extern "C"

static int attend_impl(const char* fn, const void* q, int q_fmt, const void* kv_c, int kv_fmt, int64_t kvc_bstride,
                       const Paged* pg, int64_t n_cap, const int32_t* idx, int k, int m, const void* kv_w,
                       int64_t kvw_bstride, int64_t kvw_pos0, int64_t kvw_rows, const float* sink,
                       const int32_t* q_pos, int W, int B, int Tq, int H, int d, int r, float scale, void* out,
                       int out_fmt, float* out_lse, void* ws, size_t ws_bytes, void* stream,
                       const csl::CompressArgs* kvj = nullptr) {
    int rc = validate_attend(fn, q, q_fmt, kv_c, kv_fmt, pg ? 0 : kvc_bstride, n_cap, kv_w, kvw_bstride, kvw_rows,
                             q_pos, W, B, Tq, H, d, r, out, out_fmt);
    if (rc) return rc;
    if (pg && (rc = validate_paged(fn, *pg, n_cap, row_bytes(kv_fmt, d, r)))) return rc;
    const int64_t rows_max = (idx ? (int64_t)k : n_cap) + W;
    int nhb, nsplit, rps;
    plan_attend(B, Tq, H, rows_max, true, nhb, nsplit, rps);
    const size_t need = attend_ws(B, Tq, d, nhb, nsplit);
    if (B * (int64_t)Tq == 0) { g_err.clear(); return CSL_OK; }
    if (out_lse && !al4(out_lse)) return fail(CSL_EINVAL, "%s: out_lse misaligned", fn);
    if (sink && !al4(sink)) return fail(CSL_EINVAL, "%s: sink misaligned", fn);
    if (need > 0 && (!ws || ws_bytes < need || !al16(ws)))
        return fail(CSL_EWORKSPACE, "%s: needs %zu bytes of 16-byte aligned workspace", fn, need);
    rc = check_device();
    if (rc) return rc;
    csl::AttendArgs a{};
    a.q = (const uint8_t*)q; a.q_fmt = q_fmt;
    a.kvc = (const uint8_t*)kv_c; a.kv_fmt = kv_fmt; a.kvc_bstride = kvc_bstride; a.n_cap = n_cap;
    if (pg) { a.bt = pg->bt; a.bt_stride = pg->bt_stride; a.epb = pg->epb; a.blk_bytes = pg->blk_bytes; a.n_blocks = pg->n_blocks; }
    a.idx = idx; a.k = k; a.m = m;
    a.kvw = (const uint8_t*)kv_w; a.kvw_bstride = kvw_bstride; a.kvw_pos0 = kvw_pos0; a.kvw_rows = kvw_rows > 0 ? kvw_rows : 1;
    a.sink = sink;
    a.q_pos = q_pos; a.W = W; a.B = B; a.Tq = Tq; a.H = H; a.d = d; a.r = r; a.scale = scale;
    a.out = (uint8_t*)out; a.out_fmt = out_fmt; a.lse = out_lse;
    a.nhb = nhb; a.nsplit = nsplit; a.rps = rps;
    if (nsplit > 1) {
        const size_t rows = (size_t)B * Tq * nhb * nsplit * 64;
        a.ws_o = (float*)ws;
        a.ws_lse = (float*)((uint8_t*)ws + ((rows * d * 4 + 255) & ~(size_t)255));
    }
    const hipStream_t s = (hipStream_t)stream;
    if (kvj) {
        // hca_attend_step: the compression runs inside the attention kernel when the job
        // writes exactly the entries this call reads and the shapes are the fused ones;
        // otherwise the compression launch, then the attention
        const csl::CompressArgs& j = *kvj;
        const bool same = j.out == (const uint8_t*)kv_c && j.out_fmt == kv_fmt && j.d == d && j.r == r && j.m == m &&
            (pg ? (j.bt == pg->bt && j.bt_stride == pg->bt_stride && j.epb == pg->epb && j.blk_bytes == pg->blk_bytes &&
                   j.n_blocks == pg->n_blocks)
                : (!j.bt && j.out_bstride == kvc_bstride));
        // The split that attends the newest entry compresses it before its tiles; that pays
        // only when the split has rows to spare: at a full context (the newest entry is row
        // n_cap - 1) its split must hold at most half the rows of the others.
        const int64_t se = n_cap > 0 ? (n_cap - 1) / rps : 0;
        const int64_t l_all = n_cap + W;
        const int64_t rows_e = (l_all < (se + 1) * rps ? l_all : (se + 1) * rps) - se * rps;
        const bool slack = nsplit > 1 && 2 * rows_e <= rps;
        csl::AttendPre pre{j, 0};
        if (same && slack && csl::attend_takes_pre(a) && csl::compress_in_attend(j, pre.gz))
            return launched(csl::launch_attend(a, s, &pre));
        const hipError_t e = csl::launch_compress(j, s);
        if (e != hipSuccess) return launched(e);
    }
    return launched(csl::launch_attend(a, s));
}

static int csa_check(const char* fn, const int32_t* idx, int k, int B, int Tq) {
    if (k < 1) return fail(CSL_EINVAL, "%s: k must be >= 1", fn);
    if (B * (int64_t)Tq > 0 && (!idx || !al4(idx))) return fail(CSL_EINVAL, "%s: null or misaligned idx", fn);
    return CSL_OK;
}

extern "C" {

int csa_attend(const void* q, int q_fmt, const void* kv_c, int kv_fmt, int64_t kvc_bstride, int64_t n_cap,
               const int32_t* idx, int k,
               const void* kv_w, int64_t kvw_bstride, int64_t kvw_pos0, int64_t kvw_rows, const float* sink,
               const int32_t* q_pos, int W, int B, int Tq, int H, int d, int r, float scale,
               void* out, int out_fmt, float* out_lse, void* ws, size_t ws_bytes, void* stream) {
    if (int rc = csa_check("csa_attend", idx, k, B, Tq)) return rc;
    return attend_impl("csa_attend", q, q_fmt, kv_c, kv_fmt, kvc_bstride, nullptr, n_cap, idx, k, 1, kv_w,
                       kvw_bstride, kvw_pos0, kvw_rows, sink, q_pos, W, B, Tq, H, d, r, scale, out, out_fmt, out_lse,
                       ws, ws_bytes, stream);
}

int hca_attend(const void* q, int q_fmt, const void* kv_c, int kv_fmt, int64_t kvc_bstride, int64_t n_cap, int m,
               const void* kv_w, int64_t kvw_bstride, int64_t kvw_pos0, int64_t kvw_rows, const float* sink,
               const int32_t* q_pos, int W, int B, int Tq, int H, int d, int r, float scale,
               void* out, int out_fmt, float* out_lse, void* ws, size_t ws_bytes, void* stream) {
    if (m < 1) return fail(CSL_EINVAL, "hca_attend: m must be >= 1");
    return attend_impl("hca_attend", q, q_fmt, kv_c, kv_fmt, kvc_bstride, nullptr, n_cap, nullptr, 0, m, kv_w,
                       kvw_bstride, kvw_pos0, kvw_rows, sink, q_pos, W, B, Tq, H, d, r, scale, out, out_fmt, out_lse,
                       ws, ws_bytes, stream);
}

int csa_attend_paged(const void* q, int q_fmt, const void* kv_pool, int kv_fmt, const int32_t* block_table,
                     int64_t bt_stride, int entries_per_block, int64_t block_bytes, int64_t n_blocks, int64_t n_cap,
                     const int32_t* idx, int k,
                     const void* kv_w, int64_t kvw_bstride, int64_t kvw_pos0, int64_t kvw_rows, const float* sink,
                     const int32_t* q_pos, int W, int B, int Tq, int H, int d, int r, float scale,
                     void* out, int out_fmt, float* out_lse, void* ws, size_t ws_bytes, void* stream) {
    if (int rc = csa_check("csa_attend_paged", idx, k, B, Tq)) return rc;
    Paged pg;
    pg.bt = block_table; pg.bt_stride = bt_stride; pg.epb = entries_per_block; pg.blk_bytes = block_bytes;
    pg.n_blocks = n_blocks;
    return attend_impl("csa_attend_paged", q, q_fmt, kv_pool, kv_fmt, 0, &pg, n_cap, idx, k, 1, kv_w, kvw_bstride,
                       kvw_pos0, kvw_rows, sink, q_pos, W, B, Tq, H, d, r, scale, out, out_fmt, out_lse, ws, ws_bytes,
                       stream);
}

int hca_attend_step(const csl_compress_job* kv_job, const void* q, int q_fmt, const void* kv_c, int kv_fmt,
                    int64_t kvc_bstride, const int32_t* block_table, int64_t bt_stride, int entries_per_block,
                    int64_t block_bytes, int64_t n_blocks, int64_t n_cap, int m,
                    const void* kv_w, int64_t kvw_bstride, int64_t kvw_pos0, int64_t kvw_rows, const float* sink,
                    const int32_t* q_pos, int W, int B, int Tq, int H, int d, int r, float scale,
                    void* out, int out_fmt, float* out_lse, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "hca_attend_step";
    if (!kv_job) return fail(CSL_EINVAL, "%s: null job", fn);
    if (m < 1) return fail(CSL_EINVAL, "%s: m must be >= 1", fn);
    csl::CompressArgs a0;
    int rc = step_job(fn, *kv_job, q_pos, B, Tq, a0);
    if (rc) return rc;
    Paged pg;
    if (block_table) {
        pg.bt = block_table; pg.bt_stride = bt_stride; pg.epb = entries_per_block; pg.blk_bytes = block_bytes;
        pg.n_blocks = n_blocks;
    }
    return attend_impl(fn, q, q_fmt, kv_c, kv_fmt, block_table ? 0 : kvc_bstride, block_table ? &pg : nullptr, n_cap,
                       nullptr, 0, m, kv_w, kvw_bstride, kvw_pos0, kvw_rows, sink, q_pos, W, B, Tq, H, d, r, scale, out,
                       out_fmt, out_lse, ws, ws_bytes, stream, &a0);
}

int hca_attend_paged(const void* q, int q_fmt, const void* kv_pool, int kv_fmt, const int32_t* block_table,
                     int64_t bt_stride, int entries_per_block, int64_t block_bytes, int64_t n_blocks, int64_t n_cap,
                     int m, const void* kv_w, int64_t kvw_bstride, int64_t kvw_pos0, int64_t kvw_rows,
                     const float* sink, const int32_t* q_pos, int W, int B, int Tq, int H, int d, int r, float scale,
                     void* out, int out_fmt, float* out_lse, void* ws, size_t ws_bytes, void* stream) {
    if (m < 1) return fail(CSL_EINVAL, "hca_attend_paged: m must be >= 1");
    Paged pg;
    pg.bt = block_table; pg.bt_stride = bt_stride; pg.epb = entries_per_block; pg.blk_bytes = block_bytes;
    pg.n_blocks = n_blocks;
    return attend_impl("hca_attend_paged", q, q_fmt, kv_pool, kv_fmt, 0, &pg, n_cap, nullptr, 0, m, kv_w,
                       kvw_bstride, kvw_pos0, kvw_rows, sink, q_pos, W, B, Tq, H, d, r, scale, out, out_fmt, out_lse,
                       ws, ws_bytes, stream);
}

int grouped_out_proj(const void* x, int x_fmt, const void* w, int w_fmt, int M, int G, int K, int R,
                     void* out, int out_fmt, void* stream) {
    const char* fn = "grouped_out_proj";
    if (M < 0 || G < 1 || K < 1 || R < 1) return fail(CSL_EINVAL, "%s: need M >= 0 and G, K, R >= 1", fn);
    if (x_fmt != CSL_BF16 || w_fmt != CSL_BF16) return fail(CSL_EUNSUPPORTED, "%s: x and w must be CSL_BF16", fn);
    if (out_fmt != CSL_F32 && out_fmt != CSL_BF16) return fail(CSL_EINVAL, "%s: out_fmt must be F32 or BF16", fn);
    if (K % 128 || R % 128) return fail(CSL_EUNSUPPORTED, "%s: K and R must be multiples of 128", fn);
    if ((int64_t)G * K > INT32_MAX || (int64_t)G * R > INT32_MAX || M > 65535 * 128)
        return fail(CSL_EUNSUPPORTED, "%s: sizes too large", fn);
    if (M == 0) { g_err.clear(); return CSL_OK; }
    if (!x || !w || !out) return fail(CSL_EINVAL, "%s: null x, w or out", fn);
    if (!al16(x) || !al16(w) || !al16(out)) return fail(CSL_EINVAL, "%s: x, w and out must be 16-byte aligned", fn);
    int rc = check_device();
    if (rc) return rc;
    csl::GprojArgs a{(const uint8_t*)x, (const uint8_t*)w, M, G, K, R, (uint8_t*)out, out_fmt};
    return launched(csl::launch_grouped_out_proj(a, (hipStream_t)stream));
}

}  // extern "C"
