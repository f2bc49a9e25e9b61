// device.h -- gfx950 device helpers shared by the CSA/HCA kernels: storage-format
// codecs (bf16, OCP fp8 e4m3fn, e2m1 + e8m0 block scales), MFMA wrappers, wave
// reductions.  Internal header of the HIP library; not part of the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csl {

enum Fmt { F32 = 0, BF16 = 1, KV_PACKED = 2, MXFP4 = 3 };

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define CSL_LOG2E 1.4426950408889634f
#define CSL_LN2 0.6931471805599453f

// ---------------------------------------------------------------------------
// Storage codecs.  Stored KV rows: the RoPE dims as bf16, then the remaining
// dims as fp8 e4m3fn (mixed-precision KV cache).  Indexer operands may be MXFP4:
// e2m1 nibbles (even element in the low nibble) with one e8m0 scale per 32.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// fp32 -> OCP e4m3fn, round to nearest even, saturating to +-448.
__device__ __forceinline__ uint32_t f32_to_e4m3_rne_sat(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const float a = fabsf(x);
    if (a != a) return 0x7fu;
    if (a < 0x1p-6f) {                       // subnormal range: quantum 2^-9
        return sign | (uint32_t)rintf(a * 512.0f);  // 8 -> 0x08, the smallest normal
    }
    if (a >= 448.0f) return sign | 0x7eu;
    const uint32_t au = __float_as_uint(a);
    const int e = (int)(au >> 23) - 127;     // -6 .. 8
    const uint32_t m = au & 0x7fffffu;
    const uint32_t mr = (m + 0x7ffffu + ((m >> 20) & 1u)) >> 20;  // 0..8, carry ok
    uint32_t code = ((uint32_t)(e + 7) << 3) + mr;
    if (code > 0x7eu) code = 0x7eu;
    return sign | code;
}

// Value already divided by its block scale -> e2m1 code, nearest-even, saturating.
__device__ __forceinline__ uint32_t f32_to_e2m1_rne_sat(float x) {
    const float a = fabsf(x);
    uint32_t c;
    if (a <= 0.25f) c = 0;
    else if (a < 0.75f) c = 1;
    else if (a <= 1.25f) c = 2;
    else if (a < 1.75f) c = 3;
    else if (a <= 2.5f) c = 4;
    else if (a < 3.5f) c = 5;
    else if (a <= 5.0f) c = 6;
    else c = 7;
    return c | ((__float_as_uint(x) >> 28) & 8u);
}

// Shared exponent of an MXFP4 block: the smallest e with 6 * 2^e >= amax.
__device__ __forceinline__ int mx_block_exponent(float amax) {
    if (!(amax > 0.0f)) return -127;
    int E;
    const float f = frexpf(amax, &E);        // amax = f * 2^E, f in [0.5, 1)
    int e = (f <= 0.75f) ? E - 3 : E - 2;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Two fp32 -> two bf16 in one dword (element 0 in the low half), round to nearest
// even, by the gfx950 packed conversion.
// Two fp32 values -> two fp16 (round to nearest even), low half first.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    const _Float16 ha = (_Float16)a, hb = (_Float16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}
__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{a, b}, v2bf));
}

// 4 fp8 e4m3fn (one dword) -> 4 bf16 (two dwords).  The gfx950 conversion is the
// OCP e4m3fn decode; every e4m3 value is exact in bf16, so truncation is exact.
__device__ __forceinline__ void e4m3x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
    const v2f a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const v2f b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    lo = __builtin_amdgcn_perm(__float_as_uint(a[1]), __float_as_uint(a[0]), 0x07060302u);
    hi = __builtin_amdgcn_perm(__float_as_uint(b[1]), __float_as_uint(b[0]), 0x07060302u);
}

// Order-preserving map float -> uint32 (larger float -> larger key).  -0 is
// folded onto +0 first so that equal scores compare equal.
__device__ __forceinline__ uint32_t score_key(float s) {
    const uint32_t u = __float_as_uint(s + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// ---------------------------------------------------------------------------
// MFMA wrappers (layouts checked on gfx950):
//  16x16x32 bf16 : A lane l = row l%16, k 8*(l/16)..+8; B lane l = col l%16, same k
//  16x16x4  f32  : A lane l = row l%16, k = l/16;       B lane l = col l%16, k = l/16
//  16x16x128 fp4 (scaled): A lane l = row l%16, k 32*(l/16)..+32 (16 bytes in dwords
//                0..3, low nibble first), e8m0 scale (byte 0) for that 32-block.
//  C (all three): lane l holds C[4*(l/16)+i][l%16], i = 0..3.
// ---------------------------------------------------------------------------
__device__ __forceinline__ v4f mfma_bf16(const u32x4& a, const u32x4& b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ v4f mfma_f32(float a, float b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma_fp4(const u32x4& a, const u32x4& b, int sa, int sb, v4f c) {
    // FP4 operands use only the low four registers of the eight-register operand
    typedef int v4i __attribute__((ext_vector_type(4)));
    const v4i a4 = __builtin_bit_cast(v4i, a), b4 = __builtin_bit_cast(v4i, b);
    const v8i A = __builtin_shufflevector(a4, a4, 0, 1, 2, 3, -1, -1, -1, -1);
    const v8i B = __builtin_shufflevector(b4, b4, 0, 1, 2, 3, -1, -1, -1, -1);
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 4, 0, sa, 0, sb);
}

// LDS transpose read (gfx950): within each 16-lane group, lane i receives element
// (i % 4) of the 64-bit chunks read by source lanes 4*j + i/4, j = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
    v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p));
    return __builtin_bit_cast(u32x2, v);
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m) { return __shfl_xor(v, m, 64); }

// Reductions over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48) with
// the gfx950 row-swap moves; every lane ends with identical bits.
__device__ __forceinline__ float cross4_max(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float cross4_sum(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Load through a pointer known to address global memory.  A pointer that went
// through LDS (or any generic pointer the compiler cannot trace to a kernel
// argument) would otherwise become a flat load, which also counts against the LDS
// wait counter: every later LDS wait would then wait for the global load too.
template <typename T>
__device__ __forceinline__ T ld_global(const void* p) {
    return *(const __attribute__((address_space(1))) T*)p;
}

// Load of a block-uniform value that no kernel of the launch writes, through the scalar
// data cache (a scalar load, counted by lgkmcnt): waiting for it does not wait for the
// vector-memory operations in flight, such as LDS-DMA copies the compiler cannot see.
template <typename T>
__device__ __forceinline__ T ld_uniform(const void* p) {
    return *(const __attribute__((address_space(4))) T*)p;
}

// Reductions over each row of 16 lanes with DPP moves (VALU, no LDS round trip):
// swap neighbours, swap pairs, mirror the halves of 8, mirror the halves of 16.
// After each step the partners hold identical values, so every lane of the row ends
// with the same bits (the sum is order-independent only up to commutativity).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_mov<0xB1>(x));     // quad_perm(1,0,3,2)
    x = fmaxf(x, dpp_mov<0x4E>(x));     // quad_perm(2,3,0,1)
    x = fmaxf(x, dpp_mov<0x141>(x));    // row_half_mirror
    x = fmaxf(x, dpp_mov<0x140>(x));    // row_mirror
    return x;
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_mov<0xB1>(x);
    x += dpp_mov<0x4E>(x);
    x += dpp_mov<0x141>(x);
    x += dpp_mov<0x140>(x);
    return x;
}

// max(x, 0) as an integer max on the bit pattern: negative floats are negative
// integers, non-negative floats keep their bits (one instruction, no NaN quieting).
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Workgroup barrier for LDS-only communication: waits for this wave's LDS
// operations, not for its outstanding global loads (so asynchronous global->LDS
// loads of a later tile stay in flight across it).  The memory clobber keeps the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Work-groups go to the 8 XCDs (each with its own L2) round-robin by linear id.  For
// a grid of nb blocks (nb a multiple of 8) this maps hardware id `lin` to a logical
// id such that logical ids [x nb/8, (x+1) nb/8) all run on XCD x: consecutive logical
// blocks share an L2.  Otherwise the identity.
__device__ __forceinline__ unsigned xcd_local_id(unsigned lin, unsigned nb) {
    return (nb & 7u) ? lin : (lin & 7u) * (nb >> 3) + (lin >> 3);
}

}  // namespace csl
