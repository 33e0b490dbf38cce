// device_common.h -- small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// dtype codes, equal to pda_dtype
enum : int { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2, DT_INT8 = 3, DT_INT4 = 4 };

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round-to-nearest-even fp32 -> bf16 bits (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Split x into bf16 hi (truncation) and bf16 lo (the exact remainder
// rounded to nearest, ties away from zero): |x - hi - lo| <= 2^-16 |x|
// (the remainder is below 2^-7 |x|, and rounding it to 8 significant bits
// errs by at most half its last place). Truncating the remainder too would
// allow twice that. Returns the two bf16 bit patterns in the low halves.
__device__ __forceinline__ void split_bf16(float x, uint32_t& hi, uint32_t& lo) {
    const uint32_t u = __float_as_uint(x) & 0xFFFF0000u;
    const float r = x - __uint_as_float(u);       // exact
    hi = u >> 16;
    lo = (__float_as_uint(r) + 0x8000u) >> 16;    // the magnitude rounds; the sign bit stays
}

// Two values at once, with the gfx950 packed conversion: hi = bf16 RNE of x,
// lo = bf16 RNE of the exact remainder x - hi; the same bound,
// |x - hi - lo| <= 2^-16 |x| (the remainder is at most 2^-8 |x| and its
// rounding errs by at most 2^-8 of it). Returns the packed pairs (x0 in the
// low half).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split_bf16x2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    const f32x2 x = {x0, x1};
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
    const f32x2 r = {x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xFFFF0000u)};
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
}

// fp32 -> OCP E4M3 code, round to nearest even with saturation to +-448.
// NaN -> 0x7F; the sign of y is kept (so -0 -> 0x80).
__device__ __forceinline__ uint32_t quant_fp8_e4m3(float y) {
    const uint32_t u = __float_as_uint(y);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7Fu;
    const uint32_t sign = (u >> 24) & 0x80u;
    const float a = __uint_as_float(u & 0x7FFFFFFFu);
    uint32_t code;
    if (a >= 448.0f) {
        code = 0x7Eu;
    } else if (a < 0.015625f) {
        // subnormal range: value = m * 2^-9, m = 0..8 (m = 8 is the smallest
        // normal, whose code is also 8)
        code = (uint32_t)__builtin_rintf(a * 512.0f);
    } else {
        const int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;   // -6..8
        const float mul = __uint_as_float((uint32_t)(127 + 3 - e) << 23); // 2^(3-e)
        const float t = a * mul - 8.0f;                                   // exact, in [0, 8)
        code = (uint32_t)((e + 7) << 3) + (uint32_t)__builtin_rintf(t);  // carry = next exponent
    }
    return code | sign;
}

// fp32 -> symmetric int8 code: round half to even, clamp to [-127, 127]; NaN -> 0.
__device__ __forceinline__ int32_t quant_int8(float y) {
    if (y != y) return 0;
    const float r = __builtin_rintf(y);
    return (int32_t)fminf(fmaxf(r, -127.0f), 127.0f);
}

// Two fp32 values holding exact bf16 values -> packed bf16x2 (lo, hi).
__device__ __forceinline__ uint32_t pack_bf16_trunc(float lo, float hi) {
    // bytes 2, 3 of lo, then bytes 2, 3 of hi: one v_perm_b32
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// 4 fp8 codes (one dword) -> 4 bf16 (two dwords), exact.
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    u32x2 r;
    r.x = __builtin_bit_cast(uint32_t, a);
    r.y = __builtin_bit_cast(uint32_t, b);
    return r;
}

// 4 int8 codes (one dword) -> 4 bf16 (two dwords), exact (|code| <= 128).
__device__ __forceinline__ u32x2 int8x4_to_bf16x4(uint32_t w) {
    const float f0 = (float)(int32_t)(int8_t)(w & 0xFFu);
    const float f1 = (float)(int32_t)(int8_t)((w >> 8) & 0xFFu);
    const float f2 = (float)(int32_t)(int8_t)((w >> 16) & 0xFFu);
    const float f3 = (float)(int32_t)(int8_t)(w >> 24);
    u32x2 r;
    r.x = pack_bf16_trunc(f0, f1);
    r.y = pack_bf16_trunc(f2, f3);
    return r;
}

// Attended positions of an n-token row: all t < n (window == 0), or with a
// sliding window t < sinks or t >= n - window. A row lists the logical blocks
// that hold attended positions: the sink blocks [0, sb) and the window blocks
// [wstart, nblk); the blocks in between are skipped entirely.
struct RowBlocks {
    int count;    // attended blocks of the row
    int sb;       // leading (sink) blocks
    int wstart;   // logical block of the first window block
};

__device__ __forceinline__ RowBlocks row_blocks(int n, int window, int sinks) {
    const int nblk = (n + 15) >> 4;
    if (window <= 0 || n <= sinks + window) return RowBlocks{nblk, nblk, nblk};
    const int sb = (sinks + 15) >> 4;
    const int wstart = max((n - window) >> 4, sb);
    return RowBlocks{sb + (nblk - wstart), sb, wstart};
}

// The i-th attended block of a row -> its logical block.
__device__ __forceinline__ int row_block_logical(const RowBlocks& r, int i) {
    return i < r.sb ? i : r.wstart + (i - r.sb);
}

// Bit k set <=> position 16 L + k of the row is attended.
__device__ __forceinline__ uint32_t block_token_mask(int L, int n, int window, int sinks) {
    const int t0 = 16 * L;
    uint32_t m = n - t0 >= 16 ? 0xFFFFu : (n > t0 ? (1u << (n - t0)) - 1u : 0u);
    if (window > 0) {
        uint32_t keep = 0;
        const int s = sinks - t0;             // positions below it are sinks
        if (s > 0) keep |= s >= 16 ? 0xFFFFu : (1u << s) - 1u;
        const int w0 = n - window - t0;       // first window position in the block
        if (w0 <= 0) keep = 0xFFFFu;
        else if (w0 < 16) keep |= 0xFFFFu & ~((1u << w0) - 1u);
        m &= keep;
    }
    return m;
}


// XOR swizzle of the bf16 K staging tile (16 rows of 2 * HD bytes).
template <int HD>
__device__ __forceinline__ constexpr int kswz(int r) {
    return HD == 128 ? (r & 15) : ((r >> 1) & 7);
}

// Byte offset of (row t, 16-B chunk cb) in a bf16 LDS tile; the XOR keeps the
// 16 rows of a transposed read on distinct banks.
template <int HD>
__device__ __forceinline__ int lds_off(int t, int cb) {
    constexpr int CPR = HD / 8, RPS = 256 / (HD * 2);
    const int f = 2 * ((t / RPS) % (CPR / 2));
    return t * (HD * 2) + 16 * (cb ^ f);
}

// Reductions over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 16-lane
// rows of a wave) with the gfx950 row swaps: permlane16_swap exchanges rows
// 1 <-> 0 and 3 <-> 2 between its two operands, permlane32_swap the two
// halves; with both operands equal, each result pair holds a lane's value
// and its partner's.
__device__ __forceinline__ float max_rows4(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float sum_rows4(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int KV>
__device__ __forceinline__ bf16x8 kv_operand_from_bytes(uint4 w, int half) {
    if (KV == DT_BF16) {
        return __builtin_bit_cast(bf16x8, w);
    } else {
        const uint32_t a = half ? w.z : w.x;
        const uint32_t b = half ? w.w : w.y;
        u32x2 lo, hi;
        if (KV == DT_FP8) { lo = fp8x4_to_bf16x4(a); hi = fp8x4_to_bf16x4(b); }
        else { lo = int8x4_to_bf16x4(a); hi = int8x4_to_bf16x4(b); }
        u32x4 r = {lo.x, lo.y, hi.x, hi.y};
        return __builtin_bit_cast(bf16x8, r);
    }
}


// Shared-prefix length of a row as the attention kernels use it: logical
// blocks 0 .. p - 1 of the row are the shared prefix blocks. `n` is the
// row's context length, `pl` its requested prefix length. Returns -1 when the
// row is invalid (n outside [0, max_blocks * 16], or a prefix that is
// negative, longer than the prefix table, or reaching the block that holds
// the row's newest position, which copy on write keeps private), else the
// prefix length (0 for an empty row).
__device__ __forceinline__ int row_prefix_len(int n, int pl, int max_blocks, int prefix_blocks) {
    if (n < 0 || n > max_blocks * 16) return -1;
    if (n == 0) return 0;
    if (pl < 0 || pl > prefix_blocks || pl >= ((n + 15) >> 4)) return -1;
    return pl;
}

// One packed group of 8 four-bit channels (a dword: byte i holds channel i
// in its low nibble and channel i + 4 in its high nibble, each stored as
// code + 8) -> the bf16 values 128 + nibble = 136 + code, in channel order.
// 128 + n is exact in bf16 (exponent 2^7, mantissa unit 1), so the bytes are
// only moved: v_perm_b32 pairs each nibble with the exponent byte 0x43.
__device__ __forceinline__ bf16x8 int4x8_to_bf16_biased(uint32_t w) {
    const uint32_t lo = w & 0x0F0F0F0Fu;          // channels 0..3
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // channels 4..7
    const uint32_t e = 0x43434343u;
    const u32x4 r = {__builtin_amdgcn_perm(e, lo, 0x04010400u), __builtin_amdgcn_perm(e, lo, 0x04030402u),
                     __builtin_amdgcn_perm(e, hi, 0x04010400u), __builtin_amdgcn_perm(e, hi, 0x04030402u)};
    return __builtin_bit_cast(bf16x8, r);
}
constexpr float kInt4Bias = 136.0f;   // 128 + 8: the biased value minus the code

// fp32 -> symmetric 4-bit code nibble: RNE(y) clamped to [-7, 7] (NaN -> 0),
// returned as code + 8.
__device__ __forceinline__ uint32_t quant_int4_nibble(float y) {
    const float r = y != y ? 0.0f : fminf(fmaxf(__builtin_rintf(y), -7.0f), 7.0f);
    return (uint32_t)((int)r + 8);
}

}  // namespace pda
