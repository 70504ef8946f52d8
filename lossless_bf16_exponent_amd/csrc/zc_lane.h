// Per-lane bit manipulation of the BF16 exponent codec (gfx950).
//
// One lane handles 8 consecutive BF16 values held in 4 dwords (two values per
// dword, the lower-indexed value in the low half).  Everything is integer
// byte/bit work on whole dwords: v_perm_b32 byte shuffles, v_bfi_b32 bit
// merges and packed 16-bit saturating arithmetic, so one instruction handles
// two or four values.  The helpers are __host__ __device__ so that a CPU build
// can check them bit for bit.
//
// The split follows the ZipCCL explainer pages ("ZipCCL: Efficient Lossless
// Data Compression of Communication Collectives for Accelerating LLM
// Training", section 2.B): a BF16 value is 1 sign bit, 8 exponent bits and 7
// mantissa bits; the sign and mantissa travel as one byte, the exponent is
// replaced by a 3-bit code, and the code is stored as three 1-bit planes
// (section 2.C).
#pragma once

#include "zc_format.h"

namespace zc {

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// v_perm_b32: byte i of the result is byte sel[i] of the 64-bit value
// {hi:lo} (selectors 0..3 pick from lo, 4..7 from hi, 12 gives 0x00).
ZC_HD uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_perm(hi, lo, sel);
#else
    uint64_t v = ((uint64_t)hi << 32) | lo;
    uint32_t r = 0;
    for (int i = 0; i < 4; ++i) {
        uint32_t s = (sel >> (8 * i)) & 0xFFu;
        uint32_t b = s < 8 ? (uint32_t)(v >> (8 * s)) & 0xFFu : (s == 12 ? 0u : 0xFFu);
        r |= b << (8 * i);
    }
    return r;
#endif
}

// v_bfi_b32: bits of a where mask is set, bits of b elsewhere.
ZC_HD uint32_t bfi(uint32_t mask, uint32_t a, uint32_t b) { return (mask & a) | (~mask & b); }

ZC_HD u16x2 as_u16x2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }
ZC_HD uint32_t as_u32(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// Byte selectors over two dwords d0 (values 0,1) and d1 (values 2,3).
constexpr uint32_t kSelLowBytes = 0x06040200u;   // low byte of each value
constexpr uint32_t kSelHighBytes = 0x07050301u;  // high byte of each value

// Sign+mantissa bytes of 4 values: sign (bit 15) to bit 7, mantissa (bits 6..0)
// stays.  The high byte supplies bit 7, the low byte bits 6..0.
ZC_HD uint32_t sign_mantissa4(uint32_t d0, uint32_t d1) {
    uint32_t lo = perm(d1, d0, kSelLowBytes);
    uint32_t hi = perm(d1, d0, kSelHighBytes);
    return bfi(0x80808080u, hi, lo);
}

// Each value shifted left by one inside its 16-bit half: the exponent field
// then fills the high byte of the half (the sign bit drops out).
ZC_HD uint32_t exponent_high(uint32_t d) { return as_u32(as_u16x2(d) << (uint16_t)1); }

// Exponent bytes of 4 values from two exponent_high() words.
ZC_HD uint32_t exponents4(uint32_t t0, uint32_t t1) { return perm(t1, t0, kSelHighBytes); }

// Codes of 4 values when the seven exponents are the window base+1 .. base+7:
// high byte of sat(t - base<<8) is e - base (0 below the window), clamped to
// 8 above it; 1..7 are the codes, 0 and 8 mean zero-point (bits 0..2 clear).
ZC_HD uint32_t window_codes4(uint32_t t0, uint32_t t1, uint32_t base_hi) {
    const u16x2 b = as_u16x2(base_hi);
    const u16x2 cap = as_u16x2(0x08000800u);
    uint32_t v0 = as_u32(__builtin_elementwise_min(__builtin_elementwise_sub_sat(as_u16x2(t0), b), cap));
    uint32_t v1 = as_u32(__builtin_elementwise_min(__builtin_elementwise_sub_sat(as_u16x2(t1), b), cap));
    return perm(v1, v0, kSelHighBytes);
}

// Two 4x4 bit transposes at once, one on the low nibbles of the four bytes and
// one on the high nibbles: bit b of byte k moves to bit k of byte b, and bit
// 4 + b of byte k to bit 4 + k of byte b (k, b in 0..3).  Two exchange stages
// (single bits across a distance of 7, then 2x2 blocks across 14); every
// exchanged pair lies inside one nibble matrix, so the two never mix.
// Each stage swaps bit p with bit p + d for p in a mask, written as
// t = (x ^ x >> d) & mask, x ^= t ^ t << d (two 3-input bit operations).
ZC_HD uint32_t nibble_transpose2(uint32_t x) {
    uint32_t t = (x ^ (x >> 7)) & 0x00AA00AAu;
    x = x ^ t ^ (t << 7);
    t = (x ^ (x >> 14)) & 0x0000CCCCu;
    return x ^ t ^ (t << 14);
}

// Code bytes of 8 values (c_lo: values 0..3, c_hi: 4..7; each byte at most 8)
// -> plane bytes: byte b of the result holds bit b of the 8 codes, value k in
// bit k.  Byte 3 (bit 3 of the codes) is unspecified.
ZC_HD uint32_t codes_to_planes(uint32_t c_lo, uint32_t c_hi) { return nibble_transpose2(c_lo | (c_hi << 4)); }

// Inverse: plane bytes (byte b = plane b, byte 3 ignored) -> code bytes 0..7.
ZC_HD void planes_to_codes(uint32_t planes, uint32_t &c_lo, uint32_t &c_hi) {
    const uint32_t x = nibble_transpose2(planes);
    c_lo = x & 0x07070707u;
    c_hi = (x >> 4) & 0x07070707u;
}

// Zero-point mask of 8 values: bit k set when value k has code 000.
ZC_HD uint32_t zero_point_mask(uint32_t planes) {
    return ~(planes | (planes >> 8) | (planes >> 16)) & 0xFFu;
}

// Rebuild 4 BF16 values (two dwords) from 4 sign+mantissa bytes and 4
// exponent bytes: high byte = sign | e >> 1, low byte = (e & 1) << 7 | mantissa.
ZC_HD void rebuild4(uint32_t sm, uint32_t e, uint32_t &d0, uint32_t &d1) {
    uint32_t hi = bfi(0x80808080u, sm, e >> 1);
    uint32_t lo = bfi(0x7F7F7F7Fu, sm, e << 7);
    d0 = perm(hi, lo, 0x05010400u);
    d1 = perm(hi, lo, 0x07030602u);
}

// Byte k (0..7) of the 8-byte value {hi:lo}.
ZC_HD uint32_t get_byte8(uint32_t lo, uint32_t hi, uint32_t k) {
    return ((k < 4 ? lo : hi) >> (8u * (k & 3u))) & 0xFFu;
}

}  // namespace zc
