// dsa_device.h -- device-side helpers shared by the DSA kernels (gfx950 only).
//
// Vector types for MFMA operands, bit-exact number-format conversions
// (bf16, OCP E4M3), wavefront helpers and the order-preserving float key
// used by the top-k selection.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

#define DSA_LDS __attribute__((address_space(3)))

constexpr int kWave = 64;
constexpr int kPage = 64;       // indexer key-cache page (tokens)
constexpr int kDk = 576;        // latent key width
constexpr int kDv = 512;        // value width (leading dims of the latent row)

// ---------------------------------------------------------------- MFMA
// FP8 (OCP E4M3) x FP8 -> fp32, 32x32 tile, K = 64.  Operand layout
// (measured): lane l holds row/col l%32 and K bytes [32*(l/32), +32) of the
// K block; the accumulator's element i of lane l is row 8*(i/4) + 4*(l/32)
// + i%4, column l%32.  Scale operands 0 select unit scales.
__device__ __forceinline__ f32x16 mfma_f8_32x32x64(const i32x8 &a, const i32x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// bf16 x bf16 -> fp32, 32x32 tile, K = 16: lane l holds row/col l%32 and
// K elements [8*(l/32), +8); accumulator layout as above.
__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- formats
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// OCP E4M3 code -> bf16 bits, exact (3 mantissa bits, exponents 2^-9..2^8
// all fit bf16).  Written from the format definition: normal codes move the
// exponent from bias 7 to bias 127; subnormal codes m * 2^-9 are normalised.
__device__ __forceinline__ uint32_t e4m3_to_bf16_bits(uint32_t c) {
    uint32_t s = (c & 0x80u) << 8;
    uint32_t e = (c >> 3) & 15u;
    uint32_t m = c & 7u;
    if (e != 0) return s | ((e + 120u) << 7) | (m << 4);
    if (m == 0) return s;
    // m in 1..7: value m * 2^-9; leading bit position p = 0..2
    uint32_t p = 31u - __builtin_clz(m);
    uint32_t frac = (m << (3u - p)) & 7u;                  // remaining bits below the leading one
    return s | ((p + 118u) << 7) | (frac << 4);            // exponent p - 9 + 127
}

// fp32 -> OCP E4M3 code, round to nearest even, saturate to +-448, NaN -> 0x7F.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
    uint32_t u = __float_as_uint(x);
    uint32_t sign = (u >> 24) & 0x80u;
    float a = __builtin_fabsf(x);
    if (!(a < 448.0f)) return (a != a) ? 0x7Fu : (sign | 0x7Eu);
    if (a < 0.015625f) {                                    // below 2^-6: steps of 2^-9
        float q = __builtin_rintf(a * 512.0f);              // exact scaling, RNE
        return sign | (uint32_t)q;                          // q == 8 encodes 2^-6 (0x08)
    }
    uint32_t ua = __float_as_uint(a);
    uint32_t r = ua + 0x7FFFFu + ((ua >> 20) & 1u);         // RNE to 3 mantissa bits
    r &= 0xFFF00000u;
    uint32_t e = (r >> 23) - 120u;                          // (E - 127) + 7
    return sign | (e << 3) | ((r >> 20) & 7u);
}

// ---------------------------------------------------------------- keys
// Order-preserving map fp32 -> uint32 (larger float -> larger key), with
// -0.0 and +0.0 mapped to the same key.
__device__ __forceinline__ uint32_t f32_order_key(float x) {
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// gfx950 lane swap between the two 32-lane halves (measured):
//   r = permlane32_swap(a, b):  r[0] = a with lanes 32..63 replaced by b's lanes 0..31,
//                               r[1] = b with lanes 0..31 replaced by a's lanes 32..63.
// Reduce-scatter of two per-lane partials: lane i < 32 gets a[i] + a[i+32],
// lane 32+i gets b[i] + b[32+i].
__device__ __forceinline__ float halves_reduce_scatter(float a, float b) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// x from lane l ^ 32.
__device__ __forceinline__ float swap_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

}  // namespace dsa
