// Device-side helpers shared by the gfx950 kernels of libdg.
//
// Philox4x32-10 follows Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
// as easy as 1, 2, 3" (SC'11): ten rounds; each multiplies counter words 0 and
// 2 by fixed odd constants, keeps both 32-bit halves of the two products, and
// mixes the high halves with counter words 1 and 3 and the key; the key takes
// a Weyl increment before every round after the first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;

// ---------------------------------------------------------------- bf16 ----
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// Activation storage types: float (fp32 path) or uint16_t bf16 bits.
template <typename T> struct Act;
template <> struct Act<float> {
  static __device__ __forceinline__ float load(const float *p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float *p, int64_t i, float v) { p[i] = v; }
};
template <> struct Act<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t *p, int64_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(uint16_t *p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// -------------------------------------------------------------- Philox ----
struct u32x4 {
  uint32_t x, y, z, w;
};

// a ^ b ^ c in one gfx950 V_BITOP3_B32 (truth table 0x96 over the inputs
// 0xF0, 0xCC, 0xAA); the compiler emits two V_XOR_B32 for the plain form.
// Two of the six VALU instructions of every Philox round are saved this way:
// a Philox-only loop runs 28 % faster, and the corruption kernel (whose
// Philox work competes with its loads) streams 12-15 % faster.
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
  constexpr uint32_t kMul0 = 0xD2511F53u, kMul1 = 0xCD9E8D57u;
  constexpr uint32_t kWeyl0 = 0x9E3779B9u, kWeyl1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kWeyl0;
      k1 += kWeyl1;
    }
    const uint64_t p0 = static_cast<uint64_t>(kMul0) * c0;
    const uint64_t p1 = static_cast<uint64_t>(kMul1) * c2;
    const uint32_t n0 = xor3(static_cast<uint32_t>(p1 >> 32), c1, k0);
    const uint32_t n2 = xor3(static_cast<uint32_t>(p0 >> 32), c3, k1);
    c1 = static_cast<uint32_t>(p1);
    c3 = static_cast<uint32_t>(p0);
    c0 = n0;
    c2 = n2;
  }
  return {c0, c1, c2, c3};
}

// Word -> float in (0, 1): centre of one of 2^23 equal cells; exact in fp32.
__device__ __forceinline__ float u01(uint32_t w) {
  return static_cast<float>((w >> 9) * 2u + 1u) * 0x1p-24f;
}

// Gumbel(0, 1) noise -log(-log U) from the hardware base-2 logarithm
// (v_log_f32, relative error ~1e-7 even for U next to 1, where -log U is
// tiny and its relative accuracy is what matters).
__device__ __forceinline__ float gumbel(uint32_t w) {
  constexpr float kLn2 = 0.6931471805599453f;
  const float e = -kLn2 * __builtin_amdgcn_logf(u01(w));   // -ln U > 0
  return -kLn2 * __builtin_amdgcn_logf(e);
}

enum : uint32_t { kStreamGumbel = 0, kStreamBernoulli = 1, kStreamCorrupt = 2 };

// word 3 of a raw buffer resource on gfx950 (32-bit data format, no
// swizzle); loads past the resource's size return zero
constexpr int kBufferFlags = 0x00020000;

// Gumbel-stream counter layout: vocabulary id v uses word (v >> 4) & 3 of
// block 16 (v >> 6) + (v & 15), so block j of each aligned group of 64 ids
// serves ids j, j + 16, j + 32, j + 48.
__device__ __forceinline__ uint32_t gumbel_block_of(int v) {
  return 16u * static_cast<uint32_t>(v >> 6) + static_cast<uint32_t>(v & 15);
}
__device__ __forceinline__ int gumbel_word_of(int v) { return (v >> 4) & 3; }

// GELU in its tanh form, a/2 (1 + tanh(sqrt(2/pi) (a + 0.044715 a^3))), the
// activation of the gated self-conditioning block.
__device__ __forceinline__ float gelu_tanh(float a) {
  constexpr float kC = 0.7978845608028654f;   // sqrt(2 / pi)
  return 0.5f * a * (1.f + tanhf(kC * fmaf(0.044715f * a, a * a, a)));
}

// ------------------------------------------------------ small reductions ---
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace dg
