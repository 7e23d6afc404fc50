// Bandwidth-bound kernels: forward corruption, embedding + self-conditioning,
// p0 materialisation for checking, and a fill.
#include "dg_device.hpp"
#include "dg_kernels.hpp"

namespace dg {

// Forward corruption (DiffusionGemma Technical Report, hyper.ai summary,
// Method, forward path equation): each token keeps x0 with probability kappa_b
// and is otherwise a uniform token over [0, V). One Philox block serves the
// token pair (2j, 2j+1) of a canvas: words 0/1 for the even token, 2/3 for the
// odd one (keep draw, replacement word). x0 and out may be the same array.
__global__ void __launch_bounds__(256) corrupt_kernel(const int32_t *x0,
                                                      const float *__restrict__ kappa, int B,
                                                      int C, uint32_t V, uint32_t k0, uint32_t k1,
                                                      int32_t *out, bool vec2) {
  const uint32_t pairs = (static_cast<uint32_t>(C) + 1u) >> 1;
  const uint64_t total = static_cast<uint64_t>(B) * pairs;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  for (uint64_t p = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; p < total;
       p += stride) {
    const uint32_t b = static_cast<uint32_t>(p / pairs);
    const uint32_t j = static_cast<uint32_t>(p - static_cast<uint64_t>(b) * pairs);
    const u32x4 w = philox4x32_10(j, 0u, b, kStreamCorrupt, k0, k1);
    const float kap = kappa[b];
    const int64_t base = static_cast<int64_t>(b) * C + 2 * static_cast<int64_t>(j);
    if (vec2) {  // C even and 8-byte aligned rows: one 8-byte load and store
      const int2 xv = *reinterpret_cast<const int2 *>(x0 + base);
      int2 r;
      r.x = (u01(w.x) < kap) ? xv.x : static_cast<int32_t>(__umulhi(w.y, V));
      r.y = (u01(w.z) < kap) ? xv.y : static_cast<int32_t>(__umulhi(w.w, V));
      *reinterpret_cast<int2 *>(out + base) = r;
    } else {
      const int32_t xa = x0[base];
      out[base] = (u01(w.x) < kap) ? xa : static_cast<int32_t>(__umulhi(w.y, V));
      if (2 * j + 1 < static_cast<uint32_t>(C)) {
        const int32_t xb = x0[base + 1];
        out[base + 1] = (u01(w.z) < kap) ? xb : static_cast<int32_t>(__umulhi(w.w, V));
      }
    }
  }
}

// The same draws for C % 4 == 0, 16-byte aligned arrays and fewer than 2^32
// quads. A quad is four tokens (two pairs) of one canvas: one 16-byte load and
// store. A thread takes quads base + 256 u, u < kQuadU, per iteration and
// issues all their loads before the Philox work, so each wave keeps kQuadU
// streaming loads in flight. The loads and stores are nontemporal: x0 is read
// once and x_t written once. Measured with plain copies of 1 GiB: one 8-byte
// load per thread and iteration copies at about 4.8 TB/s, four 16-byte
// nontemporal loads per thread at about 6 TB/s; this kernel, Philox included,
// at 5.6-5.7 TB/s with up to 64 blocks per CU.
constexpr int kQuadU = 4;
typedef int i32x4v __attribute__((ext_vector_type(4)));

// x0 and out may be the same array (no __restrict__): every quad is loaded
// before it is stored, by the same thread.
__global__ void __launch_bounds__(256) corrupt_quad_kernel(const int32_t *x0,
                                                           const float *__restrict__ kappa,
                                                           uint32_t qpc, uint64_t nquads, uint32_t V,
                                                           uint32_t k0, uint32_t k1, int32_t *out) {
  const i32x4v *src = reinterpret_cast<const i32x4v *>(x0);
  i32x4v *dst = reinterpret_cast<i32x4v *>(out);
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * 256 * kQuadU;
  for (uint64_t base = static_cast<uint64_t>(blockIdx.x) * 256 * kQuadU + threadIdx.x; base < nquads;
       base += stride) {
    i32x4v xv[kQuadU];
#pragma unroll
    for (int u = 0; u < kQuadU; ++u) {
      const uint64_t q = base + 256u * u;
      xv[u] = (q < nquads) ? __builtin_nontemporal_load(src + q) : i32x4v{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kQuadU; ++u) {
      const uint64_t q = base + 256u * u;
      if (q >= nquads) break;
      const uint32_t q32 = static_cast<uint32_t>(q);   // nquads < 2^32
      const uint32_t b = q32 / qpc;
      const uint32_t j = 2u * (q32 - b * qpc);
      // u01(w) < kappa in integers: u01(w) = (2 (w >> 9) + 1) 2^-24 exactly,
      // so the draw keeps x0 iff 2 (w >> 9) + 1 < T = kappa 2^24 (exact), iff
      // (w >> 9) < ceil((T - 1) / 2); every step of that bound is exact in
      // fp32 for T up to 2^24 (and the conversion saturates above)
      const int kth = static_cast<int>(ceilf((kappa[b] * 16777216.f - 1.f) * 0.5f));
      const u32x4 w0 = philox4x32_10(j, 0u, b, kStreamCorrupt, k0, k1);
      const u32x4 w1 = philox4x32_10(j + 1u, 0u, b, kStreamCorrupt, k0, k1);
      i32x4v r;
      r.x = (static_cast<int>(w0.x >> 9) < kth) ? xv[u].x : static_cast<int32_t>(__umulhi(w0.y, V));
      r.y = (static_cast<int>(w0.z >> 9) < kth) ? xv[u].y : static_cast<int32_t>(__umulhi(w0.w, V));
      r.z = (static_cast<int>(w1.x >> 9) < kth) ? xv[u].z : static_cast<int32_t>(__umulhi(w1.y, V));
      r.w = (static_cast<int>(w1.z >> 9) < kth) ? xv[u].w : static_cast<int32_t>(__umulhi(w1.w, V));
      __builtin_nontemporal_store(r, dst + q);
    }
  }
}

hipError_t launch_corrupt(const int32_t *x0, const float *kappa, int B, int C, int V,
                          uint64_t seed, int32_t *out, hipStream_t st) {
  const uint64_t nquads = static_cast<uint64_t>(B) * (C / 4);
  const bool quad = (C % 4 == 0) && nquads < (uint64_t{1} << 32) &&
                    (reinterpret_cast<uintptr_t>(x0) % 16 == 0) &&
                    (reinterpret_cast<uintptr_t>(out) % 16 == 0);
  if (quad) {
    if (nquads == 0) return hipSuccess;
    uint64_t blocks = (nquads + 256 * kQuadU - 1) / (256 * kQuadU);
    if (blocks > 256 * 64) blocks = 256 * 64;  // grid-stride beyond 64 blocks per CU
    hipLaunchKernelGGL(corrupt_quad_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st, x0,
                       kappa, static_cast<uint32_t>(C / 4), nquads, static_cast<uint32_t>(V),
                       static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32), out);
    return hipGetLastError();
  }
  const uint64_t pairs = static_cast<uint64_t>(B) * ((C + 1) / 2);
  const bool vec2 = (C % 2 == 0) && (reinterpret_cast<uintptr_t>(x0) % 8 == 0) &&
                    (reinterpret_cast<uintptr_t>(out) % 8 == 0);
  uint64_t blocks = (pairs + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;  // grid-stride beyond 64 blocks per CU
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(corrupt_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st, x0,
                     kappa, B, C, static_cast<uint32_t>(V), static_cast<uint32_t>(seed),
                     static_cast<uint32_t>(seed >> 32), out, vec2);
  return hipGetLastError();
}

// h0 = round(E[x] + z): one block per row, 8 elements (16 bytes of bf16) per
// thread and iteration when the row width allows it.
// Step constants of up to kInlineParams canvases ride along with the embedding
// launch as a kernel argument: block 0 stores them for the later kernels of
// the step, which run after this one on the same stream.
struct InlineParams {
  StepParams p[kInlineParams];
};

__device__ __forceinline__ void store_inline_params(StepParams *dst, const InlineParams &c, int n) {
  if (blockIdx.x == 0 && static_cast<int>(threadIdx.x) < n) dst[threadIdx.x] = c.p[threadIdx.x];
}

// A token outside [0, V) reads as a zero embedding row instead of faulting.
template <typename T>
__global__ void __launch_bounds__(256) embed_kernel(const T *__restrict__ E,
                                                    const int32_t *__restrict__ x,
                                                    const T *__restrict__ z, int d, int V,
                                                    T *__restrict__ h0, StepParams *prm,
                                                    InlineParams pc, int np) {
  store_inline_params(prm, pc, np);
  const int r = blockIdx.x;
  const int32_t tok = x[r];
  const bool in = tok >= 0 && tok < V;
  const T *er = E + static_cast<int64_t>(in ? tok : 0) * d;
  const T *zr = z ? z + static_cast<int64_t>(r) * d : nullptr;
  T *hr = h0 + static_cast<int64_t>(r) * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    float v = in ? Act<T>::load(er, c) : 0.f;
    if (zr) v += Act<T>::load(zr, c);
    Act<T>::store(hr, c, v);
  }
}

__global__ void __launch_bounds__(256) embed_bf16_vec_kernel(const uint16_t *__restrict__ E,
                                                             const int32_t *__restrict__ x,
                                                             const uint16_t *__restrict__ z,
                                                             int d, int V,
                                                             uint16_t *__restrict__ h0,
                                                             StepParams *prm, InlineParams pc,
                                                             int np) {
  store_inline_params(prm, pc, np);
  const int r = blockIdx.x;
  const int32_t tok = x[r];
  const bool in = tok >= 0 && tok < V;
  const uint4 *er = reinterpret_cast<const uint4 *>(E + static_cast<int64_t>(in ? tok : 0) * d);
  const uint4 *zr = z ? reinterpret_cast<const uint4 *>(z + static_cast<int64_t>(r) * d) : nullptr;
  uint4 *hr = reinterpret_cast<uint4 *>(h0 + static_cast<int64_t>(r) * d);
  for (int c = threadIdx.x; c < d / 8; c += blockDim.x) {
    const uint4 e = in ? er[c] : make_uint4(0, 0, 0, 0);
    uint4 o = e;
    if (zr) {
      const uint4 zz = zr[c];
      const uint32_t ew[4] = {e.x, e.y, e.z, e.w};
      const uint32_t zw[4] = {zz.x, zz.y, zz.z, zz.w};
      uint32_t ow[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = bf16_to_f32(ew[i] & 0xFFFFu) + bf16_to_f32(zw[i] & 0xFFFFu);
        const float hi = bf16_to_f32(ew[i] >> 16) + bf16_to_f32(zw[i] >> 16);
        ow[i] = pack_bf16x2(lo, hi);
      }
      o = make_uint4(ow[0], ow[1], ow[2], ow[3]);
    }
    hr[c] = o;
  }
}

// RMSNorm of the decoder stack: y = round(x / sqrt(mean(x^2) + eps) * g), one
// block per row, fp32 sums. Rows of up to 512 16-byte pieces stay in
// registers between the sum of squares and the scaling (16-byte loads and
// stores); longer rows or unaligned pointers take the scalar loop.
template <typename T>
__device__ __forceinline__ void unpack16(const uint4 &q, float (&v)[16 / sizeof(T)]) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    v[0] = __uint_as_float(q.x); v[1] = __uint_as_float(q.y);
    v[2] = __uint_as_float(q.z); v[3] = __uint_as_float(q.w);
  }
}
template <typename T>
__device__ __forceinline__ uint4 pack16(const float (&v)[16 / sizeof(T)]) {
  if constexpr (sizeof(T) == 2) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16(v[2 * i])) | (static_cast<uint32_t>(f32_to_bf16(v[2 * i + 1])) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
  }
}

template <typename T>
__global__ void __launch_bounds__(256) rmsnorm_kernel(const T *__restrict__ x,
                                                      const T *__restrict__ g, int d, float eps,
                                                      T *__restrict__ y) {
  constexpr int VW = 16 / sizeof(T);               // elements per 16-byte piece
  constexpr int PPT = 2;                           // pieces per thread, at most
  __shared__ float red[4];
  const int r = blockIdx.x;
  const T *xr = x + static_cast<int64_t>(r) * d;
  T *yr = y + static_cast<int64_t>(r) * d;
  const bool vec = (d % VW) == 0 && d / VW <= PPT * 256 &&
                   ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(g) |
                     reinterpret_cast<uintptr_t>(y)) & 15) == 0;
  float v[PPT][VW];
  float ss = 0.f;
  if (vec) {
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int c = threadIdx.x + 256 * k;         // this thread's pieces
      if (c < d / VW) {
        unpack16<T>(*reinterpret_cast<const uint4 *>(xr + c * VW), v[k]);
#pragma unroll
        for (int i = 0; i < VW; ++i) ss = fmaf(v[k][i], v[k][i], ss);
      }
    }
  } else {
    for (int k = threadIdx.x; k < d; k += blockDim.x) {
      const float t = Act<T>::load(xr, k);
      ss = fmaf(t, t, ss);
    }
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float inv = 1.f / sqrtf(tot / static_cast<float>(d) + eps);
  if (vec) {
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int c = threadIdx.x + 256 * k;
      if (c < d / VW) {
        float gv[VW];
        unpack16<T>(*reinterpret_cast<const uint4 *>(g + c * VW), gv);
#pragma unroll
        for (int i = 0; i < VW; ++i) v[k][i] = v[k][i] * inv * gv[i];
        *reinterpret_cast<uint4 *>(yr + c * VW) = pack16<T>(v[k]);
      }
    }
  } else {
    for (int k = threadIdx.x; k < d; k += blockDim.x)
      Act<T>::store(yr, k, Act<T>::load(xr, k) * inv * Act<T>::load(g, k));
  }
}

hipError_t launch_rmsnorm(bool bf16, const void *x, const void *g, int R, int d, float eps, void *y,
                          hipStream_t st) {
  if (R == 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(rmsnorm_kernel<uint16_t>, dim3(R), dim3(256), 0, st,
                       static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(g), d, eps,
                       static_cast<uint16_t *>(y));
  else
    hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3(R), dim3(256), 0, st, static_cast<const float *>(x),
                       static_cast<const float *>(g), d, eps, static_cast<float *>(y));
  return hipGetLastError();
}

// Token rows for the encoder: row m = b * n + i embeds x[b * ld + i] (a token
// outside [0, V) reads as a zero row).
template <typename T>
__global__ void __launch_bounds__(256) embed_tokens_kernel(const T *__restrict__ E,
                                                           const int32_t *__restrict__ x, int ld,
                                                           int n, int d, int V, T *__restrict__ h) {
  const int m = blockIdx.x;
  const int b = m / n, i = m - b * n;
  const int32_t tok = x[static_cast<int64_t>(b) * ld + i];
  const bool in = tok >= 0 && tok < V;
  const T *er = E + static_cast<int64_t>(in ? tok : 0) * d;
  T *hr = h + static_cast<int64_t>(m) * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) hr[c] = in ? er[c] : T(0);
}

// One thread per unit U (16 or 4 bytes) of a (canvas, kv head, row) of k and of v.
template <typename U>
__global__ void __launch_bounds__(256) kv_to_cache_kernel(const U *__restrict__ k, const U *__restrict__ v,
                                                          int64_t rows, int C, int Pst, int row0, int q,
                                                          U *__restrict__ K, U *__restrict__ V) {
  const int64_t half = rows * q;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < 2 * half;
       t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const bool isv = t >= half;
    const int64_t u = isv ? t - half : t;
    const int64_t row = u / q;               // (slice, i) with slice = b * Hkv + g
    const int e = static_cast<int>(u - row * q);
    const int64_t slice = row / C;
    const int i = static_cast<int>(row - slice * C);
    const int64_t dst = (slice * Pst + row0 + i) * q + e;
    if (isv)
      V[dst] = v[u];
    else
      K[dst] = k[u];
  }
}

hipError_t launch_kv_to_cache(bool bf16, const void *k, const void *v, const Shape &s, int row0,
                              void *K, void *V, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(s.B) * s.Hkv * s.C;
  const int bytes = s.hd * (bf16 ? 2 : 4);
  if (rows == 0) return hipSuccess;
  const auto a16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  const bool wide = bytes % 16 == 0 && a16(k) && a16(v) && a16(K) && a16(V);
  const int q = wide ? bytes / 16 : bytes / 4;
  int64_t blocks = (2 * rows * q + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (wide)
    hipLaunchKernelGGL(kv_to_cache_kernel<uint4>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st,
                       static_cast<const uint4 *>(k), static_cast<const uint4 *>(v), rows, s.C,
                       s.pstride(), row0, q, static_cast<uint4 *>(K), static_cast<uint4 *>(V));
  else
    hipLaunchKernelGGL(kv_to_cache_kernel<uint32_t>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                       st, static_cast<const uint32_t *>(k), static_cast<const uint32_t *>(v), rows, s.C,
                       s.pstride(), row0, q, static_cast<uint32_t *>(K), static_cast<uint32_t *>(V));
  return hipGetLastError();
}

hipError_t launch_embed_tokens(bool bf16, const void *E, const int32_t *x, int ld, int B, int n,
                               int d, int V, void *h, hipStream_t st) {
  if (static_cast<int64_t>(B) * n == 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(embed_tokens_kernel<uint16_t>, dim3(B * n), dim3(256), 0, st,
                       static_cast<const uint16_t *>(E), x, ld, n, d, V, static_cast<uint16_t *>(h));
  else
    hipLaunchKernelGGL(embed_tokens_kernel<float>, dim3(B * n), dim3(256), 0, st,
                       static_cast<const float *>(E), x, ld, n, d, V, static_cast<float *>(h));
  return hipGetLastError();
}

hipError_t launch_embed(bool bf16, const void *E, const int32_t *x, const void *z, int R, int d,
                        int V, void *h0, StepParams *prm, const StepParams *prm_src, int np,
                        hipStream_t st) {
  if (np < 0 || np > kInlineParams || (np > 0 && (!prm || !prm_src))) return hipErrorInvalidValue;
  if (R == 0) return np ? launch_set_params(prm, prm_src, np, st) : hipSuccess;
  InlineParams pc;
  for (int i = 0; i < np; ++i) pc.p[i] = prm_src[i];
  for (int i = np; i < kInlineParams; ++i) pc.p[i] = StepParams{0.f, 0.f};
  if (bf16) {
    if (d % 8 == 0)
      hipLaunchKernelGGL(embed_bf16_vec_kernel, dim3(R), dim3(256), 0, st,
                         static_cast<const uint16_t *>(E), x, static_cast<const uint16_t *>(z), d,
                         V, static_cast<uint16_t *>(h0), prm, pc, np);
    else
      hipLaunchKernelGGL(embed_kernel<uint16_t>, dim3(R), dim3(256), 0, st,
                         static_cast<const uint16_t *>(E), x, static_cast<const uint16_t *>(z), d,
                         V, static_cast<uint16_t *>(h0), prm, pc, np);
  } else {
    hipLaunchKernelGGL(embed_kernel<float>, dim3(R), dim3(256), 0, st,
                       static_cast<const float *>(E), x, static_cast<const float *>(z), d,
                       V, static_cast<float *>(h0), prm, pc, np);
  }
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) p0_kernel(float *__restrict__ p0,
                                                 const float *__restrict__ lse, int V) {
  const int r = blockIdx.y;
  const float l = lse[r];
  float *row = p0 + static_cast<int64_t>(r) * V;
  for (int v = blockIdx.x * blockDim.x + threadIdx.x; v < V; v += gridDim.x * blockDim.x)
    row[v] = expf(row[v] - l);
}

hipError_t launch_p0_from_logits(float *p0, const float *lse, int R, int V, hipStream_t st) {
  if (R == 0) return hipSuccess;
  int bx = (V + 255) / 256;
  if (bx > 64) bx = 64;
  hipLaunchKernelGGL(p0_kernel, dim3(bx, R), dim3(256), 0, st, p0, lse, V);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) fill_zero_kernel(uint32_t *__restrict__ p, size_t n) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

__global__ void __launch_bounds__(256) fill_i32_kernel(int32_t *__restrict__ p, size_t n, int32_t v) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_i32(int32_t *p, size_t n, int32_t v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t st) {
  // bytes is a multiple of 4 for every caller (fp32 or bf16 pairs of even width)
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st,
                     static_cast<uint32_t *>(p), n);
  return hipGetLastError();
}

// Small host arrays travel as kernel arguments (copied at launch), so no host
// buffer has to outlive the call and no pinned memory is needed.
struct ParamChunk {
  StepParams p[256];
};
struct FloatChunk {
  float f[512];
};

__global__ void set_params_kernel(StepParams *__restrict__ dst, ParamChunk c, int n) {
  const int i = threadIdx.x;
  if (i < n) dst[i] = c.p[i];
}

__global__ void set_floats_kernel(float *__restrict__ dst, FloatChunk c, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = c.f[i];
}

hipError_t launch_set_params(StepParams *dst, const StepParams *src, int n, hipStream_t st) {
  for (int off = 0; off < n; off += 256) {
    ParamChunk c;
    const int k = (n - off < 256) ? n - off : 256;
    for (int i = 0; i < k; ++i) c.p[i] = src[off + i];
    hipLaunchKernelGGL(set_params_kernel, dim3(1), dim3(256), 0, st, dst + off, c, k);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_set_floats(float *dst, const float *src, int n, hipStream_t st) {
  for (int off = 0; off < n; off += 512) {
    FloatChunk c;
    const int k = (n - off < 512) ? n - off : 512;
    for (int i = 0; i < k; ++i) c.f[i] = src[off + i];
    hipLaunchKernelGGL(set_floats_kernel, dim3(1), dim3(256), 0, st, dst + off, c, k);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dg
