// Merge of the vocabulary-split partials and the Step select.
//
// DiffusionGemma Technical Report (hyper.ai summary), Method, three-line
// update. Per row: lse = logsumexp of the scaled logits, z = p0 E from the
// unnormalised split sums, and the Step draw (our Euler reading of Step):
// keep x_t unless the row's Bernoulli u < lambda_b, in which case take the
// Gumbel argmax over the whole vocabulary (ties: lowest id, i.e. the lowest
// split wins an exact tie between splits).
//
// Entropy-bounded step: every row keeps its Gumbel draw, and the merge also
// yields the row's entropy H = ln 2 (log2 L - S1 / L), with L the merged sum
// of exp2(t - M) and S1 the merged sum of exp2(t - M) (t - M) (t the scaled
// logits in log2 units, M the merged reference), and the plain argmax; the
// select kernel then decides which draws to keep.
//
// Grid: (row, strip of 1024 columns). The first wave of each block merges
// the row's split statistics (one split per lane, wave-wide max / sum /
// argmax); then every thread streams 4 consecutive columns of all splits.
// z partials are bf16 from the MFMA LM head and fp32 from the fp32 path.
#include "dg_device.hpp"
#include "dg_kernels.hpp"

namespace dg {
namespace {

constexpr int kMaxSplits = 64;

__device__ __forceinline__ float4 load4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ float4 load4(const uint16_t *p) {
  const uint2 v = *reinterpret_cast<const uint2 *>(p);
  return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                     __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
}
__device__ __forceinline__ float load1(const float *p) { return *p; }
__device__ __forceinline__ float load1(const uint16_t *p) { return bf16_to_f32(*p); }

template <typename T, typename ZP>
__global__ void __launch_bounds__(256) combine_kernel(const RowPartial *__restrict__ part,
                                                      const ZP *__restrict__ zpart, int splits,
                                                      const int32_t *__restrict__ x_t,
                                                      const StepParams *__restrict__ prm, int R,
                                                      int C, int d, uint32_t k0, uint32_t k1,
                                                      int32_t *__restrict__ x_out,
                                                      T *__restrict__ z_out,
                                                      float *__restrict__ lse,
                                                      int32_t *__restrict__ best, EntropyRows ent,
                                                      const int32_t *__restrict__ frozen,
                                                      const T *__restrict__ z_t) {
  __shared__ float wsh[kMaxSplits];
  __shared__ float inv_l;
  const int r = blockIdx.x;
  if (frozen && frozen[r / C]) {
    // a stopped canvas keeps its self-conditioning signal
    const int c0 = (blockIdx.y * blockDim.x + threadIdx.x) * 4;
    for (int c = c0; c < c0 + 4 && c < d; ++c)
      z_out[static_cast<int64_t>(r) * d + c] = z_t[static_cast<int64_t>(r) * d + c];
    return;
  }
  if (threadIdx.x < 64) {
    const int s = threadIdx.x;
    RowPartial p;
    p.m = -INFINITY;
    p.l = 0.f;
    p.best = -INFINITY;
    p.arg = -1;
    p.s1 = 0.f;
    p.dbest = -INFINITY;
    p.darg = -1;
    p.pad = 0;
    if (s < splits) p = part[static_cast<int64_t>(s) * R + r];
    const float M = wave_max(p.m);
    const float w = (s < splits) ? exp2f(p.m - M) : 0.f;
    const float L = wave_sum(w * p.l);
    wsh[s] = w;
    // argmax of the best draw over splits; an exact tie goes to the lower split
    float bv = p.arg >= 0 ? p.best : -INFINITY;
    int bs = p.arg >= 0 ? s : kMaxSplits;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int os = __shfl_xor(bs, o, 64);
      if (ov > bv || (ov == bv && os < bs)) { bv = ov; bs = os; }
    }
    const int bi = __shfl(p.arg, bs < kMaxSplits ? bs : 0, 64);
    if (ent.H) {
      // entropy and plain argmax of the row (exact ties: the lower split)
      const float S1 = wave_sum((s < splits && p.l > 0.f) ? w * (p.s1 + (p.m - M) * p.l) : 0.f);
      float dv = (s < splits && p.darg >= 0) ? p.dbest : -INFINITY;
      int ds = (s < splits && p.darg >= 0) ? s : kMaxSplits;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(dv, o, 64);
        const int os = __shfl_xor(ds, o, 64);
        if (ov > dv || (ov == dv && os < ds)) { dv = ov; ds = os; }
      }
      const int di = __shfl(p.darg, ds < kMaxSplits ? ds : 0, 64);
      if (s == 0) {
        inv_l = 1.f / L;
        if (blockIdx.y == 0) {
          ent.H[r] = 0.6931471805599453f * (log2f(L) - S1 / L);
          ent.y[r] = bs < kMaxSplits ? bi : -1;
          ent.det[r] = ds < kMaxSplits ? di : -1;
          if (lse) lse[r] = (M + log2f(L)) * 0.6931471805599453f;
          if (best) best[r] = bs < kMaxSplits ? bi : -1;
        }
      }
    } else if (s == 0) {
      inv_l = 1.f / L;
      if (blockIdx.y == 0) {
        const int b = r / C, i = r - b * C;
        const u32x4 u = philox4x32_10(0u, static_cast<uint32_t>(i), static_cast<uint32_t>(b),
                                      kStreamBernoulli, k0, k1);
        const bool rs = u01(u.x) < prm[b].lam;
        const int y = bs < kMaxSplits ? bi : -1;
        x_out[r] = rs ? y : x_t[r];
        if (lse) lse[r] = (M + log2f(L)) * 0.6931471805599453f;
        if (best) best[r] = rs ? y : -1;
      }
    }
  }
  __syncthreads();
  const float il = inv_l;
  const int c0 = (blockIdx.y * blockDim.x + threadIdx.x) * 4;
  if (c0 >= d) return;
  const int64_t rowoff = static_cast<int64_t>(r) * d;
  if (c0 + 4 <= d && (d & 3) == 0) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    const ZP *zp = zpart + rowoff + c0;
    const int64_t sstride = static_cast<int64_t>(R) * d;
#pragma unroll 8
    for (int s = 0; s < splits; ++s) {
      const float4 v = load4(zp + s * sstride);
      const float w = wsh[s];
      acc.x += w * v.x;
      acc.y += w * v.y;
      acc.z += w * v.z;
      acc.w += w * v.w;
    }
    Act<T>::store(z_out, rowoff + c0, acc.x * il);
    Act<T>::store(z_out, rowoff + c0 + 1, acc.y * il);
    Act<T>::store(z_out, rowoff + c0 + 2, acc.z * il);
    Act<T>::store(z_out, rowoff + c0 + 3, acc.w * il);
  } else {
    for (int c = c0; c < d && c < c0 + 4; ++c) {
      float acc = 0.f;
      for (int s = 0; s < splits; ++s)
        acc += wsh[s] * load1(zpart + (static_cast<int64_t>(s) * R + r) * d + c);
      Act<T>::store(z_out, rowoff + c, acc * il);
    }
  }
}

}  // namespace

hipError_t launch_combine(bool bf16, const void *work, int splits, const int32_t *x_t,
                          const StepParams *prm, const Shape &s, uint64_t seed, int32_t *x_out,
                          void *z_out, float *lse, int32_t *best, const EntropyRows *ent,
                          const int32_t *frozen, const void *z_t, hipStream_t st) {
  const int R = s.R();
  if (R == 0) return hipSuccess;
  if (splits < 1 || splits > kMaxSplits) return hipErrorInvalidValue;
  const RowPartial *part = static_cast<const RowPartial *>(work);
  const char *zbase = static_cast<const char *>(work) + static_cast<size_t>(splits) * R * sizeof(RowPartial);
  const uint32_t k0 = static_cast<uint32_t>(seed), k1 = static_cast<uint32_t>(seed >> 32);
  const dim3 grid(R, (s.d + 1023) / 1024);
  const EntropyRows er = ent ? *ent : EntropyRows{nullptr, nullptr, nullptr};
  if (frozen && !z_t) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL((combine_kernel<uint16_t, uint16_t>), grid, dim3(256), 0, st, part,
                       reinterpret_cast<const uint16_t *>(zbase), splits,
                       x_t, prm, R, s.C, s.d, k0, k1, x_out, static_cast<uint16_t *>(z_out), lse,
                       best, er, frozen, static_cast<const uint16_t *>(z_t));
  else
    hipLaunchKernelGGL((combine_kernel<float, float>), grid, dim3(256), 0, st, part,
                       reinterpret_cast<const float *>(zbase), splits, x_t,
                       prm, R, s.C, s.d, k0, k1, x_out, static_cast<float *>(z_out), lse, best,
                       er, frozen, static_cast<const float *>(z_t));
  return hipGetLastError();
}

}  // namespace dg
