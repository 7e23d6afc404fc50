// Merge of the vocabulary-split partials and the Step select.
//
// DiffusionGemma Technical Report (hyper.ai summary), Method, three-line
// update. Per row: lse = logsumexp of the scaled logits, z = p0 E from the
// unnormalised split sums, and the Step draw (our Euler reading of Step):
// keep x_t unless the row's Bernoulli u < lambda_b, in which case take the
// Gumbel argmax over the whole vocabulary (ties: lowest id, i.e. the lowest
// split wins an exact tie between splits).
#include "dg_device.hpp"
#include "dg_kernels.hpp"

namespace dg {
namespace {

template <typename T>
__global__ void __launch_bounds__(256) combine_kernel(const RowPartial *__restrict__ part,
                                                      const float *__restrict__ zpart, int splits,
                                                      const int32_t *__restrict__ x_t,
                                                      const StepParams *__restrict__ prm, int R,
                                                      int C, int d, uint32_t k0, uint32_t k1,
                                                      int32_t *__restrict__ x_out,
                                                      T *__restrict__ z_out,
                                                      float *__restrict__ lse,
                                                      int32_t *__restrict__ best) {
  __shared__ float wsh[64];
  __shared__ float inv_l;
  const int r = blockIdx.x;
  if (splits > 64) return;  // the host never plans more than 64 splits
  if (threadIdx.x == 0) {
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, part[static_cast<int64_t>(s) * R + r].m);
    float L = 0.f, bv = -INFINITY;
    int bi = -1;
    for (int s = 0; s < splits; ++s) {
      const RowPartial p = part[static_cast<int64_t>(s) * R + r];
      const float w = exp2f(p.m - M);
      wsh[s] = w;
      L += w * p.l;
      if (p.arg >= 0 && p.best > bv) { bv = p.best; bi = p.arg; }
    }
    inv_l = 1.f / L;
    const int b = r / C, i = r - b * C;
    const u32x4 w = philox4x32_10(0u, static_cast<uint32_t>(i), static_cast<uint32_t>(b),
                                  kStreamBernoulli, k0, k1);
    const bool rs = u01(w.x) < prm[b].lam;
    x_out[r] = rs ? bi : x_t[r];
    if (lse) lse[r] = (M + log2f(L)) * 0.6931471805599453f;
    if (best) best[r] = rs ? bi : -1;
  }
  __syncthreads();
  const float il = inv_l;
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < splits; ++s)
      acc += wsh[s] * zpart[(static_cast<int64_t>(s) * R + r) * d + c];
    Act<T>::store(z_out, static_cast<int64_t>(r) * d + c, acc * il);
  }
}

}  // namespace

hipError_t launch_combine(bool bf16, const void *work, int splits, const int32_t *x_t,
                          const StepParams *prm, const Shape &s, uint64_t seed, int32_t *x_out,
                          void *z_out, float *lse, int32_t *best, hipStream_t st) {
  const int R = s.R();
  if (R == 0) return hipSuccess;
  if (splits < 1 || splits > 64) return hipErrorInvalidValue;
  const RowPartial *part = static_cast<const RowPartial *>(work);
  const float *zpart = reinterpret_cast<const float *>(static_cast<const char *>(work) +
                                                       static_cast<size_t>(splits) * R * sizeof(RowPartial));
  const uint32_t k0 = static_cast<uint32_t>(seed), k1 = static_cast<uint32_t>(seed >> 32);
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<uint16_t>, dim3(R), dim3(256), 0, st, part, zpart, splits,
                       x_t, prm, R, s.C, s.d, k0, k1, x_out, static_cast<uint16_t *>(z_out), lse,
                       best);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3(R), dim3(256), 0, st, part, zpart, splits, x_t,
                       prm, R, s.C, s.d, k0, k1, x_out, static_cast<float *>(z_out), lse, best);
  return hipGetLastError();
}

}  // namespace dg
