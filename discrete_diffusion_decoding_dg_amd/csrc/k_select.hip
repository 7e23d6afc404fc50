// Entropy-bounded acceptance, uniform re-noise and the adaptive stop test.
//
// DiffusionGemma Technical Report (hyper.ai summary), Method, sampler
// paragraph (the recommended sampler): canvas positions are accepted in order
// of increasing entropy while the summed entropy of the accepted set (read as
// the bound on their mutual information) stays below eps_accept, and at least
// the lowest-entropy position; every other position is re-noised with a
// uniformly random token; a canvas stops once its mean entropy is below
// eps_stop and its argmax predictions repeat those of the previous step.
//
// One block per canvas, one thread per position (padded to a power of two):
// a bitonic sort of (entropy, position) in registers (cross-lane shuffles
// within a wave, LDS between waves), an inclusive scan of the sorted
// entropies, then every thread settles the position of its rank.
#include "dg_device.hpp"
#include "dg_kernels.hpp"

namespace dg {
namespace {

constexpr uint32_t kStreamRenoise = 3;

__device__ __forceinline__ bool key_less(float ha, int pa, float hb, int pb) {
  return ha < hb || (ha == hb && pa < pb);
}

__global__ void __launch_bounds__(1024) entropy_select_kernel(
    EntropyRows ent, const int32_t *__restrict__ x_t, const int32_t *__restrict__ det_prev, int C,
    int V, float eps_accept, float eps_stop, uint32_t k0, uint32_t k1, int step,
    int32_t *__restrict__ x_out, int32_t *__restrict__ det_out, float *__restrict__ entropy_out,
    int32_t *__restrict__ stop_out, int32_t *__restrict__ stopped, int32_t *__restrict__ steps_out) {
  __shared__ float key[kSelectMaxC];
  __shared__ int pos[kSelectMaxC];
  __shared__ float scan[kSelectMaxC];
  const int b = blockIdx.x, t = threadIdx.x, n = blockDim.x;   // n: a power of two >= C
  const int64_t base = static_cast<int64_t>(b) * C;
  if (stopped && stopped[b]) {
    // a stopped canvas keeps its tokens and predictions
    for (int i = t; i < C; i += n) {
      x_out[base + i] = x_t[base + i];
      det_out[base + i] = det_prev ? det_prev[base + i] : ent.det[base + i];
      if (entropy_out) entropy_out[base + i] = ent.H[base + i];
    }
    if (t == 0) stop_out[b] = 1;
    return;
  }
  const bool in = t < C;
  float kv = in ? ent.H[base + t] : INFINITY;
  int pv = in ? t : 0x7fffffff;
  if (in) {
    det_out[base + t] = ent.det[base + t];
    if (entropy_out) entropy_out[base + t] = ent.H[base + t];
  }
  // bitonic sort, ascending by (entropy, position): thread t ends holding
  // rank t. Partners less than 64 apart are in the same wave and trade
  // through cross-lane shuffles; farther ones through LDS (one barrier pair).
  for (int k = 2; k <= n; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      float kp;
      int pp;
      if (j >= 64) {
        key[t] = kv;
        pos[t] = pv;
        __syncthreads();
        kp = key[t ^ j];
        pp = pos[t ^ j];
        __syncthreads();
      } else {
        kp = __shfl_xor(kv, j, 64);
        pp = __shfl_xor(pv, j, 64);
      }
      // ascending runs (t & k == 0): the lower index of a pair keeps the
      // smaller key; descending runs the larger (keys are distinct)
      const bool up = (t & k) == 0, lower = (t & j) == 0;
      const bool p_less = key_less(kp, pp, kv, pv);
      if ((up == lower) ? p_less : !p_less) {
        kv = kp;
        pv = pp;
      }
    }
  // inclusive scan of the sorted entropies (padding sorts last): within each
  // wave by shuffles, then the totals of the earlier waves
  const int lane = t & 63, wv = t >> 6;
  float run = in ? kv : 0.f;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float add = __shfl_up(run, off, 64);
    if (lane >= off) run += add;
  }
  if (lane == 63) scan[wv] = run;
  __syncthreads();
  for (int w = 0; w < wv; ++w) run += scan[w];
  __syncthreads();
  scan[t] = run;   // the scan by rank, for the mean below
  __syncthreads();
  if (in) {
    const int i = pv;
    const bool accept = (t == 0) || (run < eps_accept);
    int32_t tok;
    if (accept) {
      tok = ent.y[base + i];
    } else {
      const u32x4 w = philox4x32_10(0u, static_cast<uint32_t>(i), static_cast<uint32_t>(b),
                                    kStreamRenoise, k0, k1);
      tok = static_cast<int32_t>((static_cast<uint64_t>(w.x) * static_cast<uint32_t>(V)) >> 32);
    }
    x_out[base + i] = tok;
  }
  const bool same = !in || !det_prev || ent.det[base + t] == det_prev[base + t];
  const int all_same = __syncthreads_and(same ? 1 : 0);
  if (t == 0) {
    const float mean = scan[C - 1] / static_cast<float>(C);
    const int stop = (det_prev && all_same && mean < eps_stop) ? 1 : 0;
    stop_out[b] = stop;
    if (stop && stopped) {
      stopped[b] = 1;
      if (steps_out) steps_out[b] = step + 1;
    }
  }
}

}  // namespace

hipError_t launch_entropy_select(const EntropyRows &ent, const int32_t *x_t,
                                 const int32_t *det_prev, int B, int C, int V, float eps_accept,
                                 float eps_stop, uint64_t seed, int step, int32_t *x_out,
                                 int32_t *det_out, float *entropy_out, int32_t *stop_out,
                                 int32_t *stopped, int32_t *steps_out, hipStream_t st) {
  if (B == 0) return hipSuccess;
  if (C < 1 || C > kSelectMaxC) return hipErrorInvalidValue;
  int n = 64;
  while (n < C) n <<= 1;
  hipLaunchKernelGGL(entropy_select_kernel, dim3(B), dim3(n), 0, st, ent, x_t, det_prev, C, V,
                     eps_accept, eps_stop, static_cast<uint32_t>(seed),
                     static_cast<uint32_t>(seed >> 32), step, x_out, det_out, entropy_out,
                     stop_out, stopped, steps_out);
  return hipGetLastError();
}

}  // namespace dg
