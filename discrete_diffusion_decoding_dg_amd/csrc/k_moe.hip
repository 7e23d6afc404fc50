// Mixture-of-experts MLP of the decoder stack: router logits and top-k
// choice, grouping of the routed (token, slot) entries by expert, and the
// weighted combine into the residual stream (the expert GEMMs themselves run
// in k_gemm.hip over the grouped entries, or below for fp32).
//
// Routing rule (a reading; the TR summary's model routes each token to a few
// experts without stating the rule): float32 logits r = m W_router^T; the
// top_k experts by logit, ties to the lower expert; weights = softmax over
// the selected logits.
#include "dg_device.hpp"
#include "dg_kernels.hpp"

namespace dg {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// One block per token row; 256 / XM threads per expert (XM >= X) take the
// row and the expert's router row in 16-byte pieces, reduce their partial
// dot products within the group, and thread 0 picks the top_k.
template <typename T>
__device__ __forceinline__ void load_piece(const T *p, float (&v)[16 / sizeof(T)]) {
  const uint4 q = *reinterpret_cast<const uint4 *>(p);
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

template <typename T, int XM>
__global__ void __launch_bounds__(256) router_topk_kernel(const T *__restrict__ m,
                                                          const T *__restrict__ Wr, int d, int X,
                                                          int top_k, int32_t *__restrict__ sel,
                                                          float *__restrict__ wts) {
  constexpr int VW = 16 / sizeof(T);               // elements per piece
  constexpr int TE = 256 / XM;                     // threads per expert (one wave or less)
  static_assert(TE >= 1 && TE <= 64 && 64 % TE == 0, "expert groups");
  __shared__ float logit[XM];
  const int r = blockIdx.x, tid = threadIdx.x;
  const int e = tid / TE, sub = tid - e * TE;      // expert and position in its group
  const T *mr = m + static_cast<int64_t>(r) * d;
  float acc = 0.f;
  if (e < X) {
    const T *we = Wr + static_cast<int64_t>(e) * d;
    for (int c = sub; c < d / VW; c += TE) {
      float mv[VW], wv[VW];
      load_piece<T>(mr + c * VW, mv);
      load_piece<T>(we + c * VW, wv);
#pragma unroll
      for (int i = 0; i < VW; ++i) acc = fmaf(mv[i], wv[i], acc);
    }
  }
#pragma unroll
  for (int o = 1; o < TE; o <<= 1) acc += __shfl_xor(acc, o, 64);
  if (sub == 0 && e < X) logit[e] = acc;
  __syncthreads();
  if (tid != 0) return;
  float lg[XM];
  for (int k = 0; k < X; ++k) lg[k] = logit[k];
  // selection by repeated maximum: strict comparison keeps the lower expert on ties
  uint64_t taken = 0;
  float top[XM];
  int idx[XM];
  for (int j = 0; j < top_k; ++j) {
    int best = -1;
    for (int x = 0; x < X; ++x)
      if (!((taken >> x) & 1) && (best < 0 || lg[x] > lg[best])) best = x;
    taken |= uint64_t(1) << best;
    idx[j] = best;
    top[j] = lg[best];
  }
  float den = 0.f;
  for (int j = 0; j < top_k; ++j) den += exp2f((top[j] - top[0]) * kLog2e);
  for (int j = 0; j < top_k; ++j) {
    sel[static_cast<int64_t>(r) * top_k + j] = idx[j];
    wts[static_cast<int64_t>(r) * top_k + j] = exp2f((top[j] - top[0]) * kLog2e) / den;
  }
}

// One block: for each expert in turn, a stable compaction of the entries
// routed to it (entry q = token * top_k + slot) into list, with entry offsets
// offs[X + 1] and 64-row tile offsets toff[X + 1].
__global__ void __launch_bounds__(1024) moe_group_kernel(const int32_t *__restrict__ sel, int n, int X,
                                                         int32_t *__restrict__ list,
                                                         int32_t *__restrict__ offs,
                                                         int32_t *__restrict__ toff) {
  __shared__ int wsum[16];
  __shared__ int base_sh, tile_sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (n + 1023) / 1024;               // contiguous entries per thread
  const int q0 = tid * per;
  if (tid == 0) {
    base_sh = 0;
    tile_sh = 0;
  }
  __syncthreads();
  for (int e = 0; e < X; ++e) {
    int cnt = 0;
    for (int i = 0; i < per; ++i) cnt += (q0 + i < n && sel[q0 + i] == e) ? 1 : 0;
    // exclusive scan of the per-thread counts
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int wbase = 0, total = 0;
    for (int w = 0; w < 16; ++w) {
      if (w < wave) wbase += wsum[w];
      total += wsum[w];
    }
    const int base = base_sh;
    int pos = base + wbase + incl - cnt;
    for (int i = 0; i < per; ++i)
      if (q0 + i < n && sel[q0 + i] == e) list[pos++] = q0 + i;
    __syncthreads();                                // everyone has read base_sh and wsum
    if (tid == 0) {
      offs[e] = base;
      toff[e] = tile_sh;
      base_sh = base + total;
      tile_sh += (total + kMoeTile - 1) / kMoeTile;
    }
    __syncthreads();
  }
  if (tid == 0) {
    offs[X] = base_sh;
    toff[X] = tile_sh;
  }
}

// The same grouping in one pass, for up to kGroupCells chunk x expert cells:
// entries are taken in chunks of 64 (a wave's lanes); per chunk and expert a
// ballot gives the count and each entry's rank among the chunk's entries of
// that expert; one exclusive scan over the (expert, chunk) counts in expert-
// major order gives every chunk's first position in the list.
constexpr int kGroupCells = 8192;
__global__ void __launch_bounds__(1024) moe_group_ballot_kernel(const int32_t *__restrict__ sel, int n,
                                                                int X, int32_t *__restrict__ list,
                                                                int32_t *__restrict__ offs,
                                                                int32_t *__restrict__ toff) {
  __shared__ int cell[kGroupCells];               // [X][chunks] counts, then exclusive prefixes
  __shared__ int tsum[1024];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = (n + 63) / 64, cells = X * nch;
  for (int c = wave; c < nch; c += 16) {
    const int q = c * 64 + lane;
    const int e_q = q < n ? sel[q] : -1;
    for (int e = 0; e < X; ++e) {
      const uint64_t bal = __builtin_amdgcn_ballot_w64(e_q == e);
      if (lane == 0) cell[e * nch + c] = __popcll(bal);
    }
  }
  __syncthreads();
  // exclusive scan of cell[0, cells): thread t owns a contiguous run
  const int per = (cells + 1023) / 1024;
  const int c0 = tid * per;
  int run = 0;
  for (int i = 0; i < per; ++i)
    if (c0 + i < cells) run += cell[c0 + i];
  tsum[tid] = run;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {             // inclusive scan of the run sums
    const int v = tid >= o ? tsum[tid - o] : 0;
    __syncthreads();
    tsum[tid] += v;
    __syncthreads();
  }
  int acc = tsum[tid] - run;
  for (int i = 0; i < per; ++i)
    if (c0 + i < cells) {
      const int v = cell[c0 + i];
      cell[c0 + i] = acc;
      acc += v;
    }
  __syncthreads();
  for (int c = wave; c < nch; c += 16) {
    const int q = c * 64 + lane;
    const int e_q = q < n ? sel[q] : -1;
    for (int e = 0; e < X; ++e) {
      const uint64_t bal = __builtin_amdgcn_ballot_w64(e_q == e);
      if (e_q == e) list[cell[e * nch + c] + __popcll(bal & ((uint64_t(1) << lane) - 1))] = q;
    }
  }
  if (tid == 0) {
    int tiles = 0;
    for (int e = 0; e < X; ++e) {
      const int b = cell[e * nch], end = (e + 1 < X) ? cell[(e + 1) * nch] : n;
      offs[e] = b;
      toff[e] = tiles;
      tiles += (end - b + kMoeTile - 1) / kMoeTile;
    }
    offs[X] = n;
    toff[X] = tiles;
  }
}

// out[r] = round(h[r] + sum_j wts[r, j] y[r * top_k + j]). Four columns per
// thread (16-byte loads of y) when d % 4 == 0.
template <typename T>
__global__ void __launch_bounds__(256) moe_combine_kernel(const T *__restrict__ h,
                                                          const float *__restrict__ y,
                                                          const float *__restrict__ wts, int d,
                                                          int top_k, T *__restrict__ out) {
  const int r = blockIdx.x;
  const int64_t row = static_cast<int64_t>(r) * d;
  if ((d & 3) == 0) {
    for (int c = 4 * threadIdx.x; c < d; c += 4 * blockDim.x) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < top_k; ++j) {
        const float w = wts[static_cast<int64_t>(r) * top_k + j];
        const float4 v = *reinterpret_cast<const float4 *>(y + (static_cast<int64_t>(r) * top_k + j) * d + c);
        acc[0] = fmaf(w, v.x, acc[0]);
        acc[1] = fmaf(w, v.y, acc[1]);
        acc[2] = fmaf(w, v.z, acc[2]);
        acc[3] = fmaf(w, v.w, acc[3]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) Act<T>::store(out, row + c + i, Act<T>::load(h, row + c + i) + acc[i]);
    }
    return;
  }
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    float acc = 0.f;
    for (int j = 0; j < top_k; ++j)
      acc = fmaf(wts[static_cast<int64_t>(r) * top_k + j],
                 y[(static_cast<int64_t>(r) * top_k + j) * d + c], acc);
    Act<T>::store(out, row + c, Act<T>::load(h, row + c) + acc);
  }
}

// fp32 experts, one thread per output: hid[q, f] for entry q of token q / top_k
__global__ void __launch_bounds__(256) moe_gate_up_f32_kernel(const float *__restrict__ m,
                                                              const int32_t *__restrict__ sel,
                                                              const float *__restrict__ Wg,
                                                              const float *__restrict__ Wu, int n,
                                                              int top_k, int d, int F,
                                                              float *__restrict__ hid) {
  const int64_t total = static_cast<int64_t>(n) * F;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int q = static_cast<int>(idx / F), f = static_cast<int>(idx - static_cast<int64_t>(q) * F);
    const int e = sel[q];
    const float *x = m + static_cast<int64_t>(q / top_k) * d;
    const float *wg = Wg + (static_cast<int64_t>(e) * F + f) * d;
    const float *wu = Wu + (static_cast<int64_t>(e) * F + f) * d;
    float g = 0.f, u = 0.f;
    for (int c = 0; c < d; ++c) {
      g = fmaf(x[c], wg[c], g);
      u = fmaf(x[c], wu[c], u);
    }
    hid[idx] = gelu_tanh(g) * u;
  }
}

__global__ void __launch_bounds__(256) moe_down_f32_kernel(const float *__restrict__ hid,
                                                           const int32_t *__restrict__ sel,
                                                           const float *__restrict__ Wd, int n,
                                                           int d, int F, float *__restrict__ y) {
  const int64_t total = static_cast<int64_t>(n) * d;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int q = static_cast<int>(idx / d), c = static_cast<int>(idx - static_cast<int64_t>(q) * d);
    const float *x = hid + static_cast<int64_t>(q) * F;
    const float *w = Wd + (static_cast<int64_t>(sel[q]) * d + c) * F;
    float acc = 0.f;
    for (int f = 0; f < F; ++f) acc = fmaf(x[f], w[f], acc);
    y[idx] = acc;
  }
}

int grid_of(int64_t total) {
  int64_t blocks = (total + 255) / 256;
  return static_cast<int>(blocks > 16384 ? 16384 : (blocks < 1 ? 1 : blocks));
}

}  // namespace

hipError_t launch_moe_route(bool bf16, const void *m, const void *Wr, int R, int d, int X, int top_k,
                            int32_t *sel, float *wts, int32_t *list, int32_t *offs, int32_t *toff,
                            hipStream_t st) {
  if (R == 0) return hipSuccess;
  if (X < 1 || X > kMoeMaxExperts || top_k < 1 || top_k > X) return hipErrorInvalidValue;
  // the row is read in 16-byte pieces
  if (d % (bf16 ? 8 : 4) != 0) return hipErrorInvalidValue;
#define DG_ROUTE(T_, XM_)                                                                          \
  hipLaunchKernelGGL((router_topk_kernel<T_, XM_>), dim3(R), dim3(256), 0, st, static_cast<const T_ *>(m), \
                     static_cast<const T_ *>(Wr), d, X, top_k, sel, wts)
  if (bf16) {
    if (X <= 8) DG_ROUTE(uint16_t, 8);
    else if (X <= 16) DG_ROUTE(uint16_t, 16);
    else DG_ROUTE(uint16_t, kMoeMaxExperts);
  } else {
    if (X <= 8) DG_ROUTE(float, 8);
    else if (X <= 16) DG_ROUTE(float, 16);
    else DG_ROUTE(float, kMoeMaxExperts);
  }
#undef DG_ROUTE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !list) return e;
  const int n = R * top_k;
  if (static_cast<int64_t>(X) * ((n + 63) / 64) <= kGroupCells)
    hipLaunchKernelGGL(moe_group_ballot_kernel, dim3(1), dim3(1024), 0, st, sel, n, X, list, offs, toff);
  else
    hipLaunchKernelGGL(moe_group_kernel, dim3(1), dim3(1024), 0, st, sel, n, X, list, offs, toff);
  return hipGetLastError();
}

hipError_t launch_moe_combine(bool bf16, const void *h, const float *y, const float *wts, int R, int d,
                              int top_k, void *out, hipStream_t st) {
  if (R == 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(moe_combine_kernel<uint16_t>, dim3(R), dim3(256), 0, st,
                       static_cast<const uint16_t *>(h), y, wts, d, top_k, static_cast<uint16_t *>(out));
  else
    hipLaunchKernelGGL(moe_combine_kernel<float>, dim3(R), dim3(256), 0, st, static_cast<const float *>(h),
                       y, wts, d, top_k, static_cast<float *>(out));
  return hipGetLastError();
}

hipError_t launch_moe_experts_f32(const float *m, const int32_t *sel, const float *Wg, const float *Wu,
                                  const float *Wd, int n, int top_k, int d, int F, float *hid, float *y,
                                  hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(moe_gate_up_f32_kernel, dim3(grid_of(static_cast<int64_t>(n) * F)), dim3(256), 0, st,
                     m, sel, Wg, Wu, n, top_k, d, F, hid);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(moe_down_f32_kernel, dim3(grid_of(static_cast<int64_t>(n) * d)), dim3(256), 0, st, hid,
                     sel, Wd, n, d, F, y);
  return hipGetLastError();
}

}  // namespace dg
