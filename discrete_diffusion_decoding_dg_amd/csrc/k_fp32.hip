// fp32 path of the decoder stand-in: plain VALU kernels for any shape, used
// when the model stores weights and activations in fp32 (the tiny fp32
// workload). Same math and rounding points as the bf16 path, fp32 storage.
// DiffusionGemma Technical Report (hyper.ai summary), Method: decoder
// equation and three-line update.
#include "dg_device.hpp"
#include "dg_kernels.hpp"

namespace dg {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// q, k, v = h0 W^T; one thread per output element.
__global__ void __launch_bounds__(256) qkv_f32_kernel(const float *__restrict__ h0,
                                                      const float *__restrict__ Wq,
                                                      const float *__restrict__ Wk,
                                                      const float *__restrict__ Wv, int R, int C,
                                                      int d, int Nq, int Nkv, int Hkv, int hd,
                                                      float *__restrict__ q, float *__restrict__ k,
                                                      float *__restrict__ v) {
  const int N = Nq + 2 * Nkv;
  const int64_t total = static_cast<int64_t>(R) * N;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int m = static_cast<int>(idx / N);
    int n = static_cast<int>(idx - static_cast<int64_t>(m) * N);
    const float *w;
    float *dst;
    int64_t off;
    const int b = m / C, i = m - b * C;
    if (n < Nq) {
      w = Wq + static_cast<int64_t>(n) * d;
      dst = q;
      off = static_cast<int64_t>(m) * Nq + n;
    } else {
      n -= Nq;
      dst = k;
      const float *W = Wk;
      if (n >= Nkv) { n -= Nkv; dst = v; W = Wv; }
      w = W + static_cast<int64_t>(n) * d;
      const int g = n / hd, e = n - g * hd;
      off = ((static_cast<int64_t>(b) * Hkv + g) * C + i) * hd + e;
    }
    const float *x = h0 + static_cast<int64_t>(m) * d;
    float acc = 0.f;
    for (int c = 0; c < d; ++c) acc = fmaf(x[c], w[c], acc);
    dst[off] = acc;
  }
}

// One block per (row, head): scores over all P + C keys in LDS, then O.
// causal: canvas query i sees canvas keys 0..i only (the encoder pass).
__global__ void __launch_bounds__(256) attn_f32_kernel(const float *__restrict__ q,
                                                       const float *__restrict__ k,
                                                       const float *__restrict__ v,
                                                       const float *__restrict__ Kp,
                                                       const float *__restrict__ Vp, int C, int P,
                                                       int Pst, int Hq, int Hkv, int hd, float scale,
                                                       int causal, float *__restrict__ o) {
  extern __shared__ float sc[];   // P + C scores
  __shared__ float red[256];
  const int r = blockIdx.x, h = blockIdx.y;
  const int b = r / C;
  const int g = h / (Hq / Hkv);
  const int Lk = causal ? P + (r - b * C) + 1 : P + C;
  const float *qr = q + (static_cast<int64_t>(r) * Hq + h) * hd;
  const float *kp = Kp + (static_cast<int64_t>(b) * Hkv + g) * Pst * hd;
  const float *vp = Vp + (static_cast<int64_t>(b) * Hkv + g) * Pst * hd;
  const float *kc = k + (static_cast<int64_t>(b) * Hkv + g) * C * hd;
  const float *vc = v + (static_cast<int64_t>(b) * Hkv + g) * C * hd;
  float mx = -INFINITY;
  for (int j = threadIdx.x; j < Lk; j += blockDim.x) {
    const float *kr = j < P ? kp + static_cast<int64_t>(j) * hd : kc + static_cast<int64_t>(j - P) * hd;
    float acc = 0.f;
    for (int e = 0; e < hd; ++e) acc = fmaf(qr[e], kr[e], acc);
    acc *= scale * kLog2e;
    sc[j] = acc;
    mx = fmaxf(mx, acc);
  }
  red[threadIdx.x] = mx;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  mx = red[0];
  __syncthreads();
  float sum = 0.f;
  for (int j = threadIdx.x; j < Lk; j += blockDim.x) {
    const float p = exp2f(sc[j] - mx);
    sc[j] = p;
    sum += p;
  }
  red[threadIdx.x] = sum;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  const float inv = 1.f / red[0];
  for (int e = threadIdx.x; e < hd; e += blockDim.x) {
    float acc = 0.f;
    for (int j = 0; j < Lk; ++j) {
      const float *vr = j < P ? vp + static_cast<int64_t>(j) * hd : vc + static_cast<int64_t>(j - P) * hd;
      acc = fmaf(sc[j], vr[e], acc);
    }
    o[(static_cast<int64_t>(r) * Hq + h) * hd + e] = acc * inv;
  }
}

// h1 = h0 + o Wo^T.
__global__ void __launch_bounds__(256) oproj_f32_kernel(const float *__restrict__ o,
                                                        const float *__restrict__ Wo,
                                                        const float *__restrict__ h0, int R,
                                                        int d, int K, float *__restrict__ h1) {
  const int64_t total = static_cast<int64_t>(R) * d;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int m = static_cast<int>(idx / d), n = static_cast<int>(idx - static_cast<int64_t>(m) * d);
    const float *x = o + static_cast<int64_t>(m) * K;
    const float *w = Wo + static_cast<int64_t>(n) * K;
    float acc = 0.f;
    for (int c = 0; c < K; ++c) acc = fmaf(x[c], w[c], acc);
    h1[idx] = h0[idx] + acc;
  }
}

// Encoder cache entries: row m = b * n + i embeds token x[b * ld + i] (zero
// row when out of range) and its k (v) projection goes to row pos + i of the
// (b, kv head) slice of K (V) [B, Hkv, Pst, hd].
__global__ void __launch_bounds__(256) kv_encode_f32_kernel(const float *__restrict__ E,
                                                            const int32_t *__restrict__ x, int ld,
                                                            const float *__restrict__ Wk,
                                                            const float *__restrict__ Wv, int B,
                                                            int n, int d, int V, int Hkv, int hd,
                                                            int pos, int Pst, float *__restrict__ K,
                                                            float *__restrict__ Vc) {
  const int Nkv = Hkv * hd;
  const int64_t total = static_cast<int64_t>(B) * n * 2 * Nkv;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int m = static_cast<int>(idx / (2 * Nkv));
    int c = static_cast<int>(idx - static_cast<int64_t>(m) * 2 * Nkv);
    const bool is_v = c >= Nkv;
    if (is_v) c -= Nkv;
    const int b = m / n, i = m - b * n;
    const int32_t tok = x[static_cast<int64_t>(b) * ld + i];
    const int g = c / hd, e = c - g * hd;
    float acc = 0.f;
    if (tok >= 0 && tok < V) {
      const float *er = E + static_cast<int64_t>(tok) * d;
      const float *w = (is_v ? Wv : Wk) + static_cast<int64_t>(c) * d;
      for (int t = 0; t < d; ++t) acc = fmaf(er[t], w[t], acc);
    }
    (is_v ? Vc : K)[((static_cast<int64_t>(b) * Hkv + g) * Pst + pos + i) * hd + e] = acc;
  }
}

// Gated self-conditioning block: hid[m, f] = gelu(u_m . Wg_f) * (u_m . Wu_f).
__global__ void __launch_bounds__(256) ffw_gate_up_f32_kernel(const float *__restrict__ u,
                                                              const float *__restrict__ Wg,
                                                              const float *__restrict__ Wu, int R,
                                                              int d, int F, float *__restrict__ hid) {
  const int64_t total = static_cast<int64_t>(R) * F;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int m = static_cast<int>(idx / F), f = static_cast<int>(idx - static_cast<int64_t>(m) * F);
    const float *x = u + static_cast<int64_t>(m) * d;
    const float *wg = Wg + static_cast<int64_t>(f) * d;
    const float *wu = Wu + static_cast<int64_t>(f) * d;
    float g = 0.f, v = 0.f;
    for (int c = 0; c < d; ++c) {
      g = fmaf(x[c], wg[c], g);
      v = fmaf(x[c], wu[c], v);
    }
    hid[idx] = gelu_tanh(g) * v;
  }
}

// z[m, n] = res[m, n] + hid_m . Wd_n (res nullable: 0); rows of canvases
// marked in `frozen` copy z_t.
__global__ void __launch_bounds__(256) ffw_down_f32_kernel(const float *__restrict__ hid,
                                                           const float *__restrict__ Wd, int R, int d,
                                                           int F, int C,
                                                           const int32_t *__restrict__ frozen,
                                                           const float *__restrict__ zt,
                                                           const float *__restrict__ res,
                                                           float *__restrict__ z) {
  const int64_t total = static_cast<int64_t>(R) * d;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int m = static_cast<int>(idx / d), n = static_cast<int>(idx - static_cast<int64_t>(m) * d);
    if (frozen && frozen[m / C]) {
      z[idx] = zt[idx];
      continue;
    }
    const float *x = hid + static_cast<int64_t>(m) * F;
    const float *w = Wd + static_cast<int64_t>(n) * F;
    float acc = 0.f;
    for (int c = 0; c < F; ++c) acc = fmaf(x[c], w[c], acc);
    z[idx] = res ? res[idx] + acc : acc;
  }
}

// LM head for one row per block, vocabulary in chunks of 256: scaled logits,
// online max / sum (log2 units, rescaled every chunk), Gumbel argmax for a
// resampling row, z accumulated by the threads that own its columns.
constexpr int kZPerThread = 16;   // d <= 256 * 16
__global__ void __launch_bounds__(256) lmhead_f32_kernel(const float *__restrict__ h1,
                                                         const float *__restrict__ E,
                                                         const StepParams *__restrict__ prm,
                                                         int R, int C, int d, int V, uint32_t k0,
                                                         uint32_t k1, RowPartial *__restrict__ part,
                                                         float *__restrict__ zpart,
                                                         float *__restrict__ p0, int ent) {
  __shared__ float pch[256];
  __shared__ float redv[256];
  __shared__ int redi[256];
  __shared__ float reds[256];
  __shared__ float hrow[4096];
  const int r = blockIdx.x, t = threadIdx.x;
  const int b = r / C, i = r - b * C;
  const float inv_tau = prm[b].inv_tau;
  const u32x4 bw = philox4x32_10(0u, static_cast<uint32_t>(i), static_cast<uint32_t>(b),
                                 kStreamBernoulli, k0, k1);
  // the entropy-bounded step draws for every row
  const bool rs = ent ? true : u01(bw.x) < prm[b].lam;
  for (int c = t; c < d; c += 256) hrow[c] = h1[static_cast<int64_t>(r) * d + c];
  __syncthreads();
  float z[kZPerThread];
#pragma unroll
  for (int j = 0; j < kZPerThread; ++j) z[j] = 0.f;
  float m_run = -INFINITY, l_run = 0.f, bv = -INFINITY;
  int bi = -1;
  float s1_run = 0.f, dv = -INFINITY;   // entropy statistics: sum p (t - m) and the plain argmax
  int di = -1;
  for (int v0 = 0; v0 < V; v0 += 256) {
    const int v = v0 + t;
    float s2 = -INFINITY;
    if (v < V) {
      const float *er = E + static_cast<int64_t>(v) * d;
      float acc = 0.f;
      for (int c = 0; c < d; ++c) acc = fmaf(hrow[c], er[c], acc);
      const float s = acc * inv_tau;
      if (p0) p0[static_cast<int64_t>(r) * V + v] = s;
      if (rs) {
        const u32x4 w = philox4x32_10(gumbel_block_of(v), static_cast<uint32_t>(i),
                                      static_cast<uint32_t>(b), kStreamGumbel, k0, k1);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        const float pv = s + gumbel(ws[gumbel_word_of(v)]);
        if (pv > bv) { bv = pv; bi = v; }
      }
      s2 = s * kLog2e;
      if (s2 > dv) { dv = s2; di = v; }
    }
    redv[t] = s2;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (t < s) redv[t] = fmaxf(redv[t], redv[t + s]);
      __syncthreads();
    }
    const float m_new = fmaxf(m_run, redv[0]);
    const float sc = exp2f(m_run - m_new);
    __syncthreads();
    const float p = (v < V) ? exp2f(s2 - m_new) : 0.f;
    pch[t] = p;
    redv[t] = p;
    reds[t] = (v < V) ? p * (s2 - m_new) : 0.f;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (t < s) {
        redv[t] += redv[t + s];
        reds[t] += reds[t + s];
      }
      __syncthreads();
    }
    // re-reference the running sums to m_new, then add this chunk
    s1_run = (l_run > 0.f) ? sc * (s1_run + (m_run - m_new) * l_run) + reds[0] : reds[0];
    l_run = l_run * sc + redv[0];
    m_run = m_new;
    const int nv = (V - v0 < 256) ? V - v0 : 256;
#pragma unroll
    for (int j = 0; j < kZPerThread; ++j) {
      const int c = t + 256 * j;
      if (c < d) {
        float acc = z[j] * sc;
        for (int u = 0; u < nv; ++u) acc = fmaf(pch[u], E[static_cast<int64_t>(v0 + u) * d + c], acc);
        z[j] = acc;
      }
    }
    __syncthreads();
  }
  // block argmax of the Gumbel-perturbed logits, lowest id on ties
  redv[t] = bv;
  redi[t] = bi;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) {
      const float ov = redv[t + s];
      const int oi = redi[t + s];
      if (ov > redv[t] || (ov == redv[t] && oi >= 0 && (redi[t] < 0 || oi < redi[t]))) {
        redv[t] = ov;
        redi[t] = oi;
      }
    }
    __syncthreads();
  }
  const float gbest = redv[0];
  const int garg = redi[0];
  __syncthreads();
  // block argmax of the plain scaled logits, lowest id on ties
  redv[t] = dv;
  redi[t] = di;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) {
      const float ov = redv[t + s];
      const int oi = redi[t + s];
      if (ov > redv[t] || (ov == redv[t] && oi >= 0 && (redi[t] < 0 || oi < redi[t]))) {
        redv[t] = ov;
        redi[t] = oi;
      }
    }
    __syncthreads();
  }
  if (t == 0) {
    RowPartial p;
    p.m = m_run;
    p.l = l_run;
    p.best = gbest;
    p.arg = garg;
    p.s1 = s1_run;
    p.dbest = redv[0];
    p.darg = redi[0];
    p.pad = 0;
    part[r] = p;
  }
#pragma unroll
  for (int j = 0; j < kZPerThread; ++j) {
    const int c = t + 256 * j;
    if (c < d) zpart[static_cast<int64_t>(r) * d + c] = z[j];
  }
}

}  // namespace

hipError_t launch_qkv_f32(const float *h0, const float *Wq, const float *Wk, const float *Wv,
                          const Shape &s, float *q, float *k, float *v, hipStream_t st) {
  const int64_t total = static_cast<int64_t>(s.R()) * (s.Hq + 2 * s.Hkv) * s.hd;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(qkv_f32_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st, h0,
                     Wq, Wk, Wv, s.R(), s.C, s.d, s.Hq * s.hd, s.Hkv * s.hd, s.Hkv, s.hd, q, k, v);
  return hipGetLastError();
}

hipError_t launch_attention_f32(const float *q, const float *k, const float *v, const float *Kp,
                                const float *Vp, const Shape &s, float *o, hipStream_t st) {
  if (s.R() == 0) return hipSuccess;
  const size_t shm = static_cast<size_t>(s.P + s.C) * sizeof(float);
  hipLaunchKernelGGL(attn_f32_kernel, dim3(s.R(), s.Hq), dim3(256), shm, st, q, k, v, Kp, Vp,
                     s.C, s.P, s.pstride(), s.Hq, s.Hkv, s.hd,
                     static_cast<float>(1.0 / sqrt((double)s.hd)), s.causal, o);
  return hipGetLastError();
}

hipError_t launch_oproj_f32(const float *o, const float *Wo, const float *h0, const Shape &s,
                            float *h1, hipStream_t st) {
  const int64_t total = static_cast<int64_t>(s.R()) * s.d;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(oproj_f32_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st, o,
                     Wo, h0, s.R(), s.d, s.Hq * s.hd, h1);
  return hipGetLastError();
}

hipError_t launch_kv_encode_f32(const float *E, const int32_t *x, int ld, const float *Wk,
                                const float *Wv, const Shape &s, int n, int pos, int Pst, float *K,
                                float *V, hipStream_t st) {
  const int64_t total = static_cast<int64_t>(s.B) * n * 2 * s.Hkv * s.hd;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(kv_encode_f32_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st, E,
                     x, ld, Wk, Wv, s.B, n, s.d, s.V, s.Hkv, s.hd, pos, Pst, K, V);
  return hipGetLastError();
}

hipError_t launch_ffw_gate_up_f32(const float *u, const float *Wg, const float *Wu, int M, int d,
                                  int F, float *hid, hipStream_t st) {
  const int64_t total = static_cast<int64_t>(M) * F;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(ffw_gate_up_f32_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st, u,
                     Wg, Wu, M, d, F, hid);
  return hipGetLastError();
}

hipError_t launch_ffw_down_f32(const float *hid, const float *Wd, int M, int d, int F, int C,
                               const int32_t *frozen, const float *z_t, float *z, hipStream_t st,
                               const float *res) {
  const int64_t total = static_cast<int64_t>(M) * d;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(ffw_down_f32_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st, hid,
                     Wd, M, d, F, C, frozen, z_t, res, z);
  return hipGetLastError();
}

size_t lmhead_f32_workspace_bytes(const Shape &s) {
  const size_t R = static_cast<size_t>(s.R());
  return R * (sizeof(RowPartial) + static_cast<size_t>(s.d) * sizeof(float));
}

hipError_t launch_lmhead_f32(const float *h1, const float *E, const StepParams *prm,
                             const Shape &s, uint64_t seed, void *work, float *p0, bool entropy,
                             hipStream_t st) {
  if (s.R() == 0) return hipSuccess;
  RowPartial *part = static_cast<RowPartial *>(work);
  float *zpart = reinterpret_cast<float *>(static_cast<char *>(work) + static_cast<size_t>(s.R()) * sizeof(RowPartial));
  hipLaunchKernelGGL(lmhead_f32_kernel, dim3(s.R()), dim3(256), 0, st, h1, E, prm, s.R(), s.C,
                     s.d, s.V, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32),
                     part, zpart, p0, entropy ? 1 : 0);
  return hipGetLastError();
}

}  // namespace dg
