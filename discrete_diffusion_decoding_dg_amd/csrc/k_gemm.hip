// bf16 MFMA GEMMs of the decoder block: the fused q/k/v projection and the
// output projection with the residual add. Both are C = A B^T with A [M, K]
// and B [N, K] row-major (K contiguous in both, the layout MFMA operands want).
//
// Tiling: 64 x 64 output tile per 256-thread block (2 x 2 waves, 32 x 32 per
// wave via v_mfma_f32_32x32x16_bf16), K staged through LDS in 64-wide slabs,
// double-buffered: the next slab is fetched into registers while the current
// one feeds the matrix cores.
#include "dg_device.hpp"
#include "dg_kernels.hpp"

namespace dg {
namespace {

constexpr int BM = 64, BN = 64, BK = 64;
constexpr int PAD = 8;                  // bf16 elements of row padding in LDS
constexpr int LDW = BK + PAD;           // LDS row pitch (elements)

// Where row n of the virtual B matrix comes from, and where C goes.
struct QkvEpi {
  const uint16_t *Wq, *Wk, *Wv;
  uint16_t *q, *k, *v;
  int Nq, Nkv, C, Hkv, hd;
  __device__ const uint16_t *brow(int n, int K) const {
    if (n < Nq) return Wq + static_cast<int64_t>(n) * K;
    n -= Nq;
    if (n < Nkv) return Wk + static_cast<int64_t>(n) * K;
    return Wv + static_cast<int64_t>(n - Nkv) * K;
  }
  __device__ void store(int m, int n, float acc) const {
    const uint16_t val = f32_to_bf16(acc);
    if (n < Nq) {
      q[static_cast<int64_t>(m) * Nq + n] = val;
      return;
    }
    n -= Nq;
    uint16_t *dst = k;
    if (n >= Nkv) {
      n -= Nkv;
      dst = v;
    }
    // [B, Hkv, C, hd] layout: one kv head of one canvas is contiguous
    const int b = m / C, i = m - b * C;
    const int g = n / hd, e = n - g * hd;
    dst[((static_cast<int64_t>(b) * Hkv + g) * C + i) * hd + e] = val;
  }
};

struct ResidualEpi {
  const uint16_t *W;
  const uint16_t *res;
  uint16_t *out;
  int N;
  __device__ const uint16_t *brow(int n, int K) const { return W + static_cast<int64_t>(n) * K; }
  __device__ void store(int m, int n, float acc) const {
    const int64_t idx = static_cast<int64_t>(m) * N + n;
    out[idx] = f32_to_bf16(bf16_to_f32(res[idx]) + acc);
  }
};

template <class Epi>
__global__ void __launch_bounds__(256) gemm_tn_bf16_kernel(const uint16_t *__restrict__ A, int M,
                                                           int N, int K, Epi epi) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDW];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDW];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;

  // Global -> register staging: 2 chunks of 16 B per thread per operand.
  uint4 ra[2], rb[2];
  const uint16_t *arow[2];
  const uint16_t *brow[2];
  int srow[2], scol[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = tid + 256 * u;
    srow[u] = c >> 3;
    scol[u] = (c & 7) * 8;
    const int am = m0 + srow[u], bn = n0 + srow[u];
    arow[u] = am < M ? A + static_cast<int64_t>(am) * K : nullptr;
    brow[u] = bn < N ? epi.brow(bn, K) : nullptr;
  }
  auto fetch = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kk = k0 + scol[u];
      const bool kin = kk < K;  // K % 8 == 0: a chunk is all in or all out
      ra[u] = (arow[u] && kin) ? *reinterpret_cast<const uint4 *>(arow[u] + kk) : make_uint4(0, 0, 0, 0);
      rb[u] = (brow[u] && kin) ? *reinterpret_cast<const uint4 *>(brow[u] + kk) : make_uint4(0, 0, 0, 0);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      *reinterpret_cast<uint4 *>(&As[buf][srow[u] * LDW + scol[u]]) = ra[u];
      *reinterpret_cast<uint4 *>(&Bs[buf][srow[u] * LDW + scol[u]]) = rb[u];
    }
  };

  f32x16 acc = {};
  const int nk = (K + BK - 1) / BK;
  fetch(0);
  stash(0);
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    const int buf = it & 1;
    if (it + 1 < nk) fetch((it + 1) * BK);
    const uint16_t *a_base = &As[buf][(wm * 32 + (lane & 31)) * LDW + (lane >> 5) * 8];
    const uint16_t *b_base = &Bs[buf][(wn * 32 + (lane & 31)) * LDW + (lane >> 5) * 8];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8 *>(a_base + ks * 16);
      const bf16x8 b = *reinterpret_cast<const bf16x8 *>(b_base + ks * 16);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    }
    if (it + 1 < nk) {
      stash(buf ^ 1);
      __syncthreads();
    }
  }

  // C layout of the 32x32 MFMA: lane holds column (lane % 32) and rows
  // 8*j + 4*(lane / 32) + i in register 4*j + i.
  const int n = n0 + wn * 32 + (lane & 31);
  if (n < N) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * 32 + 8 * j + 4 * (lane >> 5) + i;
        if (m < M) epi.store(m, n, acc[4 * j + i]);
      }
  }
}

}  // namespace

hipError_t launch_qkv_bf16(const uint16_t *h0, const uint16_t *Wq, const uint16_t *Wk,
                           const uint16_t *Wv, const Shape &s, uint16_t *q, uint16_t *k,
                           uint16_t *v, hipStream_t st) {
  QkvEpi epi{Wq, Wk, Wv, q, k, v, s.Hq * s.hd, s.Hkv * s.hd, s.C, s.Hkv, s.hd};
  const int M = s.R(), N = s.Hq * s.hd + 2 * s.Hkv * s.hd;
  if (M == 0) return hipSuccess;
  dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
  hipLaunchKernelGGL(gemm_tn_bf16_kernel<QkvEpi>, grid, dim3(256), 0, st, h0, M, N, s.d, epi);
  return hipGetLastError();
}

hipError_t launch_oproj_bf16(const uint16_t *o, const uint16_t *Wo, const uint16_t *h0,
                             const Shape &s, uint16_t *h1, hipStream_t st) {
  ResidualEpi epi{Wo, h0, h1, s.d};
  const int M = s.R(), N = s.d, K = s.Hq * s.hd;
  if (M == 0) return hipSuccess;
  dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
  hipLaunchKernelGGL(gemm_tn_bf16_kernel<ResidualEpi>, grid, dim3(256), 0, st, o, M, N, K, epi);
  return hipGetLastError();
}

}  // namespace dg
