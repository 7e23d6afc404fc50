// bf16 MFMA GEMMs of the decoder block: the fused q/k/v projection, the
// output projection with the residual add, and the two halves of the gated
// self-conditioning block (gate and up projections with the GELU product;
// down projection). All are C = A B^T with A [M, K] and B [N, K] row-major
// (K contiguous in both, the layout MFMA operands want).
//
// Kernels, by row count (all v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   - rows >= 2048 (batched canvases): 256 x 256 tiles, K in 32-wide slabs
//     through four LDS stages (big::);
//   - fewer rows with K % 128 == 0: 64 x 64 or 64 x 32 tiles, K in 128-wide
//     slabs, the eight waves splitting K (skinny::), or 128 x 64 tiles for
//     wide outputs (two row halves of four waves splitting K);
//   - K % 64 == 0 otherwise: 64 x 64 tiles, 64-wide slabs, nine stages;
//   - anything else: 64 x 64 tiles, register double buffering.
// Operand slabs reach LDS through direct global->LDS loads except in the
// last kernel.
#include "dg_device.hpp"
#include "dg_kernels.hpp"

namespace dg {
namespace {

constexpr int BM = 64, BN = 64, BK = 64;
constexpr int PAD = 8;                  // bf16 elements of row padding in LDS
constexpr int LDW = BK + PAD;           // LDS row pitch (elements)

// Eight fp32 values rounded to bf16 and packed for one 16-byte store.
__device__ __forceinline__ uint4 pack8(const float (&a)[8]) {
  return make_uint4(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(a[4], a[5]),
                    pack_bf16x2(a[6], a[7]));
}
__device__ __forceinline__ bool aligned16(const void *p) {
  return (reinterpret_cast<uintptr_t>(p) & 15) == 0;
}

// Where row n of the virtual B matrix comes from, and where C goes.
// kPair: the tile's output columns come in gate/up pairs (see GegluEpi) and
// are stored through store_pair(m, n, gate, up) instead of store(m, n, acc).
// kVec8: store8(m, n, a) writes columns n .. n + 7 (n % 8 == 0) of row m as
// one 16-byte access with the same rounding as store(), whenever vec8_ok()
// (every column group of 8 then stays within one destination row segment).
struct QkvEpi {
  static constexpr bool kPair = false;
  static constexpr bool kVec8 = true;
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
  __device__ bool vec8_ok() const {
    return ((Nq | Nkv | hd) & 7) == 0 && aligned16(q) && aligned16(k) && aligned16(v);
  }
  __device__ void store8(int m, int n, const float (&a)[8]) const {
    const uint4 val = pack8(a);
    if (n < Nq) {
      *reinterpret_cast<uint4 *>(q + static_cast<int64_t>(m) * Nq + n) = val;
      return;
    }
    n -= Nq;
    uint16_t *dst = k;
    if (n >= Nkv) {
      n -= Nkv;
      dst = v;
    }
    const int b = m / C, i = m - b * C;
    const int g = n / hd, e = n - g * hd;
    *reinterpret_cast<uint4 *>(dst + ((static_cast<int64_t>(b) * Hkv + g) * C + i) * hd + e) = val;
  }
};

struct ResidualEpi {
  static constexpr bool kPair = false;
  static constexpr bool kVec8 = true;
  const uint16_t *W;
  const uint16_t *res;
  uint16_t *out;
  int N;
  __device__ const uint16_t *brow(int n, int K) const { return W + static_cast<int64_t>(n) * K; }
  __device__ void store(int m, int n, float acc) const {
    const int64_t idx = static_cast<int64_t>(m) * N + n;
    out[idx] = f32_to_bf16(bf16_to_f32(res[idx]) + acc);
  }
  __device__ bool vec8_ok() const { return (N & 7) == 0 && aligned16(res) && aligned16(out); }
  __device__ void store8(int m, int n, const float (&a)[8]) const {
    const int64_t idx = static_cast<int64_t>(m) * N + n;
    const uint4 r = *reinterpret_cast<const uint4 *>(res + idx);
    const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
    float o[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = bf16_to_f32(static_cast<uint16_t>(rw[i] & 0xFFFFu)) + a[2 * i];
      o[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(rw[i] >> 16)) + a[2 * i + 1];
    }
    *reinterpret_cast<uint4 *>(out + idx) = pack8(o);
  }
};

// Encoder cache entries: rows m = b * n + i of the token embeddings, columns
// [0, Nkv) the k projection and [Nkv, 2 Nkv) the v projection; results go to
// row pos + i of the (b, kv head) slices of the caches [B, Hkv, Pst, hd].
struct KvCacheEpi {
  static constexpr bool kPair = false;
  static constexpr bool kVec8 = true;
  const uint16_t *Wk, *Wv;
  uint16_t *K, *V;
  int Nkv, n, pos, Pst, Hkv, hd;
  __device__ const uint16_t *brow(int c, int Kd) const {
    return (c < Nkv ? Wk + static_cast<int64_t>(c) * Kd : Wv + static_cast<int64_t>(c - Nkv) * Kd);
  }
  __device__ void store(int m, int c, float acc) const {
    uint16_t *dst = K;
    if (c >= Nkv) {
      c -= Nkv;
      dst = V;
    }
    const int b = m / n, i = m - b * n;
    const int g = c / hd, e = c - g * hd;
    dst[((static_cast<int64_t>(b) * Hkv + g) * Pst + pos + i) * hd + e] = f32_to_bf16(acc);
  }
  __device__ bool vec8_ok() const { return ((Nkv | hd) & 7) == 0 && aligned16(K) && aligned16(V); }
  __device__ void store8(int m, int c, const float (&a)[8]) const {
    uint16_t *dst = K;
    if (c >= Nkv) {
      c -= Nkv;
      dst = V;
    }
    const int b = m / n, i = m - b * n;
    const int g = c / hd, e = c - g * hd;
    *reinterpret_cast<uint4 *>(dst + ((static_cast<int64_t>(b) * Hkv + g) * Pst + pos + i) * hd + e) = pack8(a);
  }
};

// Plain fp32 store of C = A B^T [M, N] (expert down projections).
struct F32StoreEpi {
  static constexpr bool kPair = false;
  static constexpr bool kVec8 = false;
  const uint16_t *W;
  float *out;
  int N;
  __device__ const uint16_t *brow(int n, int K) const { return W + static_cast<int64_t>(n) * K; }
  __device__ void store(int m, int n, float acc) const { out[static_cast<int64_t>(m) * N + n] = acc; }
};

// Gate and up projections of the self-conditioning block in one GEMM over
// the packed matrix W [2F, K]: rows 64 j + [0, 32) are gate rows 32 j + [0, 32)
// and rows 64 j + 32 + [0, 32) the up rows of the same hidden units, so a
// 32-column MFMA block of gate outputs and the block of up outputs of the
// same units sit side by side in every tile. hid[m, f] = round(gelu(g) * u).
struct GegluEpi {
  static constexpr bool kPair = true;
  const uint16_t *W;
  uint16_t *hid;
  int F;
  __device__ const uint16_t *brow(int n, int K) const { return W + static_cast<int64_t>(n) * K; }
  // n: the packed column of the gate value
  __device__ void store_pair(int m, int n, float g, float u) const {
    const int f = (n >> 6) * 32 + (n & 31);
    hid[static_cast<int64_t>(m) * F + f] = f32_to_bf16(gelu_tanh(g) * u);
  }
};

// Down projection of the self-conditioning block, z = hid W^T; rows of
// canvases marked in `frozen` (nullable) copy z_t instead.
struct DownEpi {
  static constexpr bool kPair = false;
  static constexpr bool kVec8 = true;
  const uint16_t *W;
  uint16_t *out;
  const uint16_t *zt;
  const int32_t *frozen;
  int N, C;
  __device__ const uint16_t *brow(int n, int K) const { return W + static_cast<int64_t>(n) * K; }
  __device__ void store(int m, int n, float acc) const {
    const int64_t idx = static_cast<int64_t>(m) * N + n;
    out[idx] = (frozen && frozen[m / C]) ? zt[idx] : f32_to_bf16(acc);
  }
  __device__ bool vec8_ok() const { return (N & 7) == 0 && aligned16(out) && aligned16(zt); }
  __device__ void store8(int m, int n, const float (&a)[8]) const {
    const int64_t idx = static_cast<int64_t>(m) * N + n;
    *reinterpret_cast<uint4 *>(out + idx) =
        (frozen && frozen[m / C]) ? *reinterpret_cast<const uint4 *>(zt + idx) : pack8(a);
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

// ---------------------------------------------------------------------------
// Deep-pipelined variant for K % 64 == 0: NS stages of 64-wide A and B slabs
// (8 KB each) are requested NS-1 slabs ahead with direct global->LDS loads,
// so about 128 KB per block is in flight: with few rows the tile is small and
// the memory latency, not the matrix cores, sets the pace. Rows of a slab are 128
// bytes; the 16-byte piece p of row r sits at p ^ ((r ^ (r >> 3)) & 7), which
// keeps the 32-row operand reads free of bank conflicts (32 or 64 banks).
constexpr int NS = 9;
constexpr int SLAB = 64 * 64;            // elements per operand slab

__device__ __forceinline__ int gswz(int r, int p) { return p ^ ((r ^ (r >> 3)) & 7); }

// 16 bytes per lane from base + voff into LDS at lds + 16 * lane (see the LM
// head for why this is issued through inline asm).
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, const uint16_t *lds) {
  const uint32_t m0 = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint16_t *)lds))));
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32)));
  const uint64_t sb = (static_cast<uint64_t>(hi) << 32) | lo;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0), "v"(voff), "s"(sb)
      : "memory");
}

template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}
// wait until at most k * STEP of this wave's vector-memory operations are
// outstanding, for a runtime k in [0, K]: K + 1 compile-time cases
template <int STEP, int K>
__device__ __forceinline__ void vm_wait_steps(int k) {
  if constexpr (K > 0) {
    if (k >= K) {
      vm_wait<K * STEP>();
      return;
    }
    vm_wait_steps<STEP, K - 1>(k);
  } else {
    vm_wait<0>();
  }
}

// 8 waves: wave (wk, wm, wn) computes the 32 x 32 quadrant (wm, wn) over the
// k-steps 2 wk, 2 wk + 1 of every slab; the two k-halves meet in LDS at the
// end. Two waves per SIMD and two independent accumulation chains per
// quadrant keep the matrix cores fed while slabs stream in.
template <class Epi>
__global__ void __launch_bounds__(512) gemm_tn_bf16_dma_kernel(const uint16_t *__restrict__ A,
                                                               int M, int N, int K, Epi epi) {
  __shared__ __attribute__((aligned(16))) uint16_t As[NS * SLAB];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[NS * SLAB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wk = wave >> 2, wm = (wave >> 1) & 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int nk = K / 64;

  // wave w loads slab rows 8 w .. 8 w + 7 of A and of B: one DMA instruction
  // each, lane i -> row 8 w + i / 8, physical piece i % 8. A lane's row is
  // clamped to the last valid one, so rows past M (or N) re-read a valid row
  // and every access stays inside the matrix; their results are never
  // stored. Offsets are bytes from the matrix (A) or tile (B) base and fit
  // in 32 bits (rows * K * 2 < 2^32). The rows of a tile come from one
  // weight matrix (N-sections are multiples of 64), whose row n0 is the base.
  const uint16_t *bbase = epi.brow(n0, K);
  const int r = 8 * wave + (lane >> 3);                // slab row of this lane
  const int piece = gswz(r, lane & 7);                 // logical piece kept at piece lane & 7
  const int am = (m0 + r < M) ? m0 + r : M - 1;
  const int bn = (n0 + r < N) ? r : N - 1 - n0;
  const uint32_t voff_a = static_cast<uint32_t>((static_cast<int64_t>(am) * K + piece * 8) * 2);
  const uint32_t voff_b = static_cast<uint32_t>((static_cast<int64_t>(bn) * K + piece * 8) * 2);
  auto issue = [&](int it) {
    const int buf = it % NS;
    dma16(A + it * 64, voff_a, As + buf * SLAB + 8 * wave * 64);
    dma16(bbase + it * 64, voff_b, Bs + buf * SLAB + 8 * wave * 64);
  };
  for (int it = 0; it < NS - 1 && it < nk; ++it) issue(it);

  f32x16 acc = {}, acc1 = {};
  const int ar = wm * 32 + (lane & 31), br = wn * 32 + (lane & 31);
  for (int it = 0; it < nk; ++it) {
    int younger = nk - 1 - it;                      // slabs issued after this one
    if (younger > NS - 2) younger = NS - 2;
    vm_wait_steps<2, NS - 2>(younger);
    __syncthreads();                                // every wave's part of slab `it` landed
    if (it + NS - 1 < nk) issue(it + NS - 1);       // refill the slab computed last iteration
    const uint16_t *as = As + (it % NS) * SLAB;
    const uint16_t *bs = Bs + (it % NS) * SLAB;
    {
      const int p0 = 2 * (2 * wk) + (lane >> 5), p1 = p0 + 2;
      const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(as + ar * 64 + gswz(ar, p0) * 8);
      const bf16x8 b0 = *reinterpret_cast<const bf16x8 *>(bs + br * 64 + gswz(br, p0) * 8);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(as + ar * 64 + gswz(ar, p1) * 8);
      const bf16x8 b1 = *reinterpret_cast<const bf16x8 *>(bs + br * 64 + gswz(br, p1) * 8);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc, 0, 0, 0);     // two independent chains
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc1, 0, 0, 0);
    }
  }
  acc += acc1;

  // k-halves meet in LDS (the stage buffers are free once everyone is here)
  __syncthreads();
  float *part = reinterpret_cast<float *>(As) + ((wm * 2 + wn) * 16) * 64;
  if (wk == 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) part[i * 64 + lane] = acc[i];
  }
  __syncthreads();
  if constexpr (Epi::kPair) {
    // the gate quadrant (wn = 0) and the up quadrant (wn = 1) of the same
    // hidden units meet in LDS as well
    if (wk == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] += part[i * 64 + lane];
    }
    __syncthreads();                                // `part` fully read
    float *upv = reinterpret_cast<float *>(As) + (wm * 16) * 64;
    if (wk == 0 && wn == 1) {
#pragma unroll
      for (int i = 0; i < 16; ++i) upv[i * 64 + lane] = acc[i];
    }
    __syncthreads();
    if (wk != 0 || wn != 0) return;
    const int n = n0 + (lane & 31);
    if (n < N) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + wm * 32 + 8 * j + 4 * (lane >> 5) + i;
          if (m < M) epi.store_pair(m, n, acc[4 * j + i], upv[(4 * j + i) * 64 + lane]);
        }
    }
  } else {
    if (wk == 1) return;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] += part[i * 64 + lane];

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
}

// ---------------------------------------------------------------------------
// Large-tile variant for many rows (batched canvases): 256 x 256 output tile
// per block, 8 waves as 2 x 4, each wave 128 x 64 (eight independent 32x32
// accumulators), K in 32-wide slabs (16 KB per operand) streamed by direct
// global->LDS loads through NS_BIG stages. A slab row is 64 bytes; its
// 16-byte piece p sits at p ^ bswz(r), which keeps the 32-row operand reads
// free of bank conflicts (32 or 64 banks).
namespace big {
constexpr int BMB = 256, BNB = 256, BKB = 32, NS_BIG = 4;
constexpr int kGroup = 4;        // row tiles per group of the XCD-aware order
constexpr int SLB = BMB * BKB;   // elements per operand slab

__device__ __forceinline__ int bswz(int r) { return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1); }

// 16 bytes per lane from a per-lane 64-bit address into lds + 16 * lane.
__device__ __forceinline__ void dma16_va(const void *src, const uint16_t *lds) {
  const uint32_t m0 = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint16_t *)lds))));
  const uint64_t addr = reinterpret_cast<uint64_t>(src);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0), "v"(addr)
      : "memory");
}

template <class Epi>
__global__ void __launch_bounds__(512) gemm_big_kernel(const uint16_t *__restrict__ A, int M, int N,
                                                       int K, Epi epi) {
  __shared__ __attribute__((aligned(16))) uint16_t As[NS_BIG * SLB];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[NS_BIG * SLB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  // XCD-aware tile order: the hardware deals blocks to the 8 XCDs in turn,
  // so block b runs on XCD b % 8. Give XCD x a contiguous run of tiles in a
  // grouped order (kGroup row tiles, column tiles slowest) so that the
  // blocks resident on one XCD share A and B tiles through its L2.
  const int gm = gridDim.y, gn = gridDim.x, T = gm * gn;
  int tm = blockIdx.y, tn = blockIdx.x;
  if ((T & 7) == 0 && gm % kGroup == 0) {
    const int b = blockIdx.y * gn + blockIdx.x;
    const int idx = (b & 7) * (T >> 3) + (b >> 3);
    const int grp = idx / (kGroup * gn), within = idx - grp * (kGroup * gn);
    tm = grp * kGroup + within % kGroup;
    tn = within / kGroup;
  }
  const int m0 = tm * BMB, n0 = tn * BNB;
  const int nk = K / BKB;

  // loads: a slab is 16 instructions per operand, each 16 rows x 64 bytes;
  // wave w issues instructions 2 w and 2 w + 1 of both. Lane i fills row
  // 16 u + i / 4, physical piece i % 4 (logical piece (i % 4) ^ bswz(row)).
  // Rows past M (N) re-read the last valid row; their results are dropped.
  const uint16_t *bbase = epi.brow(n0, K);   // the tile's rows come from one matrix
  const uint16_t *asrc[2], *bsrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 16 * (2 * wave + j) + (lane >> 2);
    const int lp = (lane & 3) ^ bswz(r);
    const int am = (m0 + r < M) ? m0 + r : M - 1;
    const int bn = (n0 + r < N) ? r : N - 1 - n0;
    asrc[j] = A + static_cast<int64_t>(am) * K + lp * 8;
    bsrc[j] = bbase + static_cast<int64_t>(bn) * K + lp * 8;
  }
  auto issue = [&](int it) {
    const int buf = it % NS_BIG, k0 = it * BKB;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      dma16_va(asrc[j] + k0, As + buf * SLB + (2 * wave + j) * 16 * BKB);
      dma16_va(bsrc[j] + k0, Bs + buf * SLB + (2 * wave + j) * 16 * BKB);
    }
  };
  for (int it = 0; it < NS_BIG - 1 && it < nk; ++it) issue(it);

  f32x16 acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    acc[mi][0] = f32x16{};
    acc[mi][1] = f32x16{};
  }
  for (int it = 0; it < nk; ++it) {
    int younger = nk - 1 - it;                      // slabs issued after this one
    if (younger > NS_BIG - 2) younger = NS_BIG - 2;
    vm_wait_steps<4, NS_BIG - 2>(younger);
    __syncthreads();                                // every wave's part of slab `it` landed
    if (it + NS_BIG - 1 < nk) issue(it + NS_BIG - 1);   // refill the slab computed last iteration
    const uint16_t *as = As + (it % NS_BIG) * SLB;
    const uint16_t *bs = Bs + (it % NS_BIG) * SLB;
#pragma unroll
    for (int ks = 0; ks < BKB / 16; ++ks) {
      const int p = 2 * ks + (lane >> 5);
      bf16x8 a[4], b[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int r = wm * 128 + mi * 32 + (lane & 31);
        a[mi] = *reinterpret_cast<const bf16x8 *>(as + r * BKB + ((p ^ bswz(r)) << 3));
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int r = wn * 64 + ni * 32 + (lane & 31);
        b[ni] = *reinterpret_cast<const bf16x8 *>(bs + r * BKB + ((p ^ bswz(r)) << 3));
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
  }

  // C layout of the 32x32 MFMA: lane holds column lane % 32 and rows
  // 8 j + 4 (lane / 32) + i in register 4 j + i
  if constexpr (Epi::kPair) {
    // a wave's 64 columns are one gate block (ni = 0) and the up block of
    // the same hidden units (ni = 1): the pair meets in registers
    const int n = n0 + wn * 64 + (lane & 31);
    if (n < N) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = m0 + wm * 128 + mi * 32 + 8 * j + 4 * (lane >> 5) + i;
            if (m < M) epi.store_pair(m, n, acc[mi][0][4 * j + i], acc[mi][1][4 * j + i]);
          }
    }
  } else {
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int n = n0 + wn * 64 + ni * 32 + (lane & 31);
      if (n >= N) continue;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = m0 + wm * 128 + mi * 32 + 8 * j + 4 * (lane >> 5) + i;
            if (m < M) epi.store(m, n, acc[mi][ni][4 * j + i]);
          }
    }
  }
}
}  // namespace big

// ---------------------------------------------------------------------------
// Few-row variant (up to a couple of thousand rows: one canvas, or a few):
// 64 x BN output tile per block, the chip filled by N / BN x M / 64 tiles.
// K streams through LDS in 128-wide slabs (direct global->LDS loads, whole
// 256-byte row segments), and the eight waves split each slab by K instead
// of splitting the tile: wave w multiplies k-step w (16 wide) of every slab
// for the whole 64 x BN tile, so each element staged in LDS is read exactly
// once. The eight partial tiles meet once, through LDS, at the end. Wide
// outputs take 128 x 64 tiles instead (see the kernel).
namespace skinny {
constexpr int BM = 64, BK = 128;
constexpr int PITCH64 = 72, PITCH32 = 40;   // LDS row pitch (floats) of a wave's partial tile:
                                            // rows 4 apart fall 32 banks apart

// slab row r (256 bytes, 16 pieces of 8 elements): logical piece p sits at
// physical piece p ^ (r & 15), which keeps the 16-row operand reads of one
// k-step on 16 distinct pieces (all 64 banks)
__device__ __forceinline__ int sk_off(int r, int p) { return r * BK + ((p ^ (r & 15)) << 3); }

// BMT rows per tile: 64, or 128 (row halves of 64, see the kernel)
template <int BN, int BMT = BM>
struct Cfg {
  static constexpr int NS = BMT == 128 ? 3 : (BN == 64 ? 4 : 5);   // slab stages
  static constexpr int STAGE = (BMT + BN) * BK;               // elements per stage
  static constexpr int PITCH = BN == 64 ? PITCH64 : PITCH32;
  static constexpr int RED = 8 * BM * PITCH * 4;              // bytes of the 8 partial 64-row tiles
  static constexpr int LDS = (NS * STAGE * 2 > RED) ? NS * STAGE * 2 : RED;
  static constexpr int DMA = (BMT + BN) / 32;                 // direct loads per wave and slab
  static_assert(LDS <= 160 * 1024, "LDS");
};

// Row sources of a block's 64-row tile: begin(tm) sets up row tile tm (false:
// the block has no rows), a_row(r) is the A row of tile row r (always a valid
// row: padding rows repeat a valid one), out(r) the output row (-1: padding),
// and b_off the element offset of the B matrix.
struct DenseRows {   // rows m0 .. m0 + bm - 1 of an [M, K] matrix
  int M;
  int bm = BM;
  int m0 = 0;
  int64_t b_off = 0;
  __device__ bool begin(int tm) {
    m0 = tm * bm;
    return true;
  }
  __device__ int a_row(int r) const { return m0 + r < M ? m0 + r : M - 1; }
  __device__ int out(int r) const { return m0 + r < M ? m0 + r : -1; }
};

// Mixture of experts: the (token, slot) entries routed to each expert are
// listed expert by expert (list, with offsets offs[X + 1]); expert e owns
// row tiles toff[e] .. toff[e + 1] - 1 and its B matrix sits bstride elements
// after expert e - 1's. The A row of entry q is q / adiv (the token for the
// gate/up GEMM, the entry itself for the down GEMM); outputs go to row q.
struct GroupRows {
  const int32_t *list, *offs, *toff;
  int X, adiv;
  int64_t bstride;
  int base = 0, cnt = 0;
  int64_t b_off = 0;
  __device__ bool begin(int tm) {
    if (tm >= toff[X]) return false;
    int e = 0;
    while (toff[e + 1] <= tm) ++e;
    base = offs[e] + BM * (tm - toff[e]);
    cnt = offs[e + 1] - base < BM ? offs[e + 1] - base : BM;
    b_off = e * bstride;
    return true;
  }
  __device__ int a_row(int r) const { return list[base + (r < cnt ? r : cnt - 1)] / adiv; }
  __device__ int out(int r) const { return r < cnt ? list[base + r] : -1; }
};

// BMT = 128: wave w computes row half w / 4 of the tile over k-steps w % 4
// and w % 4 + 4 of every slab; the four partials of each half meet in LDS.
template <class Epi, int BN, class Rows, int BMT = BM>
__global__ void __launch_bounds__(512) gemm_skinny_kernel(const uint16_t *__restrict__ A, Rows rows,
                                                          int mt, int N, int K, Epi epi) {
  static_assert(BMT == BM || BMT == 2 * BM, "row tile");
  using G = Cfg<BN, BMT>;
  constexpr int NR = BN / 32;                       // 32-column blocks per tile
  constexpr int NS = G::NS, PITCH = G::PITCH;
  __shared__ __attribute__((aligned(16))) uint16_t smem[G::LDS / 2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // XCD-aware order (block b runs on XCD b % 8): consecutive tiles in the
  // regrouped order share an XCD, and row tiles run fastest, so the blocks
  // that read the same weight rows share that XCD's L2
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int tn = bid / mt, tm = bid - tn * mt;
  if (!rows.begin(tm)) return;                      // uniform over the block, before any barrier
  const int n0 = tn * BN;

  // loads: one direct load fills 4 slab rows (1 KB); the slab's A rows and
  // then its B rows are dealt to the waves, G::DMA loads each. Lane i fills
  // row 4 g + i / 16 at physical piece i % 16. Padding rows (past the tile's
  // rows or past N) re-read a valid row; their results are never stored.
  const uint16_t *src[G::DMA];
  int dst[G::DMA];
#pragma unroll
  for (int j = 0; j < G::DMA; ++j) {
    const int g = wave * G::DMA + j;                // load index within the slab
    const int r = 4 * g + (lane >> 4);              // slab row, A rows first
    const int lp = (lane & 15) ^ (r & 15);          // logical piece this lane fetches
    if (r < BMT) {
      src[j] = A + static_cast<int64_t>(rows.a_row(r)) * K + 8 * lp;
    } else {
      const int n = (n0 + r - BMT < N) ? n0 + r - BMT : N - 1;
      src[j] = epi.brow(n, K) + rows.b_off + 8 * lp;
    }
    dst[j] = 4 * g * BK;                            // element offset of the load within a stage
  }
  auto issue = [&](int it) {
    uint16_t *stage = smem + (it % NS) * G::STAGE;
#pragma unroll
    for (int j = 0; j < G::DMA; ++j) big::dma16_va(src[j] + it * BK, stage + dst[j]);
  };
  const int nk = K / BK;
  for (int it = 0; it < NS - 1 && it < nk; ++it) issue(it);

  f32x16 acc[2][NR];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NR; ++j) acc[i][j] = f32x16{};
  const int p = 2 * wave + (lane >> 5);             // logical piece of this lane's k-step half
  const int rg = wave >> 2, kg = wave & 3;          // BMT = 128: row half and k-step group
  for (int it = 0; it < nk; ++it) {
    int younger = nk - 1 - it;                      // slabs issued after this one
    if (younger > NS - 2) younger = NS - 2;
    vm_wait_steps<G::DMA, NS - 2>(younger);
    __syncthreads();                                // every wave's part of slab `it` landed
    if (it + NS - 1 < nk) issue(it + NS - 1);       // refill the stage every wave finished reading
    const uint16_t *as = smem + (it % NS) * G::STAGE;
    const uint16_t *bs = as + BMT * BK;
    if constexpr (BMT == BM) {
      bf16x8 a[2], b[NR];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = *reinterpret_cast<const bf16x8 *>(as + sk_off(32 * i + (lane & 31), p));
#pragma unroll
      for (int j = 0; j < NR; ++j) b[j] = *reinterpret_cast<const bf16x8 *>(bs + sk_off(32 * j + (lane & 31), p));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NR; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    } else {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int pk = 2 * (kg + 4 * kk) + (lane >> 5);
        bf16x8 a[2], b[NR];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          a[i] = *reinterpret_cast<const bf16x8 *>(as + sk_off(64 * rg + 32 * i + (lane & 31), pk));
#pragma unroll
        for (int j = 0; j < NR; ++j) b[j] = *reinterpret_cast<const bf16x8 *>(bs + sk_off(32 * j + (lane & 31), pk));
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < NR; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
    }
  }

  // the eight partial tiles meet in LDS (the stages are free once everyone is
  // here); MFMA C layout: lane holds column lane % 32 of each 32-column block
  // and rows 8 q + 4 (lane / 32) + e in register 4 q + e
  __syncthreads();
  float *red = reinterpret_cast<float *>(smem);
  float *mine = red + wave * BM * PITCH;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NR; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          mine[(32 * i + 8 * q + 4 * (lane >> 5) + e) * PITCH + 32 * j + (lane & 31)] = acc[i][j][4 * q + e];
  __syncthreads();
  // tile row r: the sum of the eight K-split partials (BMT = 64), or of the
  // four partials of its row half (BMT = 128)
  auto sum8 = [&](int r, int col) {
    float s = 0.f;
    if constexpr (BMT == BM) {
#pragma unroll
      for (int w = 0; w < 8; ++w) s += red[w * BM * PITCH + r * PITCH + col];
    } else {
      const float *h = red + (r >> 6) * 4 * BM * PITCH + (r & 63) * PITCH + col;
#pragma unroll
      for (int w = 0; w < 4; ++w) s += h[w * BM * PITCH];
    }
    return s;
  };
  if constexpr (Epi::kPair) {
    // columns [0, 32) of the tile are gate values, [32, 64) the up values of the same units
    static_assert(BN == 64, "gate/up pairs need 64-column tiles");
    for (int e = tid; e < BMT * 32; e += 512) {
      const int r = e >> 5, col = e & 31;
      const int m = rows.out(r), n = n0 + col;
      if (m >= 0 && n < N) epi.store_pair(m, n, sum8(r, col), sum8(r, col + 32));
    }
  } else {
    if constexpr (Epi::kVec8) {
      if ((N & 7) == 0 && epi.vec8_ok()) {
        // one thread per 8 consecutive columns of a tile row: 16-byte
        // partial reads, one destination computation and one 16-byte store;
        // the partials are summed in the same order as sum8
        for (int e = tid; e < BMT * BN / 8; e += 512) {
          const int r = e / (BN / 8), col = 8 * (e - r * (BN / 8));
          const int m = rows.out(r), n = n0 + col;
          if (m < 0 || n >= N) continue;
          float a[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) a[i] = 0.f;
          const float *base;
          int nw, wstride;
          if constexpr (BMT == BM) {
            base = red + r * PITCH + col;
            nw = 8;
            wstride = BM * PITCH;
          } else {
            base = red + (r >> 6) * 4 * BM * PITCH + (r & 63) * PITCH + col;
            nw = 4;
            wstride = BM * PITCH;
          }
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            if (w < nw) {
              const f32x4 lo = *reinterpret_cast<const f32x4 *>(base + w * wstride);
              const f32x4 hi = *reinterpret_cast<const f32x4 *>(base + w * wstride + 4);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                a[i] += lo[i];
                a[4 + i] += hi[i];
              }
            }
          }
          epi.store8(m, n, a);
        }
        return;
      }
    }
    for (int e = tid; e < BMT * BN; e += 512) {
      const int r = e / BN, col = e - r * BN;
      const int m = rows.out(r), n = n0 + col;
      if (m >= 0 && n < N) epi.store(m, n, sum8(r, col));
    }
  }
}

// 64-column tiles (fewest operand bytes per output) once they cover most of
// the 256 CUs, 32-column ones below that (twice the tiles). K % 128 == 0.
template <class Epi, class Rows>
hipError_t launch_rows(const uint16_t *A, const Rows &rows, int mt, int N, int K, const Epi &epi,
                       hipStream_t st) {
  if (Epi::kPair || static_cast<int64_t>(mt) * ((N + 63) / 64) >= 160) {
    const int blocks = mt * ((N + 63) / 64);
    hipLaunchKernelGGL((gemm_skinny_kernel<Epi, 64, Rows>), dim3(blocks), dim3(512), 0, st, A, rows, mt,
                       N, K, epi);
  } else if constexpr (!Epi::kPair) {
    const int blocks = mt * ((N + 31) / 32);
    hipLaunchKernelGGL((gemm_skinny_kernel<Epi, 32, Rows>), dim3(blocks), dim3(512), 0, st, A, rows, mt,
                       N, K, epi);
  }
  return hipGetLastError();
}

// Dense rows: 128-row tiles where 64-row ones would give at least two blocks
// per CU of 64-column tiles (wide outputs, e.g. the gate/up GEMM of a wide
// MLP): each B tile then serves twice the rows, and each CU moves 3/4 of
// the operand bytes.
template <class Epi>
hipError_t launch(const uint16_t *A, int M, int N, int K, const Epi &epi, hipStream_t st) {
  const int mt = (M + BM - 1) / BM;
  if (M > BM && static_cast<int64_t>(mt) * ((N + 63) / 64) >= 512) {
    DenseRows rows{M};
    rows.bm = 2 * BM;
    const int mt2 = (M + 2 * BM - 1) / (2 * BM);
    const int blocks = mt2 * ((N + 63) / 64);
    hipLaunchKernelGGL((gemm_skinny_kernel<Epi, 64, DenseRows, 2 * BM>), dim3(blocks), dim3(512), 0, st, A,
                       rows, mt2, N, K, epi);
    return hipGetLastError();
  }
  return launch_rows(A, DenseRows{M}, mt, N, K, epi, st);
}
}  // namespace skinny

}  // namespace

// below this many rows the 256-row tiles would leave most of the chip idle
constexpr int kBigRows = 2048;

hipError_t launch_qkv_bf16(const uint16_t *h0, const uint16_t *Wq, const uint16_t *Wk,
                           const uint16_t *Wv, const Shape &s, uint16_t *q, uint16_t *k,
                           uint16_t *v, hipStream_t st) {
  QkvEpi epi{Wq, Wk, Wv, q, k, v, s.Hq * s.hd, s.Hkv * s.hd, s.C, s.Hkv, s.hd};
  const int M = s.R(), N = s.Hq * s.hd + 2 * s.Hkv * s.hd;
  if (M == 0) return hipSuccess;
  dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
  if (M >= kBigRows && s.d % big::BKB == 0 && (s.Hq * s.hd) % big::BNB == 0 &&
      (s.Hkv * s.hd) % big::BNB == 0)
    hipLaunchKernelGGL(big::gemm_big_kernel<QkvEpi>, dim3(N / big::BNB, (M + big::BMB - 1) / big::BMB),
                       dim3(512), 0, st, h0, M, N, s.d, epi);
  else if (s.d % skinny::BK == 0)
    return skinny::launch(h0, M, N, s.d, epi, st);
  else if (s.d % 64 == 0 && (s.Hq * s.hd) % 64 == 0 && (s.Hkv * s.hd) % 64 == 0)
    hipLaunchKernelGGL(gemm_tn_bf16_dma_kernel<QkvEpi>, grid, dim3(512), 0, st, h0, M, N, s.d, epi);
  else
    hipLaunchKernelGGL(gemm_tn_bf16_kernel<QkvEpi>, grid, dim3(256), 0, st, h0, M, N, s.d, epi);
  return hipGetLastError();
}

hipError_t launch_kv_encode_bf16(const uint16_t *h, const uint16_t *Wk, const uint16_t *Wv,
                                 const Shape &s, int n, int pos, int Pst, uint16_t *K, uint16_t *V,
                                 hipStream_t st) {
  const int Nkv = s.Hkv * s.hd;
  KvCacheEpi epi{Wk, Wv, K, V, Nkv, n, pos, Pst, s.Hkv, s.hd};
  const int M = s.B * n, N = 2 * Nkv;
  if (M == 0) return hipSuccess;
  if (M >= kBigRows && s.d % big::BKB == 0 && Nkv % big::BNB == 0)
    hipLaunchKernelGGL(big::gemm_big_kernel<KvCacheEpi>, dim3(N / big::BNB, (M + big::BMB - 1) / big::BMB),
                       dim3(512), 0, st, h, M, N, s.d, epi);
  else if (s.d % skinny::BK == 0)
    return skinny::launch(h, M, N, s.d, epi, st);
  else
    hipLaunchKernelGGL(gemm_tn_bf16_kernel<KvCacheEpi>, dim3((N + BN - 1) / BN, (M + BM - 1) / BM),
                       dim3(256), 0, st, h, M, N, s.d, epi);
  return hipGetLastError();
}

hipError_t launch_moe_experts_bf16(const uint16_t *m, const uint16_t *Wgu, const uint16_t *Wd,
                                   const int32_t *list, const int32_t *offs, const int32_t *toff,
                                   int R, int top_k, int X, int d, int F, uint16_t *hid, float *y,
                                   hipStream_t st) {
  static_assert(skinny::BM == kMoeTile, "expert tiles are the few-row kernel's row tiles");
  const int n = R * top_k;
  if (n == 0) return hipSuccess;
  if (d % skinny::BK != 0 || F % skinny::BK != 0) return hipErrorInvalidValue;
  // every expert's last tile may be partial: at most n / 64 + X row tiles
  const int mt = (n + kMoeTile - 1) / kMoeTile + X;
  skinny::GroupRows gu{list, offs, toff, X, top_k, static_cast<int64_t>(2) * F * d};
  hipError_t e = skinny::launch_rows(m, gu, mt, 2 * F, d, GegluEpi{Wgu, hid, F}, st);
  if (e != hipSuccess) return e;
  skinny::GroupRows dn{list, offs, toff, X, 1, static_cast<int64_t>(d) * F};
  return skinny::launch_rows(hid, dn, mt, d, F, F32StoreEpi{Wd, y, d}, st);
}

hipError_t launch_ffw_gate_up_bf16(const uint16_t *u, const uint16_t *Wgu, int M, int d, int F,
                                   uint16_t *hid, hipStream_t st) {
  GegluEpi epi{Wgu, hid, F};
  const int N = 2 * F, K = d;
  if (M == 0) return hipSuccess;
  if (K % 64 != 0 || F % 32 != 0) return hipErrorInvalidValue;
  if (M >= kBigRows && N % big::BNB == 0)
    hipLaunchKernelGGL(big::gemm_big_kernel<GegluEpi>, dim3(N / big::BNB, (M + big::BMB - 1) / big::BMB),
                       dim3(512), 0, st, u, M, N, K, epi);
  else if (K % skinny::BK == 0)
    return skinny::launch(u, M, N, K, epi, st);
  else
    hipLaunchKernelGGL(gemm_tn_bf16_dma_kernel<GegluEpi>, dim3(N / BN, (M + BM - 1) / BM), dim3(512), 0,
                       st, u, M, N, K, epi);
  return hipGetLastError();
}

hipError_t launch_ffw_down_bf16(const uint16_t *hid, const uint16_t *Wd, int M, int d, int F, int C,
                                const int32_t *frozen, const uint16_t *z_t, uint16_t *z,
                                hipStream_t st) {
  DownEpi epi{Wd, z, z_t, frozen, d, C};
  const int N = d, K = F;
  if (M == 0) return hipSuccess;
  if (K % 64 != 0 || N % 64 != 0) return hipErrorInvalidValue;
  if (M >= kBigRows && N % big::BNB == 0)
    hipLaunchKernelGGL(big::gemm_big_kernel<DownEpi>, dim3(N / big::BNB, (M + big::BMB - 1) / big::BMB),
                       dim3(512), 0, st, hid, M, N, K, epi);
  else if (K % skinny::BK == 0)
    return skinny::launch(hid, M, N, K, epi, st);
  else
    hipLaunchKernelGGL(gemm_tn_bf16_dma_kernel<DownEpi>, dim3(N / BN, (M + BM - 1) / BM), dim3(512), 0,
                       st, hid, M, N, K, epi);
  return hipGetLastError();
}

hipError_t launch_residual_gemm_bf16(const uint16_t *A, const uint16_t *W, const uint16_t *res, int M,
                                    int N, int K, uint16_t *out, hipStream_t st) {
  ResidualEpi epi{W, res, out, N};
  if (M == 0) return hipSuccess;
  dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
  if (M >= kBigRows && K % big::BKB == 0 && N % big::BNB == 0)
    hipLaunchKernelGGL(big::gemm_big_kernel<ResidualEpi>, dim3(N / big::BNB, (M + big::BMB - 1) / big::BMB),
                       dim3(512), 0, st, A, M, N, K, epi);
  else if (K % skinny::BK == 0)
    return skinny::launch(A, M, N, K, epi, st);
  else if (K % 64 == 0)
    hipLaunchKernelGGL(gemm_tn_bf16_dma_kernel<ResidualEpi>, grid, dim3(512), 0, st, A, M, N, K, epi);
  else
    hipLaunchKernelGGL(gemm_tn_bf16_kernel<ResidualEpi>, grid, dim3(256), 0, st, A, M, N, K, epi);
  return hipGetLastError();
}

}  // namespace dg
