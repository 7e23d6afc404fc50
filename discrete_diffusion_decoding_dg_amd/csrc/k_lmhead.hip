// Fused LM head, softmax statistics, self-conditioning z and Gumbel-max draw
// on bf16 MFMA. The C x V logits never leave the chip.
//
// DiffusionGemma Technical Report (hyper.ai summary), Method, three-line
// update: p0 = Softmax(L / tau), z = FFW(p0 E) (FFW read as identity, E the
// tied embedding), x_{t-dt} ~ Step(x_t, p0). The Step draw for a row that
// resamples (Bernoulli u < lambda, decided before the vocabulary loop) is
// argmax_v s_v + G_v with Philox Gumbel noise; kept rows skip the noise.
//
// Decomposition. A block owns MT canvas rows and a contiguous vocabulary
// range (one "split"); 8 waves split the model width d into slices of DW.
// Per 16-row vocabulary tile:
//   1. every wave stages E[tile, its slice] in LDS;
//   2. partial scores S^T[v, m] over the slice, v_mfma_f32_16x16x32_bf16 with
//      E as A operand (rows = vocab) and the register-resident h1 slice as B;
//   3. the 8 partials are summed through LDS; two waves turn the 16 x MT
//      tile into scaled logits, online max / sum (log2 units, the reference
//      max moves only when the tile max exceeds it by more than 8, so z is
//      rarely rescaled), bf16 probabilities P in LDS, and the Gumbel argmax;
//   4. every wave accumulates z[m, slice] += P[m, tile] E[tile, slice] with
//      v_mfma_f32_16x16x16_bf16 (vocab as K; E read transposed from LDS).
// A block ends by writing (m, l, best, arg) per row and its unnormalised z
// slice partials; the combine kernel merges the splits.
#include "dg_device.hpp"
#include "dg_kernels.hpp"

namespace dg {
namespace {

constexpr int NW = 8;            // waves per block
constexpr int VT = 16;           // vocabulary rows per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;   // log2 units

struct LmArgs {
  const uint16_t *h1, *E;
  const int32_t *x_t;
  const StepParams *prm;
  RowPartial *part;   // [splits][R]
  float *zpart;       // [splits][R][d]
  float *p0;          // optional [R][V] raw scaled logits
  int R, C, d, V, splits, tiles_per_split;
  uint32_t k0, k1;
};

template <int MT, int DW>
__global__ void __launch_bounds__(512) lmhead_kernel(LmArgs a) {
  constexpr int RB = MT / 16;        // 16-row blocks
  constexpr int NKS = DW / 32;       // k-steps of the score contraction per wave
  constexpr int NB = DW / 16;        // 16-wide z column blocks per wave
  constexpr int EP = DW + 8;         // LDS pitch of an E slice row (elements)
  constexpr int CH = DW / 8;         // 16-byte chunks per slice row

  __shared__ __attribute__((aligned(16))) uint16_t Es[NW][VT * EP];
  __shared__ __attribute__((aligned(16))) f32x4 red[NW][RB][64];
  __shared__ __attribute__((aligned(16))) uint16_t Ps[MT][VT];
  __shared__ float m_ref[MT], l_run[MT], best_val[MT], scale[MT];
  __shared__ int best_idx[MT], resample[MT];
  __shared__ int any_rescale;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row0 = blockIdx.x * MT;
  const int split = blockIdx.y;
  const int dcol0 = wave * DW;

  if (tid < MT) {
    const int r = row0 + tid;
    int rs = 0;
    if (r < a.R) {
      const int b = r / a.C, i = r - b * a.C;
      const u32x4 w = philox4x32_10(0u, static_cast<uint32_t>(i), static_cast<uint32_t>(b),
                                    kStreamBernoulli, a.k0, a.k1);
      rs = u01(w.x) < a.prm[b].lam ? 1 : 0;
    }
    resample[tid] = rs;
    m_ref[tid] = -INFINITY;
    l_run[tid] = 0.f;
    best_val[tid] = -INFINITY;
    best_idx[tid] = -1;
    scale[tid] = 1.f;
  }
  if (tid == 0) any_rescale = 0;

  // h1 slice as the B operand: lane holds canvas row 16 rb + (lane & 15),
  // columns dcol0 + 32 ks + 8 (lane >> 4) + [0, 8)
  bf16x8 hreg[RB][NKS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = row0 + rb * 16 + (lane & 15);
    const uint16_t *hrow = a.h1 + static_cast<int64_t>(r) * a.d + dcol0 + (lane >> 4) * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      hreg[rb][ks] = (r < a.R) ? *reinterpret_cast<const bf16x8 *>(hrow + ks * 32) : bf16x8{};
  }

  f32x4 zacc[RB][NB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) zacc[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int total_tiles = a.V / VT;
  const int t_begin = split * a.tiles_per_split;
  int t_end = t_begin + a.tiles_per_split;
  if (t_end > total_tiles) t_end = total_tiles;

  uint16_t *es = Es[wave];
  for (int tile = t_begin; tile < t_end; ++tile) {
    const int v0 = tile * VT;
    // 1. stage this wave's E slice
    for (int c = lane; c < VT * CH; c += 64) {
      const int vr = c / CH, col = (c - vr * CH) * 8;
      *reinterpret_cast<uint4 *>(&es[vr * EP + col]) = *reinterpret_cast<const uint4 *>(
          a.E + static_cast<int64_t>(v0 + vr) * a.d + dcol0 + col);
    }
    __syncthreads();

    // 2. partial S^T over the slice
    {
      const uint16_t *erow = &es[(lane & 15) * EP + (lane >> 4) * 8];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const bf16x8 ef = *reinterpret_cast<const bf16x8 *>(erow + ks * 32);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ef, hreg[rb][ks], acc, 0, 0, 0);
        }
        red[wave][rb][lane] = acc;
      }
    }
    __syncthreads();

    // 3. reduce, softmax statistics, probabilities, Gumbel argmax
    if (tid < MT * 4) {
      const int rb = tid >> 6, ln = tid & 63;
      const int lrow = rb * 16 + (ln & 15);
      const int r = row0 + lrow;
      f32x4 acc = red[0][rb][ln];
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        const f32x4 t = red[w][rb][ln];
        acc[0] += t[0]; acc[1] += t[1]; acc[2] += t[2]; acc[3] += t[3];
      }
      const bool valid = r < a.R;
      const int b = valid ? r / a.C : 0;
      const float inv_tau = valid ? a.prm[b].inv_tau : 0.f;
      const int vq = v0 + (ln >> 4) * 4;   // first of this lane's 4 vocab ids
      float s[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) s[j] = acc[j] * inv_tau;
      if (a.p0 && valid) {
        float *prow = a.p0 + static_cast<int64_t>(r) * a.V + vq;
#pragma unroll
        for (int j = 0; j < 4; ++j) prow[j] = s[j];
      }
      // Gumbel-max over this lane's 4 ids, then across the 4 lanes of the row
      float bv = -INFINITY;
      int bi = -1;
      if (valid && resample[lrow]) {
        const int i = r - b * a.C;
        const u32x4 w = philox4x32_10(static_cast<uint32_t>(vq >> 2), static_cast<uint32_t>(i),
                                      static_cast<uint32_t>(b), kStreamGumbel, a.k0, a.k1);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float pv = s[j] + gumbel(ws[j]);
          if (pv > bv) { bv = pv; bi = vq + j; }
        }
      }
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (ov > bv || (ov == bv && oi >= 0 && (bi < 0 || oi < bi))) { bv = ov; bi = oi; }
      }
      // softmax statistics in log2 units
      float s2[4], tmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s2[j] = s[j] * kLog2e;
        tmax = fmaxf(tmax, s2[j]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_old = m_ref[lrow];
      float m_new = m_old, sc = 1.f;
      if (tmax > m_old + kRescaleSlack) {
        m_new = tmax;
        sc = exp2f(m_old - m_new);   // 0 when m_old = -inf
      }
      float psum = 0.f;
      uint16_t pb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = exp2f(s2[j] - m_new);
        psum += p;
        pb[j] = f32_to_bf16(p);
      }
      psum += __shfl_xor(psum, 16, 64);
      psum += __shfl_xor(psum, 32, 64);
      *reinterpret_cast<uint2 *>(&Ps[lrow][(ln >> 4) * 4]) =
          make_uint2(pb[0] | (static_cast<uint32_t>(pb[1]) << 16),
                     pb[2] | (static_cast<uint32_t>(pb[3]) << 16));
      __builtin_amdgcn_wave_barrier();   // all 4 lanes of the row have read m_ref
      if ((ln >> 4) == 0) {
        scale[lrow] = sc;
        m_ref[lrow] = m_new;
        l_run[lrow] = l_run[lrow] * sc + psum;
        if (bi >= 0 && bv > best_val[lrow]) { best_val[lrow] = bv; best_idx[lrow] = bi; }
        if (sc != 1.f) any_rescale = 1;
      }
    }
    __syncthreads();

    // 4. z += P E over this wave's slice
    if (any_rescale) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float sr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sr[i] = scale[rb * 16 + (lane >> 4) * 4 + i];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) zacc[rb][nb][i] *= sr[i];
      }
    }
    {
      s16x4 pa[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        pa[rb] = *reinterpret_cast<const s16x4 *>(&Ps[rb * 16 + (lane & 15)][(lane >> 4) * 4]);
      const uint16_t *ecol = &es[((lane >> 4) * 4) * EP + (lane & 15)];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        s16x4 eb;
#pragma unroll
        for (int j = 0; j < 4; ++j) eb[j] = static_cast<short>(ecol[j * EP + nb * 16]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          zacc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa[rb], eb, zacc[rb][nb], 0, 0, 0);
      }
    }
    __syncthreads();
    if (tid == 0) any_rescale = 0;
  }

  // write the split partials
  if (tid < MT) {
    const int r = row0 + tid;
    if (r < a.R) {
      RowPartial p;
      p.m = m_ref[tid];
      p.l = l_run[tid];
      p.best = best_val[tid];
      p.arg = best_idx[tid];
      a.part[static_cast<int64_t>(split) * a.R + r] = p;
    }
  }
  float *zs = a.zpart + static_cast<int64_t>(split) * a.R * a.d;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = row0 + rb * 16 + (lane >> 4) * 4 + i;
      if (r >= a.R) continue;
      float *zr = zs + static_cast<int64_t>(r) * a.d + dcol0 + (lane & 15);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) zr[nb * 16] = zacc[rb][nb][i];
    }
}

// ---------------------------------------------------------------------------
// Version for d = 8 * DW with DW <= 256 (32-row vocabulary tiles).
//
// Each of the 8 waves owns a DW-wide slice of d for both contractions. Its
// slice of the 32 x d E tile lives in a private LDS region, chunk-major
// (chunks of 32 columns, 32 rows x 64 B each, 16-byte pieces XOR-swizzled by
// row), and is filled by direct global->LDS loads. Chunk c of the next tile
// is requested as soon as the z contraction of this tile is done with it, so
// the loads overlap the rest of the tile's work.
//   S^T partial: A = E chunk (ds_read_b128), B = h1 slice in registers.
//   Partials of the 8 slices meet in LDS; wave w reduces rows 4w..4w+3 (its
//   rows for the whole kernel: their running max, sum and best draw stay in
//   its registers) and writes P (bf16) and the rescale factor back in place,
//   into the positions of its own partial slot that only it reads.
//   z += P E: A = P (4 ds_read_b32 per 16 rows), B = E chunk read transposed
//   with ds_read_b64_tr_b16 (lane (q, n) gets 4 consecutive vocab rows of
//   column n), v_mfma_f32_16x16x32_bf16 with K = 32 vocabulary rows.
namespace v2 {

constexpr int NW = 8, MT = 32, VT = 32;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their
// maxima). The builtin is visible to the compiler's own wait insertion.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");   // no memory access moves across the wait
}
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

// Physical 16-byte piece of logical piece q in row r of a chunk (64-byte
// rows). The XOR pattern keeps the three access patterns free of LDS bank
// conflicts for both 32 and 64 banks of 4 bytes: DMA writes (contiguous),
// 16-byte operand reads of 16 rows, and transposed 8-byte reads of 4 rows.
__device__ __forceinline__ int swz(int r, int q) {
  return q ^ (((r >> 2) & 1) | ((((r >> 1) ^ (r >> 2) ^ (r >> 3)) & 1) << 1));
}
// Position of the 16-byte vocabulary group g (4 fp32) in row r of a 32 x 32
// fp32 tile of the reduction buffer: conflict-free partial writes (16-byte,
// 16 rows x 4 groups) and epilogue reads (8-byte, 4 rows x 32 values).
__device__ __forceinline__ int rswz(int r, int g) {
  return g ^ (((r >> 1) & 1) | (((r >> 2) & 1) << 1) | (((r ^ (r >> 3)) & 1) << 2));
}

// Direct global -> LDS load of 16 bytes per lane: lane i's bytes land at
// lds + 16 i (lds must be wave-uniform). Issued through inline asm so that
// the compiler does not add conservative waits before unrelated LDS reads;
// every read of DMA'd data is preceded by an explicit vmcnt wait instead.
// The instruction has no register result: its address registers are read at
// issue.
// `base` is wave-uniform (scalar registers), `voff` the lane's byte offset.
__device__ __forceinline__ void lds_dma16(const void *base, uint32_t voff, uint16_t *lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint16_t *)lds)));
  // readfirstlane returns a signed int: go through uint32_t so that the low
  // half is zero-extended (a sign-extended low half would corrupt the upper
  // address bits whenever bit 31 is set)
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32)));
  const uint64_t sb = (static_cast<uint64_t>(hi) << 32) | lo;
  uint32_t saved;
  // M0 is reserved by the compiler: keep its value across the block
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

template <int DW>
__global__ void __launch_bounds__(512) lmhead_v2_kernel(LmArgs a, int rblocks) {
  constexpr int NKS = DW / 32;           // 32-column chunks per slice
  constexpr int NB = DW / 16;            // 16-column z blocks per slice
  constexpr int CHUNK = 32 * 32;         // elements per chunk
  __shared__ __attribute__((aligned(16))) uint16_t Es[NW * NKS * CHUNK];
  __shared__ __attribute__((aligned(16))) float red[NW][MT][VT];   // [wave][row][vocab], swizzled groups

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // XCD-aware order: consecutive blocks land on different XCDs, so regroup
  // them to give each XCD a contiguous run of (split, row block) pairs: the
  // row blocks that share a vocabulary range then share that XCD's L2.
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int split = bid / rblocks;
  const int row0 = (bid - split * rblocks) * MT;
  const int dcol0 = wave * DW;
  uint16_t *es = Es + wave * NKS * CHUNK;
  auto chunk = [&](int c) -> uint16_t * { return es + c * CHUNK; };

  const int total_tiles = a.V / VT;
  const int t_begin = split * a.tiles_per_split;
  int t_end = t_begin + a.tiles_per_split;
  if (t_end > total_tiles) t_end = total_tiles;

  // DMA of chunk c of tile `tile` into this wave's slice: 2 x 64 lanes x 16 B.
  // Lane i fills LDS piece i of the half: row 16 h + i / 4, physical piece
  // i % 4, which holds the row's logical piece swz(row, i % 4) (an XOR, so
  // its own inverse); the swizzle ignores row bit 4, so both halves share it.
  const uint32_t dma_off = static_cast<uint32_t>(((lane >> 2) * a.d + swz(lane >> 2, lane & 3) * 8) * 2);
  auto dma_chunk = [&](int tile, int c) {
    const uint16_t *tb = a.E + static_cast<int64_t>(tile * VT) * a.d + dcol0 + c * 32;
#pragma unroll
    for (int h = 0; h < 2; ++h) lds_dma16(tb + static_cast<int64_t>(16 * h) * a.d, dma_off, chunk(c) + h * 16 * 32);
  };
  if (t_begin < t_end)
#pragma unroll
    for (int c = 0; c < NKS; ++c) dma_chunk(t_begin, c);

  // h1 slice as the B operand of S^T: lane holds canvas row 16 rb + (lane & 15),
  // columns dcol0 + 32 c + 8 (lane >> 4) + [0, 8)
  bf16x8 hreg[2][NKS];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = row0 + rb * 16 + (lane & 15);
    const uint16_t *hrow = a.h1 + static_cast<int64_t>(r) * a.d + dcol0 + (lane >> 4) * 8;
#pragma unroll
    for (int c = 0; c < NKS; ++c)
      hreg[rb][c] = (r < a.R) ? *reinterpret_cast<const bf16x8 *>(hrow + c * 32) : bf16x8{};
  }

  // the rows this wave reduces: M = 4 wave + (lane >> 4); lane pair index j2
  const int erow = 4 * wave + (lane >> 4);
  const int j2 = lane & 15;                  // vocab 2 j2, 2 j2 + 1 of the tile
  const int grow = row0 + erow;
  const bool rvalid = grow < a.R;
  const int gb = rvalid ? grow / a.C : 0;
  const int gi = rvalid ? grow - gb * a.C : 0;
  const float inv_tau = rvalid ? a.prm[gb].inv_tau : 0.f;
  bool resample = false;
  if (rvalid) {
    const u32x4 w = philox4x32_10(0u, static_cast<uint32_t>(gi), static_cast<uint32_t>(gb),
                                  kStreamBernoulli, a.k0, a.k1);
    resample = u01(w.x) < a.prm[gb].lam;
  }
  float m_ref = -INFINITY, l_run = 0.f, best_v = -INFINITY;
  int best_i = -1;
  // where this lane's pair (vocab 2 j2, 2 j2 + 1 of row erow) sits in a slot
  const int e_off = erow * VT + rswz(erow, j2 >> 1) * 4 + 2 * (j2 & 1);

  f32x4 zacc[2][NB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) zacc[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // everything issued so far (the first tile's chunks, h1, step constants)
  // has landed: the loop below tracks only its own chunk loads
  wait_vmcnt<0>();

  for (int tile = t_begin; tile < t_end; ++tile) {
    const int v0 = tile * VT;
    const bool more = tile + 1 < t_end;
    if (a.p0) wait_vmcnt<0>();   // checking mode: p0 stores share the counter
    // ---- S^T partial over this wave's slice
    f32x4 sacc[2][2];
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) sacc[vb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NKS; ++c) {
      wait_vmcnt_le(2 * (NKS - 1 - c));
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) {
        const int r = vb * 16 + (lane & 15);
        const bf16x8 ef = *reinterpret_cast<const bf16x8 *>(chunk(c) + r * 32 + swz(r, lane >> 4) * 8);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          sacc[vb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ef, hreg[rb][c], sacc[vb][rb], 0, 0, 0);
      }
    }
    // lane (q, m) of block (vb, rb) holds row 16 rb + m, vocab 16 vb + 4 q + [0, 4)
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int r = rb * 16 + (lane & 15);
        *reinterpret_cast<f32x4 *>(&red[wave][r][rswz(r, vb * 4 + (lane >> 4)) * 4]) = sacc[vb][rb];
      }
    __syncthreads();

    // ---- epilogue for rows 4 wave .. 4 wave + 3
    {
      float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float2 pr = *reinterpret_cast<const float2 *>(&red[w][0][0] + e_off);
        acc0 += pr.x;
        acc1 += pr.y;
      }
      const int v = v0 + 2 * j2;
      const float s0 = acc0 * inv_tau, s1 = acc1 * inv_tau;
      if (a.p0 && rvalid) {
        float *prow = a.p0 + static_cast<int64_t>(grow) * a.V + v;
        prow[0] = s0;
        prow[1] = s1;
      }
      float bv = -INFINITY;
      int bi = -1;
      if (resample) {
        const u32x4 w = philox4x32_10(static_cast<uint32_t>(v >> 2), static_cast<uint32_t>(gi),
                                      static_cast<uint32_t>(gb), kStreamGumbel, a.k0, a.k1);
        const uint32_t w0 = (v & 2) ? w.z : w.x, w1 = (v & 2) ? w.w : w.y;
        const float p0v = s0 + gumbel(w0), p1v = s1 + gumbel(w1);
        bv = p0v;
        bi = v;
        if (p1v > bv) { bv = p1v; bi = v + 1; }
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (ov > bv || (ov == bv && oi >= 0 && (bi < 0 || oi < bi))) { bv = ov; bi = oi; }
      }
      if (bi >= 0 && bv > best_v) { best_v = bv; best_i = bi; }
      const float t0 = s0 * kLog2e, t1 = s1 * kLog2e;
      float tmax = fmaxf(t0, t1);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o, 64));
      float sc = 1.f;
      if (tmax > m_ref + kRescaleSlack) {
        sc = exp2f(m_ref - tmax);   // 0 on the first tile
        m_ref = tmax;
      }
      const float p0f = exp2f(t0 - m_ref), p1f = exp2f(t1 - m_ref);
      float ps = p0f + p1f;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) ps += __shfl_xor(ps, o, 64);
      l_run = l_run * sc + ps;
      // P and the rescale factor go back into positions of this wave's own
      // slot that only this wave reads (its rows)
      float *slot = &red[wave][0][0] + e_off;
      slot[0] = __uint_as_float(pack_bf16x2(p0f, p1f));
      if (j2 == 0) slot[1] = sc;            // vocab 1 of the row: group 0, element 1
    }
    __syncthreads();

    // ---- z += P E over this wave's slice
    bf16x8 pa[2];
    float scl[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int M = rb * 16 + (lane & 15);          // A-operand row of this lane
      const int q = lane >> 4;
      const float *rowp = &red[M >> 2][M][0];
      const uint32_t w4[4] = {__float_as_uint(rowp[rswz(M, q) * 4]),
                              __float_as_uint(rowp[rswz(M, q) * 4 + 2]),
                              __float_as_uint(rowp[rswz(M, 4 + q) * 4]),
                              __float_as_uint(rowp[rswz(M, 4 + q) * 4 + 2])};
      pa[rb] = *reinterpret_cast<const bf16x8 *>(w4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int mr = rb * 16 + q * 4 + i;         // z-accumulator rows of this lane
        scl[rb][i] = red[mr >> 2][mr][rswz(mr, 0) * 4 + 1];
      }
    }
    __syncthreads();   // every wave holds its P and factors: the slots may be reused
    bool rescale = false;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) rescale |= scl[rb][i] != 1.f;
    if (__builtin_amdgcn_ballot_w64(rescale)) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) zacc[rb][nb][i] *= scl[rb][i];
    }
    // transposed read addresses: source lane supplies row 4 (lane>>4) + ((lane&15)>>2)
    // (+16 for the second read), columns 16 (nb&1) + 4 (lane&3) of chunk nb>>1
    const int tr_row = 4 * (lane >> 4) + ((lane & 15) >> 2);
    const int tr_col = 4 * (lane & 3);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int c = nb >> 1;
      const int col = 16 * (nb & 1) + tr_col;             // element column within the chunk
      s16x4 lo, hi;
      {
        const int r = tr_row;
        const uint16_t *p = chunk(c) + r * 32 + swz(r, col >> 3) * 8 + (col & 7);
        lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p);
      }
      {
        const int r = tr_row + 16;
        const uint16_t *p = chunk(c) + r * 32 + swz(r, col >> 3) * 8 + (col & 7);
        hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p);
      }
      bf16x8 eb;
      {
        const s16x4 ls = lo, hs = hi;
        const uint16_t w8[8] = {(uint16_t)ls[0], (uint16_t)ls[1], (uint16_t)ls[2], (uint16_t)ls[3],
                                (uint16_t)hs[0], (uint16_t)hs[1], (uint16_t)hs[2], (uint16_t)hs[3]};
        eb = *reinterpret_cast<const bf16x8 *>(w8);
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        zacc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[rb], eb, zacc[rb][nb], 0, 0, 0);
      if ((nb & 1) && more) dma_chunk(tile + 1, c);
    }
  }

  // ---- write the split partials
  if (rvalid && j2 == 0) {
    RowPartial p;
    p.m = m_ref;
    p.l = l_run;
    p.best = best_v;
    p.arg = best_i;
    a.part[static_cast<int64_t>(split) * a.R + grow] = p;
  }
  float *zs = a.zpart + static_cast<int64_t>(split) * a.R * a.d;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = row0 + rb * 16 + (lane >> 4) * 4 + i;
      if (r >= a.R) continue;
      float *zr = zs + static_cast<int64_t>(r) * a.d + dcol0 + (lane & 15);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) zr[nb * 16] = zacc[rb][nb][i];
    }
}

}  // namespace v2

struct Plan {
  int MT, DW, splits, tps;
  bool v2;
};

bool plan(const Shape &s, Plan &p) {
  if (s.V % VT != 0 || s.d % (NW * 32) != 0) return false;
  p.DW = s.d / NW;
  if (p.DW != 32 && p.DW != 64 && p.DW != 128 && p.DW != 256 && p.DW != 352) return false;
  p.v2 = p.DW <= 256 && s.V % v2::VT == 0;
  p.MT = p.v2 ? v2::MT : ((p.DW <= 256) ? 32 : 16);
  const int vt = p.v2 ? v2::VT : VT;
  const int rblocks = (s.R() + p.MT - 1) / p.MT;
  const int tiles = s.V / vt;
  int want = (256 + rblocks - 1) / rblocks;
  if (want < 1) want = 1;
  if (want > 64) want = 64;          // the combine kernel merges at most 64 splits
  if (want > tiles) want = tiles;
  p.tps = (tiles + want - 1) / want;
  p.splits = (tiles + p.tps - 1) / p.tps;
  return true;
}

}  // namespace

bool lmhead_supported(const Shape &s) {
  Plan p;
  return plan(s, p);
}

int lmhead_splits(const Shape &s) {
  Plan p;
  return plan(s, p) ? p.splits : 0;
}

size_t lmhead_workspace_bytes(const Shape &s) {
  Plan p;
  if (!plan(s, p)) return 0;
  const size_t R = static_cast<size_t>(s.R());
  return p.splits * R * (sizeof(RowPartial) + static_cast<size_t>(s.d) * sizeof(float));
}

hipError_t launch_lmhead_bf16(const uint16_t *h1, const uint16_t *E, const int32_t *x_t,
                              const StepParams *prm, const Shape &s, uint64_t seed, void *work,
                              float *p0, hipStream_t st) {
  Plan p;
  if (!plan(s, p)) return hipErrorInvalidValue;
  if (s.R() == 0) return hipSuccess;
  LmArgs a;
  a.h1 = h1; a.E = E; a.x_t = x_t; a.prm = prm; a.p0 = p0;
  a.R = s.R(); a.C = s.C; a.d = s.d; a.V = s.V;
  a.splits = p.splits; a.tiles_per_split = p.tps;
  a.k0 = static_cast<uint32_t>(seed); a.k1 = static_cast<uint32_t>(seed >> 32);
  a.part = static_cast<RowPartial *>(work);
  a.zpart = reinterpret_cast<float *>(static_cast<char *>(work) +
                                      static_cast<size_t>(p.splits) * s.R() * sizeof(RowPartial));
  const int rblocks = (s.R() + p.MT - 1) / p.MT;
  if (p.v2) {
    const dim3 grid(rblocks * p.splits);
    switch (p.DW) {
      case 32: hipLaunchKernelGGL(v2::lmhead_v2_kernel<32>, grid, dim3(512), 0, st, a, rblocks); break;
      case 64: hipLaunchKernelGGL(v2::lmhead_v2_kernel<64>, grid, dim3(512), 0, st, a, rblocks); break;
      case 128: hipLaunchKernelGGL(v2::lmhead_v2_kernel<128>, grid, dim3(512), 0, st, a, rblocks); break;
      case 256: hipLaunchKernelGGL(v2::lmhead_v2_kernel<256>, grid, dim3(512), 0, st, a, rblocks); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  dim3 grid(rblocks, p.splits);
#define DG_LM(MT_, DW_)                                                                  \
  if (p.MT == MT_ && p.DW == DW_) {                                                      \
    hipLaunchKernelGGL((lmhead_kernel<MT_, DW_>), grid, dim3(512), 0, st, a);            \
    return hipGetLastError();                                                            \
  }
  DG_LM(32, 32) DG_LM(32, 64) DG_LM(32, 128) DG_LM(32, 256) DG_LM(16, 352)
#undef DG_LM
  return hipErrorInvalidValue;
}

}  // namespace dg
