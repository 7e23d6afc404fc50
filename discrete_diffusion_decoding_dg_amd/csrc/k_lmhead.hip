// Fused LM head, softmax statistics, self-conditioning z and Gumbel-max draw
// on bf16 MFMA. The C x V logits never leave the chip.
//
// DiffusionGemma Technical Report (hyper.ai summary), Method, three-line
// update: p0 = Softmax(L / tau), z = FFW(p0 E) (FFW read as identity, E the
// tied embedding), x_{t-dt} ~ Step(x_t, p0). For a row that resamples
// (Bernoulli u < lambda, decided before the vocabulary loop) the Step draw is
// argmax_v s_v + G_v with Philox Gumbel noise; kept rows skip the noise.
//
// Decomposition. A block owns MT canvas rows and a contiguous vocabulary
// range (one "split", a multiple of four 16-id tiles); its 8 waves split the
// model width d into slices of DW columns. Each wave keeps its h1 slice (the
// B operand of the scores) and its z slice (fp32 accumulators) in registers
// for the whole vocabulary range. Per 16-id vocabulary tile:
//   1. S^T[v, m] over the wave's slice with v_mfma_f32_16x16x32_bf16 (E tile
//      as A operand from LDS, h1 from registers);
//   2. the 8 slice partials meet in LDS; one lane per (row, id) finishes the
//      score s = S / tau, keeps its own running Gumbel argmax and softmax sum,
//      and writes P = exp2(s log2e - m_ref) as bf16. The row reference m_ref
//      moves only when a score exceeds it by more than 2^8 (checked with one
//      wave ballot; the row maximum is reduced only then), so z is rarely
//      rescaled and no per-tile row reduction is needed;
//   3. z[m, slice] += P[m, tile] E[tile, slice] with v_mfma_f32_32x32x16_bf16
//      (16x16x16 for 16-row blocks), E read transposed from LDS by
//      ds_read_b64_tr_b16.
// E is read from a tile-major copy made when the model is created: each
// 16-id x 32-column chunk is 1 KB contiguous, already in the chunk's LDS
// order, so every load reads whole cache lines. With two tile buffers
// (d <= 2048) tiles reach LDS by direct global->LDS loads, and the next tile
// is requested in two halves between the contractions (after the scores and
// after the epilogue), where its LDS writes do not compete with the
// contractions' LDS reads. Where only one buffer fits (d = 2816) each wave
// loads its slice of the next tile into registers a whole tile ahead; the
// score contraction takes its A operand from those registers, which are then
// written to LDS once for the transposed reads of the z contraction.
//
// Gumbel noise: the Philox block of lane (row, position j) for the aligned
// group of four tiles g holds the noise of ids 64 g + j + {0, 16, 32, 48}, one
// word per tile (counter layout of the library), so a lane evaluates one
// Philox block per four tiles and turns one word into noise per tile, ahead of
// the epilogue that uses it.
//
// A block ends by writing (m, l, best, arg) per row and its unnormalised z
// slice partials; the combine kernel merges the splits.
#include <type_traits>

#include "dg_device.hpp"
#include "dg_kernels.hpp"

namespace dg {
namespace {

constexpr int NW = 8;            // waves per block, one d-slice each
constexpr int VT = 16;           // vocabulary ids per tile
constexpr int kLdsBudget = 160 * 1024;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;   // log2 units

struct LmArgs {
  const uint16_t *h1, *E;
  const int32_t *x_t;
  const StepParams *prm;
  RowPartial *part;   // [splits][R]
  uint16_t *zpart;    // [splits][R][d] bf16: the split's sum of p E
  float *p0;          // optional [R][V] raw scaled logits
  int R, C, d, V, splits, tiles_per_split;
  uint32_t k0, k1;
};

// s_waitcnt with only one counter constrained (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8; the others at their maxima). The
// builtin is visible to the compiler's own wait insertion.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");   // no memory access moves across the wait
}
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
  asm volatile("" ::: "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt_le_rt(int n) {
  if constexpr (N > 0) {
    if (n >= N) {
      wait_vmcnt<N>();
      return;
    }
    wait_vmcnt_le_rt<N - 1>(n);
  } else {
    wait_vmcnt<0>();
  }
}

// ---- LDS layouts (XOR swizzles found by exhaustive search; each keeps its
// access patterns free of bank conflicts for 32 and for 64 banks of 4 bytes)
//
// E chunk: 16 vocabulary rows x 32 columns, 64 bytes per row in four 16-byte
// pieces; logical piece p of row r sits at p ^ eswz(r). Patterns: the direct
// global->LDS write (contiguous), 16-byte A-operand reads of 16 rows, and the
// transposed 8-byte reads of 4-row groups.
__device__ __forceinline__ int eswz(int r) {
  return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 2) ^ (r >> 3)) & 1) << 1);
}
__device__ __forceinline__ int eoff(int r, int col) {   // byte offset of (row, column)
  return r * 64 + (((col >> 3) ^ eswz(r)) << 4) + (col & 7) * 2;
}
// Reduction buffer: per wave [MT rows][16 ids] fp32, 64 bytes per row; the
// 16-byte group g of row r sits at g ^ rswz(r). Patterns: 16-byte partial
// writes (16 rows x 4 groups) and 4-byte epilogue reads (4 rows x 16 ids).
__device__ __forceinline__ int rswz(int r) { return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1); }
__device__ __forceinline__ int roff(int r, int v) {     // float index
  return r * 16 + (((v >> 2) ^ rswz(r)) << 2) + (v & 3);
}
// P buffer: [MT rows][16 ids] bf16, 32 bytes per row. For 32-row blocks the
// A operand is 16 bytes (8 ids) per lane: halves swizzled by r2 ^ r3. For
// 16-row blocks it is 8 bytes: quarters swizzled by (r2, r3).
template <int MT>
__device__ __forceinline__ int poff(int r, int v) {     // byte offset
  if constexpr (MT == 32)
    return r * 32 + ((((v >> 3) ^ ((r >> 2) ^ (r >> 3))) & 1) << 4) + (v & 7) * 2;
  else
    return r * 32 + (((v >> 2) ^ (((r >> 2) & 1) | (((r >> 3) & 1) << 1))) << 3) + (v & 3) * 2;
}

// Direct global -> LDS load of 16 bytes per lane: lane i's bytes land at
// lds + 16 i (lds must be wave-uniform). Issued through inline asm so that
// the compiler does not add conservative waits before unrelated LDS reads;
// every read of the loaded data is preceded by an explicit vmcnt wait
// instead. The instruction has no register result: its address registers
// are read at issue. `base` is wave-uniform (scalar registers), `voff` the
// lane's byte offset from it.
__device__ __forceinline__ void lds_dma16(const void *base, uint32_t voff, void *lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t *)lds)));
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

__device__ __forceinline__ uint32_t sel4(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, int k) {
  return (k & 2) ? ((k & 1) ? w3 : w2) : ((k & 1) ? w1 : w0);
}

// ENT: entropy-bounded step (every row draws; entropy statistics kept).
template <int MT, int DW, int NBUF, bool ENT>
__global__ void __launch_bounds__(512) lmhead_kernel(LmArgs a, int rblocks) {
  static_assert(MT == 16 || MT == 32, "row block");
  static_assert(DW % 32 == 0, "slice width");
  static_assert(NW == 8, "the epilogue sums eight slice partials");
  constexpr int NKS = DW / 32;              // 32-column chunks per slice
  constexpr int RB = MT / 16;               // 16-row blocks of the score contraction
  constexpr int CHUNK_B = VT * 64;          // bytes per chunk
  constexpr int SLICE_B = NKS * CHUNK_B;    // bytes per wave slice and buffer
  constexpr int NZ = (MT == 32) ? NKS : 2 * NKS;   // z accumulator blocks
  typedef typename std::conditional<MT == 32, f32x16, f32x4>::type zacc_t;
  static_assert(NBUF * NW * SLICE_B + NW * MT * VT * 4 + MT * VT * 2 + MT * 4 + 16 <= kLdsBudget, "LDS");

  __shared__ __attribute__((aligned(16))) uint8_t Es[NBUF * NW * SLICE_B];
  __shared__ __attribute__((aligned(16))) float red[NW * MT * VT];
  __shared__ __attribute__((aligned(16))) uint8_t Pb[MT * VT * 2];
  __shared__ __attribute__((aligned(16))) float scl[MT];
  __shared__ int last_resc;

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

  const int total_tiles = a.V / VT;
  const int t_begin = split * a.tiles_per_split;
  int t_end = t_begin + a.tiles_per_split;
  if (t_end > total_tiles) t_end = total_tiles;

  auto ebuf = [&](int tile) -> uint8_t * {
    return Es + ((NBUF == 2 ? (tile & 1) : 0) * NW + wave) * SLICE_B;
  };
  // one direct load fills a chunk: lane i copies bytes [16 i, 16 i + 16) of
  // the chunk's 1 KB in the tile-major copy (see relayout_kernel) to the
  // same bytes of the chunk in LDS
  const uint32_t dma_off = static_cast<uint32_t>(lane * 16);
  auto dma_chunk = [&](int tile, int c) {
    const uint16_t *tb = a.E + (static_cast<int64_t>(tile) * (a.d / 32) + dcol0 / 32 + c) * (VT * 32);
    lds_dma16(tb, dma_off, ebuf(tile) + c * CHUNK_B);
  };
  // one buffer: the wave's slice of the next tile waits in registers, lane l
  // holding row l & 15, piece l >> 4 of each chunk (the score A operand)
  const uint32_t a_off = static_cast<uint32_t>(eoff(lane & 15, 8 * (lane >> 4)));
  bf16x8 ereg[NBUF == 1 ? NKS : 1];
  auto load_tile_regs = [&](int tile) __attribute__((always_inline)) {
    const uint8_t *tb = reinterpret_cast<const uint8_t *>(
        a.E + (static_cast<int64_t>(tile) * (a.d / 32) + dcol0 / 32) * (VT * 32));
#pragma unroll
    for (int c = 0; c < NKS; ++c) ereg[c] = *reinterpret_cast<const bf16x8 *>(tb + c * CHUNK_B + a_off);
  };
  // a CU accepts about 71 B/clk of load requests and a wave waits at issue
  // until its own are taken: the epilogue waves (16-row blocks: 16 x 16
  // lanes are four waves) request the next tile before the barrier, the
  // others while the epilogue runs, so that each burst is half a tile
  constexpr int EPW = MT * VT / 64;
  if (t_begin < t_end) {
    if constexpr (NBUF == 2) {
#pragma unroll
      for (int c = 0; c < NKS; ++c) dma_chunk(t_begin, c);
    } else {
      load_tile_regs(t_begin);
    }
  }

  // h1 slice as the B operand of S^T: lane holds canvas row 16 rb + (lane & 15),
  // columns dcol0 + 32 c + 8 (lane >> 4) + [0, 8)
  bf16x8 hreg[RB][NKS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = row0 + rb * 16 + (lane & 15);
    const uint16_t *hrow = a.h1 + static_cast<int64_t>(r) * a.d + dcol0 + (lane >> 4) * 8;
#pragma unroll
    for (int c = 0; c < NKS; ++c)
      hreg[rb][c] = (r < a.R) ? *reinterpret_cast<const bf16x8 *>(hrow + c * 32) : bf16x8{};
  }

  // epilogue role: thread tid < 16 MT owns row er = tid / 16 of the block and
  // position j of every tile (wave-uniform: 16 MT is a multiple of 64)
  const bool epi = tid < MT * VT;
  const int er = tid >> 4, j = lane & 15;
  const int grow = row0 + er;
  const bool rvalid = epi && grow < a.R;
  const int gb = rvalid ? grow / a.C : 0;
  const int gi = rvalid ? grow - gb * a.C : 0;
  const float inv_tau = rvalid ? a.prm[gb].inv_tau : 0.f;
  bool resample = false;
  if (rvalid) {
    if constexpr (ENT) {
      resample = true;
    } else {
      const u32x4 w = philox4x32_10(0u, static_cast<uint32_t>(gi), static_cast<uint32_t>(gb),
                                    kStreamBernoulli, a.k0, a.k1);
      resample = u01(w.x) < a.prm[gb].lam;
    }
  }
  float m_ref = -INFINITY, l_lane = 0.f, best_v = -INFINITY;
  int best_i = -1;
  // entropy statistics: sum of p (t - m_ref) and the plain argmax
  float s1_lane = 0.f, dbest_v = -INFINITY;
  int dbest_i = -1;
  uint32_t gw0 = 0, gw1 = 0, gw2 = 0, gw3 = 0;   // Philox words of the current group
  auto gumbel_block = [&](int tile) {
    const u32x4 w = philox4x32_10(static_cast<uint32_t>(16 * (tile >> 2) + j), static_cast<uint32_t>(gi),
                                  static_cast<uint32_t>(gb), kStreamGumbel, a.k0, a.k1);
    gw0 = w.x;
    gw1 = w.y;
    gw2 = w.z;
    gw3 = w.w;
  };
  float g_cur = 0.f;   // noise of id v0 + j of the current tile
  if (resample && t_begin < t_end) {
    gumbel_block(t_begin);
    g_cur = gumbel(sel4(gw0, gw1, gw2, gw3, t_begin & 3));
  }

  zacc_t zacc[NZ];
#pragma unroll
  for (int n = 0; n < NZ; ++n) zacc[n] = zacc_t{};
  if (tid == 0) last_resc = -1;
  // everything issued so far (the first tile, h1, step constants) has landed:
  // the loop below tracks only its own tile loads
  wait_vmcnt<0>();

  // transposed-read source addresses: lane S supplies 4 ids x 4 columns
  const int g4 = lane >> 4;
  const int tr_row = (MT == 32) ? 8 * (g4 >> 1) + ((lane & 15) >> 2) : 4 * g4 + ((lane & 15) >> 2);
  const int tr_col = (MT == 32) ? 16 * (g4 & 1) + 4 * (lane & 3) : 4 * (lane & 3);

  for (int tile = t_begin; tile < t_end; ++tile) {
    const int v0 = tile * VT;
    const bool more = tile + 1 < t_end;
    if (a.p0) wait_vmcnt<0>();   // checking mode: p0 stores share the counter
    // With two buffers the next tile streams into the other buffer in two
    // halves, one after the scores and one after the epilogue. Measured on the
    // 32-row blocks: issuing loads before or during either contraction (whose
    // LDS reads they compete with) costs 2-15 %, a single burst up to 35 %.
    // Each batch goes into the buffer of the previous tile, whose reads by
    // this wave's own z contraction have all returned (they fed its MFMAs).
    constexpr int kB1 = NKS / 2;   // chunk ranges [0,kB1) and [kB1,NKS)
    uint8_t *eb = ebuf(tile);

    // ---- S^T partial over this wave's slice (two accumulator sets break the
    // dependency chain of the 16-pass MFMAs)
    f32x4 sacc[2][RB];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sacc[s][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NKS; ++c) {
      bf16x8 ef;
      if constexpr (NBUF == 2) {
        // chunk c of this tile has landed once at most its NKS-1-c younger
        // siblings are outstanding (no load of the next tile is issued yet)
        wait_vmcnt_le_rt<63>(NKS - 1 - c);
        ef = *reinterpret_cast<const bf16x8 *>(eb + c * CHUNK_B + a_off);
      } else {
        ef = ereg[c];
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        sacc[c & 1][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ef, hreg[rb][c], sacc[c & 1][rb], 0, 0, 0);
    }
    // lane (q, n) of block rb holds row 16 rb + n, ids 4 q + [0, 4)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = rb * 16 + (lane & 15);
      const f32x4 s = sacc[0][rb] + sacc[1][rb];
      *reinterpret_cast<f32x4 *>(&red[wave * MT * VT + roff(r, 4 * (lane >> 4))]) = s;
    }
    if constexpr (NBUF == 2) {
      if (more) {
        wait_lgkm0();
#pragma unroll
        for (int c = 0; c < kB1; ++c) dma_chunk(tile + 1, c);
      }
    } else {
      // the buffer's previous contents fed this wave's own z contraction of
      // the previous tile, whose reads have all returned
#pragma unroll
      for (int c = 0; c < NKS; ++c)
        *reinterpret_cast<bf16x8 *>(eb + c * CHUNK_B + a_off) = ereg[c];
      if (more && wave < EPW) load_tile_regs(tile + 1);
    }
    __syncthreads();
    if constexpr (NBUF == 1) {
      if (more && wave >= EPW) load_tile_regs(tile + 1);
    }

    // ---- epilogue: one lane per (row er, id v0 + j)
    if (epi) {
      float pr[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) pr[w] = red[w * MT * VT + roff(er, j)];
      const float acc = ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
      const float s = acc * inv_tau;
      const int v = v0 + j;
      if (a.p0 && rvalid) a.p0[static_cast<int64_t>(grow) * a.V + v] = s;
      if (resample) {
        const float y = s + g_cur;
        if (y > best_v) {       // strict: the earlier (lower) id keeps a tie
          best_v = y;
          best_i = v;
        }
      }
      const float t2 = s * kLog2e;
      if constexpr (ENT) {
        if (rvalid && t2 > dbest_v) {   // strict: the earlier (lower) id keeps a tie
          dbest_v = t2;
          dbest_i = v;
        }
      }
      float sc = 1.f;
      if (__builtin_amdgcn_ballot_w64(t2 > m_ref + kRescaleSlack)) {
        float mx = t2;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        if (mx > m_ref + kRescaleSlack) {
          sc = __builtin_amdgcn_exp2f(m_ref - mx);   // 0 on the first tile
          // re-reference sum p (t - m): every p scales by sc and every
          // (t - m) grows by m_old - m_new
          if constexpr (ENT) s1_lane = (l_lane > 0.f) ? sc * (s1_lane + (m_ref - mx) * l_lane) : 0.f;
          m_ref = mx;
        }
        if (__builtin_amdgcn_ballot_w64(sc != 1.f) && lane == 0) last_resc = tile;
      }
      // hardware exp2: results below 2^-126 flush to zero, far below what a
      // bf16 probability times an embedding row can contribute to z
      const float p = __builtin_amdgcn_exp2f(t2 - m_ref);
      l_lane = l_lane * sc + p;
      if constexpr (ENT) s1_lane += p * (t2 - m_ref);
      *reinterpret_cast<uint16_t *>(Pb + poff<MT>(er, j)) = f32_to_bf16(p);
      if (j == 0) scl[er] = sc;
    }
    if constexpr (NBUF == 2) {
      if (more) {
#pragma unroll
        for (int c = kB1; c < NKS; ++c) dma_chunk(tile + 1, c);
      }
    }
    __syncthreads();

    // ---- z += P E over this wave's slice. The P operand and the first
    // chunk's E operand are requested before the rescale flag is examined
    // (independent LDS reads: one round trip instead of two)
    constexpr int NPF = (MT == 32) ? 1 : 0;   // prefetched chunks
    bf16x8 pa32{};
    bf16x8 bpf[NPF > 0 ? NPF : 1];
    if constexpr (MT == 32) {
      pa32 = *reinterpret_cast<const bf16x8 *>(Pb + poff<MT>(lane & 31, 8 * (lane >> 5)));
#pragma unroll
      for (int c = 0; c < NPF; ++c) {
        const uint8_t *ch = eb + c * CHUNK_B;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(ch + eoff(tr_row, tr_col)));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(ch + eoff(tr_row + 4, tr_col)));
        bpf[c] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
    if (__builtin_amdgcn_readfirstlane(last_resc) == tile) {
      if constexpr (MT == 32) {
        f32x4 f[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) f[jj] = *reinterpret_cast<const f32x4 *>(&scl[8 * jj + 4 * (lane >> 5)]);
#pragma unroll
        for (int n = 0; n < NZ; ++n)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int i = 0; i < 4; ++i) zacc[n][4 * jj + i] *= f[jj][i];
      } else {
        const f32x4 f = *reinterpret_cast<const f32x4 *>(&scl[4 * (lane >> 4)]);
#pragma unroll
        for (int n = 0; n < NZ; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) zacc[n][i] *= f[i];
      }
    }
    if constexpr (MT == 32) {
      // A operand: row lane & 31, ids 8 (lane >> 5) + [0, 8)
      const bf16x8 pa = pa32;
#pragma unroll
      for (int c = 0; c < NKS; ++c) {
        bf16x8 b;
        if (c < NPF) {
          b = bpf[c < NPF ? c : 0];
        } else {
          const uint8_t *ch = eb + c * CHUNK_B;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4 *)(ch + eoff(tr_row, tr_col)));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4 *)(ch + eoff(tr_row + 4, tr_col)));
          // B operand: column lane & 31 of the chunk, ids 8 (lane >> 5) + [0, 8)
          b = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
        zacc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, b, zacc[c], 0, 0, 0);
      }
    } else {
      // A operand: row lane & 15, ids 4 (lane >> 4) + [0, 4)
      const s16x4 pa = *reinterpret_cast<const s16x4 *>(Pb + poff<MT>(lane & 15, 4 * (lane >> 4)));
#pragma unroll
      for (int n = 0; n < NZ; ++n) {
        const uint8_t *ch = eb + (n >> 1) * CHUNK_B;
        // B operand: column 16 (n & 1) + (lane & 15) of the chunk, ids 4 (lane >> 4) + [0, 4)
        const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(ch + eoff(tr_row, 16 * (n & 1) + tr_col)));
        zacc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, b, zacc[n], 0, 0, 0);
      }
    }
    // noise of the next tile, off the epilogue's path
    if (resample && more) {
      const int nt = tile + 1;
      if ((nt & 3) == 0) gumbel_block(nt);
      g_cur = gumbel(sel4(gw0, gw1, gw2, gw3, nt & 3));
    }
  }

  // ---- write the split partials
  if (epi) {
    float l = l_lane, bv = best_v, s1 = s1_lane, dv = dbest_v;
    int bi = best_i, di = dbest_i;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      l += __shfl_xor(l, o, 64);
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi))) {
        bv = ov;
        bi = oi;
      }
      if constexpr (ENT) {
        s1 += __shfl_xor(s1, o, 64);
        const float odv = __shfl_xor(dv, o, 64);
        const int odi = __shfl_xor(di, o, 64);
        if (odi >= 0 && (di < 0 || odv > dv || (odv == dv && odi < di))) {
          dv = odv;
          di = odi;
        }
      }
    }
    if (rvalid && j == 0) {
      RowPartial p;
      p.m = m_ref;
      p.l = l;
      p.best = bv;
      p.arg = bi;
      p.s1 = ENT ? s1 : 0.f;
      p.dbest = ENT ? dv : -INFINITY;
      p.darg = ENT ? di : -1;
      p.pad = 0;
      a.part[static_cast<int64_t>(split) * a.R + grow] = p;
    }
  }
  // z partials travel in bf16: each is rescaled and summed in fp32 by the
  // merge, and the result is rounded to bf16 anyway; half the bytes of fp32
  uint16_t *zs = a.zpart + static_cast<int64_t>(split) * a.R * a.d;
  if constexpr (MT == 32) {
    // accumulator element 4 jj + i: row 8 jj + 4 (lane >> 5) + i, column lane & 31
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row0 + 8 * jj + 4 * (lane >> 5) + i;
        if (r >= a.R) continue;
        uint16_t *zr = zs + static_cast<int64_t>(r) * a.d + dcol0 + (lane & 31);
#pragma unroll
        for (int c = 0; c < NKS; ++c) zr[32 * c] = f32_to_bf16(zacc[c][4 * jj + i]);
      }
  } else {
    // accumulator element i: row 4 (lane >> 4) + i, column lane & 15
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = row0 + 4 * (lane >> 4) + i;
      if (r >= a.R) continue;
      uint16_t *zr = zs + static_cast<int64_t>(r) * a.d + dcol0 + (lane & 15);
#pragma unroll
      for (int n = 0; n < NZ; ++n) zr[16 * n] = f32_to_bf16(zacc[n][i]);
    }
  }
}

// Tile-major copy of E for the LM head: chunk q = tile * (d / 32) + c (ids
// 16 tile + [0, 16), columns 32 c + [0, 32)) is 1 KB at Et + 512 q, and its
// 16-byte piece i holds row i / 4, logical piece (i % 4) ^ eswz(i / 4), the
// LDS order of the chunk (the swizzle is an XOR, so its own inverse). One
// wave per chunk.
__global__ void __launch_bounds__(256) relayout_kernel(const uint16_t *__restrict__ E, int d,
                                                       int64_t chunks, uint16_t *__restrict__ Et) {
  const int lane = threadIdx.x & 63;
  const int64_t q = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (q >= chunks) return;
  const int cpr = d / 32;                          // chunks per 16-id tile
  const int64_t tile = q / cpr;
  const int c = static_cast<int>(q - tile * cpr);
  const int row = lane >> 2, lp = (lane & 3) ^ eswz(row);
  const uint4 v = *reinterpret_cast<const uint4 *>(E + (tile * VT + row) * d + 32 * c + 8 * lp);
  *reinterpret_cast<uint4 *>(Et + q * (VT * 32) + 8 * lane) = v;
}

struct Plan {
  int MT, DW, NBUF, splits, tps;
};

size_t lds_bytes(int MT, int DW, int nbuf) {
  return static_cast<size_t>(nbuf) * NW * (DW / 32) * VT * 64 + NW * MT * VT * 4 + MT * VT * 2 + MT * 4 + 16;
}

bool plan(const Shape &s, Plan &p) {
  if (s.V % VT != 0 || s.d % (NW * 32) != 0) return false;
  p.DW = s.d / NW;
  // registers hold h1 and z for the block's rows: 32 rows up to 256 columns
  // per wave, 16 rows for 352
  if (p.DW != 32 && p.DW != 64 && p.DW != 128 && p.DW != 256 && p.DW != 352) return false;
  p.MT = (p.DW <= 256) ? 32 : 16;
  p.NBUF = lds_bytes(p.MT, p.DW, 2) <= static_cast<size_t>(kLdsBudget) ? 2 : 1;
  const int rblocks = (s.R() + p.MT - 1) / p.MT;
  const int tiles = s.V / VT;
  int want = (256 + rblocks - 1) / rblocks;
  if (want < 1) want = 1;
  if (want > 64) want = 64;          // the combine kernel merges at most 64 splits
  int tps = (tiles + want - 1) / want;
  tps = (tps + 3) & ~3;              // splits start on four-tile Gumbel groups
  p.tps = tps;
  p.splits = (tiles + tps - 1) / tps;
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
  return p.splits * R * (sizeof(RowPartial) + static_cast<size_t>(s.d) * sizeof(uint16_t));
}

size_t lmhead_copy_bytes(const Shape &s) {
  return static_cast<size_t>(s.V) * s.d * sizeof(uint16_t);
}

hipError_t launch_lmhead_relayout(const uint16_t *E, const Shape &s, uint16_t *Et, hipStream_t st) {
  Plan p;
  if (!plan(s, p)) return hipErrorInvalidValue;
  const int64_t chunks = static_cast<int64_t>(s.V / VT) * (s.d / 32);
  const int64_t blocks = (chunks + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(relayout_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st, E, s.d,
                     chunks, Et);
  return hipGetLastError();
}

hipError_t launch_lmhead_bf16(const uint16_t *h1, const uint16_t *E, const int32_t *x_t,
                              const StepParams *prm, const Shape &s, uint64_t seed, void *work,
                              float *p0, bool entropy, hipStream_t st) {
  Plan p;
  if (!plan(s, p)) return hipErrorInvalidValue;
  if (s.R() == 0) return hipSuccess;
  LmArgs a;
  a.h1 = h1; a.E = E; a.x_t = x_t; a.prm = prm; a.p0 = p0;
  a.R = s.R(); a.C = s.C; a.d = s.d; a.V = s.V;
  a.splits = p.splits; a.tiles_per_split = p.tps;
  a.k0 = static_cast<uint32_t>(seed); a.k1 = static_cast<uint32_t>(seed >> 32);
  a.part = static_cast<RowPartial *>(work);
  a.zpart = reinterpret_cast<uint16_t *>(static_cast<char *>(work) +
                                      static_cast<size_t>(p.splits) * s.R() * sizeof(RowPartial));
  const int rblocks = (s.R() + p.MT - 1) / p.MT;
  const dim3 grid(rblocks * p.splits);
#define DG_LM(MT_, DW_, NB_)                                                                     \
  if (p.MT == MT_ && p.DW == DW_ && p.NBUF == NB_) {                                             \
    if (entropy)                                                                                 \
      hipLaunchKernelGGL((lmhead_kernel<MT_, DW_, NB_, true>), grid, dim3(512), 0, st, a, rblocks); \
    else                                                                                         \
      hipLaunchKernelGGL((lmhead_kernel<MT_, DW_, NB_, false>), grid, dim3(512), 0, st, a, rblocks); \
    return hipGetLastError();                                                                    \
  }
  DG_LM(32, 32, 2) DG_LM(32, 64, 2) DG_LM(32, 128, 2) DG_LM(32, 256, 2) DG_LM(16, 352, 1)
#undef DG_LM
  return hipErrorInvalidValue;
}

}  // namespace dg
