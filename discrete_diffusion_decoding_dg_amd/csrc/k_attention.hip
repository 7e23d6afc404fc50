// Fused prefix + canvas attention on bf16 MFMA (flash style, split-KV).
//
// DiffusionGemma Technical Report (hyper.ai summary), Method, three-stage
// generation pipeline and decoder equation: the canvas attends
// bidirectionally to itself and cross-attends to the prompt KV cache. Read
// here as one joint, unmasked softmax over [prefix ; canvas] keys, scale
// 1/sqrt(hd), query head h using kv head h / G.
//
// One block = 32 NWA query rows of one kv head (the G query heads of a kv
// head share its K/V, so their rows are stacked: row qr = (h - g G) C + i),
// NWA waves of 32 rows: 8 waves, or 4 where 8-wave blocks would leave half
// the CUs idle (short caches at batch 1), which doubles the blocks. Keys
// stream through LDS in tiles of 64 by direct global->LDS
// loads, NS tiles in flight. Per tile and wave:
//   S^T[key, query] = K Q^T with v_mfma_f32_32x32x16_bf16 (K from LDS as the
//   A operand, the wave's Q rows held in registers as B). A lane then holds 16
//   keys of one query, and the k-slot order of the O^T += V^T P^T contraction
//   is chosen to match, so P goes from the score accumulators to the B
//   operand without leaving registers; V is read transposed from LDS
//   (ds_read_b64_tr_b16) as the A operand. Accumulating O^T gives each lane
//   one query and four consecutive head columns per accumulator group.
// In 8-wave blocks the younger wave of each SIMD runs one tile behind in its
// softmax and P V (skewed schedule), so that the SIMD's two waves are not in
// the same phase (MFMA or VALU) at the same time.
// The online softmax runs in log2 units with a reference maximum that moves
// only when a score exceeds it by more than 2^8 (one ballot per tile; the
// rare move rescales O), so P <= 2^8 and no per-tile O rescale is needed.
// Long key ranges are split across blocks; partial (m, l, O) are merged by a
// second kernel.
//
// LDS layout of a K or V tile: piece-major, [16-byte piece p of the row]
// [64 keys], key k of piece p stored at slot k ^ 4 (p & 3). One direct load
// fills one piece for all 64 keys; the XOR keeps the score-operand reads (32
// keys of one piece) and the transposed 4-key reads of V free of bank
// conflicts for 32 and 64 banks, for any head dimension.
#include "dg_device.hpp"
#include "dg_kernels.hpp"

namespace dg {
namespace {

constexpr int BK = 64;              // keys per tile
constexpr int kLdsBudget = 160 * 1024;
constexpr float kSlack = 8.0f;      // log2 units

template <int HD>
struct Geo {
  static constexpr int HDP = (HD + 31) / 32 * 32;   // padded head dim
  static constexpr int NPC = HDP / 8;               // 16-byte pieces per row incl. padding
  static constexpr int NPR = HD / 8;                // pieces carrying data
  static constexpr int KS = (HD + 15) / 16;         // k-steps of the score contraction (data columns only)
  static constexpr int NB = HDP / 32;               // 32-column blocks of O
  static constexpr int TILE_B = NPC * BK * 16;      // bytes per tensor and stage
  static constexpr int NS = (2 * TILE_B * 4 <= kLdsBudget) ? 4 : 3;   // stages
  static constexpr int NDMA = 2 * NPR;              // direct loads per tile (K and V)
  static_assert(2 * TILE_B * NS <= kLdsBudget, "LDS");
};

struct AttnArgs {
  const uint16_t *q, *k, *v, *Kp, *Vp;
  uint16_t *o;
  uint16_t *opart;   // [splits][R][Hq][hd] unnormalised bf16, when splits > 1
  float2 *ml;     // [splits][R][Hq] (m, l), log2 units
  int B, C, P, Pst, Hq, Hkv, G, splits, tiles_per_split;   // Pst: cache rows per (b, g)
  int qblocks;                                              // query blocks per (b, g, split)
  int causal;                                               // canvas key j visible to query i iff j <= i
  float scale_log2;   // log2(e) / sqrt(hd)
};

__device__ __forceinline__ int kslot(int key, int piece) { return key ^ (4 * (piece & 3)); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}
// wait until at most k * STEP vector-memory operations are outstanding, for a
// runtime k in [0, K]: K + 1 compile-time cases
template <int STEP, int K>
__device__ __forceinline__ void wait_vmcnt_steps(int k) {
  if constexpr (K > 0) {
    if (k >= K) {
      wait_vmcnt<K * STEP>();
      return;
    }
    wait_vmcnt_steps<STEP, K - 1>(k);
  } else {
    wait_vmcnt<0>();
  }
}

// Direct global -> LDS load of 16 bytes per lane from a per-lane 64-bit
// address; lane i's bytes land at LDS byte address lds + 16 i (lds
// wave-uniform). Inline asm
// keeps the compiler from adding waits before unrelated LDS reads; reads of
// the loaded data follow an explicit vmcnt wait and a barrier. The
// instruction has no register result: its address registers are read at
// issue.
__device__ __forceinline__ void lds_dma16_va(const void *src, uint32_t lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  const uint64_t addr = reinterpret_cast<uint64_t>(src);
  uint32_t saved;
  // M0 is reserved by the compiler: keep its value across the block
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

// The same load with a wave-uniform 64-bit base (scalar registers) and a
// 32-bit per-lane byte offset: cheaper to form than a per-lane address.
__device__ __forceinline__ void lds_dma16_sa(const void *base, uint32_t voff, uint32_t lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  // readfirstlane returns a signed int: go through uint32_t so that the low
  // half is zero-extended
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

// CAUSAL: the causal encoder pass (canvas query i sees canvas keys 0..i).
// LB: the launch bound the registers are allocated for. 4-wave blocks run
// one wave per SIMD, but given 512 registers the compiler parks the score
// accumulators in AGPRs and copies them to VGPRs and back every tile; at head
// dims up to 128 they are compiled as for 8-wave blocks (256 registers, all
// of them VGPRs) and launched with 256 threads.
template <int HD, int NWA, bool CAUSAL, int LB = (NWA == 4 && HD <= 128) ? 512 : NWA * 64>
__global__ void __launch_bounds__(LB) attn_fwd_kernel(AttnArgs a) {
  constexpr int BQ = NWA * 32;                   // query rows per block
  using G_ = Geo<HD>;
  constexpr int HDP = G_::HDP, NPC = G_::NPC, NPR = G_::NPR, KS = G_::KS, NB = G_::NB;
  constexpr int TILE_B = G_::TILE_B, NS = G_::NS, NDMA = G_::NDMA;
  // With 8 waves only the first four issue the direct loads: each SIMD's
  // older wave, which otherwise waits at the barrier for the younger one,
  // takes the stall of issuing them (a CU accepts about 71 B/clk of load
  // requests, and the issuing wave waits until its own are taken)
  constexpr int LW = (NWA == 8) ? 4 : NWA;       // waves that issue loads
  constexpr int MAXL = (NDMA + LW - 1) / LW;     // loads per loading wave and tile, at most
  __shared__ __attribute__((aligned(16))) uint8_t stage_mem[NS * 2 * TILE_B];
  // LDS byte address of the stage (the M0 operand of the direct loads)
  const uint32_t stage_lds = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t *)stage_mem));

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // XCD-aware order: the hardware deals consecutive blocks round-robin to the
  // 8 XCDs; the logical id gives each XCD a contiguous run, so the query
  // blocks that share a kv head and key range (consecutive ids) share an L2
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int nqb = a.qblocks;
  const int qb = bid % nqb;
  const int rest = bid / nqb;
  const int g = rest % a.Hkv, bz = rest / a.Hkv;
  const int b = bz / a.splits, split = bz - b * a.splits;
  const int GC = a.G * a.C;
  const int Lk = a.P + a.C;
  const int qcols = a.Hq * HD;

  // padding pieces (head dims that are not a multiple of 32) are read by the
  // P V contraction into discarded O columns (and, for a head dim that ends in
  // half a 16-wide k-step, by the score contraction against zero Q): they must
  // be finite
  if constexpr (NPC > NPR) {
    for (int c = tid; c < NS * 2 * (NPC - NPR) * BK; c += NWA * 64) {
      const int key = c % BK, rest = c / BK;
      const int p = NPR + rest % (NPC - NPR), tens = rest / (NPC - NPR);
      *reinterpret_cast<uint4 *>(stage_mem + tens * TILE_B + p * BK * 16 + key * 16) = make_uint4(0, 0, 0, 0);
    }
  }

  // this wave's 32 query rows; lane holds query lane & 31 and the k-slots
  // 8 (lane >> 5) + [0, 8) of every 16-wide step
  const int hl = lane >> 5;
  const int qr = qb * BQ + wave * 32 + (lane & 31);
  const bool qvalid = qr < GC;
  const int qh = qvalid ? g * a.G + qr / a.C : 0;
  const int qi = qvalid ? qr % a.C : 0;
  bf16x8 qreg[KS];
  {
    const uint16_t *qrow = a.q + (static_cast<int64_t>(b) * a.C + qi) * qcols + qh * HD;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int e = ks * 16 + hl * 8;
      qreg[ks] = (qvalid && e < HD) ? *reinterpret_cast<const bf16x8 *>(qrow + e) : bf16x8{};
    }
  }

  const int64_t kvp_base = (static_cast<int64_t>(b) * a.Hkv + g) * a.Pst * HD;
  const int64_t kvc_base = (static_cast<int64_t>(b) * a.Hkv + g) * a.C * HD;
  const int tile0 = split * a.tiles_per_split;
  const int total_tiles = (Lk + BK - 1) / BK;
  int tile_end = tile0 + a.tiles_per_split;
  if (tile_end > total_tiles) tile_end = total_tiles;

  // direct loads of one tile: load u in [0, NDMA) fills piece u % NPR of K
  // (u < NPR) or of V; wave w < LW issues loads w, w + LW, ...
  constexpr int MINL = NDMA / LW;                // loads per loading wave and tile, at least
  // byte offset of this lane's key row inside a tile, for each piece phase
  uint32_t koff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) koff[q] = static_cast<uint32_t>((lane ^ (4 * q)) * HD * 2);
  auto issue_tile = [&](int tile) {
    const uint32_t st = stage_lds + (tile % NS) * 2 * TILE_B;
    const int j0 = tile * BK;
    if (j0 + BK <= a.P || (j0 >= a.P && j0 + BK <= Lk)) {
      // the whole tile lies in the prefix or in the canvas: one uniform base
      const bool pre = j0 + BK <= a.P;
      const uint16_t *kb = pre ? a.Kp + kvp_base + static_cast<int64_t>(j0) * HD
                               : a.k + kvc_base + static_cast<int64_t>(j0 - a.P) * HD;
      const uint16_t *vb = pre ? a.Vp + kvp_base + static_cast<int64_t>(j0) * HD
                               : a.v + kvc_base + static_cast<int64_t>(j0 - a.P) * HD;
#pragma unroll
      for (int n = 0; n < MAXL; ++n) {
        const int u = wave + n * LW;
        if (wave < LW && u < NDMA) {
          const int tensor = u >= NPR, p = tensor ? u - NPR : u;
          lds_dma16_sa((tensor ? vb : kb) + p * 8, koff[p & 3], st + tensor * TILE_B + p * BK * 16);
        }
      }
      return;
    }
#pragma unroll
    for (int n = 0; n < MAXL; ++n) {
      const int u = wave + n * LW;
      if (wave < LW && u < NDMA) {
        const int tensor = u >= NPR, p = tensor ? u - NPR : u;
        // lane i fills slot i of the piece: key i ^ 4 (p & 3) of the tile,
        // clamped to the last key (keys past the end are masked in the scores)
        int j = tile * BK + kslot(lane, p);
        if (j > Lk - 1) j = Lk - 1;
        const uint16_t *src = (j < a.P)
                                  ? (tensor ? a.Vp : a.Kp) + kvp_base + static_cast<int64_t>(j) * HD + p * 8
                                  : (tensor ? a.v : a.k) + kvc_base + static_cast<int64_t>(j - a.P) * HD + p * 8;
        lds_dma16_va(src, st + tensor * TILE_B + p * BK * 16);
      }
    }
  };
  // the Q loads must have landed before the first direct load is issued: the
  // compiler does not see the inline-asm loads, and with Q still pending it
  // would wait for every outstanding load (vmcnt 0) before the first score
  // MFMA of each tile, which would drain the pipeline every tile
  wait_vmcnt<0>();

  // byte offsets of this lane's K fragments inside a stage: piece p = 2 ks +
  // hl starts at p * BK * 16, and its key slot XOR 4 (p & 3) takes one value
  // for even ks and one for odd ks; key block mb adds 32 keys (bit 5 of the
  // key, which the XOR leaves alone). Everything else is an immediate.
  const uint32_t koff_e = hl * BK * 16 + ((lane & 31) ^ (4 * (hl & 3))) * 16;
  const uint32_t koff_o = hl * BK * 16 + ((lane & 31) ^ (4 * ((2 + hl) & 3))) * 16;
  f32x16 oacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x16{};
  float m_ref = -INFINITY, l_lane = 0.f;
  const int g4 = lane >> 4;
  const int tr_key = 4 * (g4 >> 1) + ((lane & 15) >> 2);
  const int tr_col = 16 * (g4 & 1) + 4 * (lane & 3);

  // ---- S^T for the 64 keys of a tile (two 32-key blocks, one accumulator
  // chain each) into sacc
  f32x16 sacc[2];
  auto scores = [&](const int tile) __attribute__((always_inline)) {
    const uint8_t *Ks = stage_mem + (tile % NS) * 2 * TILE_B;
    const uint8_t *Ke = Ks + koff_e, *Ko = Ks + koff_o;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) sacc[mb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(((ks & 1) ? Ko : Ke) + ks * 2 * BK * 16 + mb * 32 * 16);
        sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qreg[ks], sacc[mb], 0, 0, 0);
      }
    }
  };

  // ---- the scores of a tile (in sacc) to P: row max, lazy rescale of O and
  // l, exponentials
  bf16x8 pa[4];
  auto softmax = [&](const int tile) __attribute__((always_inline)) {
    // element e = 4 jj + i of block mb: key 32 mb + 8 jj + 4 hl + i of this
    // tile. Raw scores here; the scale folds into the exponent below
    // (scale_log2 > 0, so the max commutes with it).
    float sv[2][16];
    float rmax = -INFINITY;
    const int kv0 = tile * BK;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sv[mb][e] = sacc[mb][e];
    if (kv0 + BK > Lk) {   // the last, partial tile: keys past the end drop out
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (kv0 + mb * 32 + 8 * (e >> 2) + 4 * hl + (e & 3) >= Lk) sv[mb][e] = -INFINITY;
    }
    if constexpr (CAUSAL) {
      // canvas keys after this lane's query drop out (a whole tile may, for
      // some queries of the block)
      if (kv0 + BK > a.P + qi + 1) {
        const int last = a.P + qi;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (kv0 + mb * 32 + 8 * (e >> 2) + 4 * hl + (e & 3) > last) sv[mb][e] = -INFINITY;
      }
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) rmax = fmaxf(rmax, sv[mb][e]);
    rmax = fmaxf(rmax, __shfl_xor(rmax, 32, 64));   // both halves of the query
    const float tmax = rmax * a.scale_log2;
    if (__builtin_amdgcn_ballot_w64(tmax > m_ref + kSlack)) {
      float alpha = 1.f;
      if (tmax > m_ref + kSlack) {
        alpha = __builtin_amdgcn_exp2f(m_ref - tmax);   // 0 on the first tile
        m_ref = tmax;
      }
      l_lane *= alpha;
      // every O^T element of this lane belongs to its own query
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[nb][e] *= alpha;
    }
    // P in the k-slot order of the PV contraction: for the 16-key step kk
    // (block mb = kk / 2, half kk2 = kk % 2) the A operand is elements
    // 8 kk2 .. 8 kk2 + 7 of block mb, i.e. keys 16 kk + 4 hl + [0, 4) and
    // 16 kk + 8 + 4 hl + [0, 4)
    float psum = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float p = __builtin_amdgcn_exp2f(fmaf(sv[mb][e], a.scale_log2, -m_ref));
        // no visible key yet for this query (whole tiles masked): nothing adds
        if constexpr (CAUSAL) p = (m_ref == -INFINITY) ? 0.f : p;
        psum += p;
        pa[2 * mb + (e >> 3)][e & 7] = static_cast<__bf16>(p);
      }
    l_lane += psum;
  };

  // ---- O += P V; the B operand of column block nb and step kk is read
  // transposed: source lane S supplies key 16 kk + 4 (g / 2) + j (+ 8 for
  // the second read) at columns 32 nb + 16 (g % 2) + 4 q, with g = S / 16,
  // j = (S % 16) / 4, q = S % 4
  auto pv = [&](const int tile) __attribute__((always_inline)) {
    const uint8_t *Vs = stage_mem + (tile % NS) * 2 * TILE_B + TILE_B;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = 32 * nb + tr_col;
        const int p = col >> 3;
        const uint8_t *pb = Vs + p * BK * 16 + ((col & 7) >> 2) * 8;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(pb + kslot(16 * kk + tr_key, p) * 16));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(pb + kslot(16 * kk + 8 + tr_key, p) * 16));
        const bf16x8 vb = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        // O^T = V^T P^T: the V fragment as A operand (row = head column), P
        // as B operand (column = query); the k slots are the same as for P V
        oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb, pa[kk], oacc[nb], 0, 0, 0);
      }
    }
  };

  // Skewed schedule (8-wave blocks, at least four stages): waves w and w + 4
  // share a SIMD, and phases in which both issue only MFMAs or only VALU work
  // add up. The older waves take each tile in order (scores, softmax, P V);
  // the younger ones run the softmax and P V of the previous tile and then the
  // scores of this one, so each SIMD's two waves are in different phases for
  // two of the three. The younger waves read V of tile - 1 during step tile:
  // after the barrier of step tile the free stage is that of tile - 2, which
  // takes tile + NS - 2 (two tiles of lookahead instead of three).
  constexpr bool SKEW = NWA == 8 && NS >= 4;
  constexpr int AHEAD = SKEW ? NS - 2 : NS - 1;   // tiles issued ahead of the current one, plus it
  const bool lag = SKEW && wave >= 4;
  for (int t = tile0; t < tile_end && t < tile0 + AHEAD; ++t) issue_tile(t);
  // this wave's loads of `tile` have landed once at most those of the tiles
  // issued after it are outstanding (MINL or MINL + 1 per tile for a loading
  // wave, none for the others; MINL is the safe bound); the barrier makes
  // every wave's loads visible and frees the stage read last. Both loops
  // pass the same barriers.
  auto top = [&](const int tile) __attribute__((always_inline)) {
    int after = tile_end - 1 - tile;
    if (after > AHEAD - 1) after = AHEAD - 1;
    wait_vmcnt_steps<MINL, AHEAD - 1>(after);
    __syncthreads();
    if (tile + AHEAD < tile_end) issue_tile(tile + AHEAD);
  };
  if (!lag) {
    for (int tile = tile0; tile < tile_end; ++tile) {
      top(tile);
      scores(tile);
      softmax(tile);
      pv(tile);
    }
  } else if (tile0 < tile_end) {
    top(tile0);
    scores(tile0);
    for (int tile = tile0 + 1; tile < tile_end; ++tile) {
      top(tile);
      softmax(tile - 1);
      pv(tile - 1);
      scores(tile);
    }
    softmax(tile_end - 1);
    pv(tile_end - 1);
  }

  // ---- normalise, or write the split partials. oacc[nb] holds O^T: lane
  // (hl, q) has query q = lane & 31 and, per element 4 jj + i, head column
  // 32 nb + 8 jj + 4 hl + i. Each wave stages its 32 x HD tile row-major in
  // the (now free) K/V stages and then stores whole 16-byte pieces of its
  // rows, consecutive lanes along a row: every store instruction writes
  // contiguous row segments instead of a 16-byte piece in each of 32 rows.
  {
    const float l_q = l_lane + __shfl_xor(l_lane, 32, 64);   // lanes q and q + 32 hold query q
    const bool whole = a.splits == 1;
    const float sc = whole ? 1.f / l_q : 1.f;
    // staged row pitch: 16 bytes of padding put consecutive rows four banks apart
    constexpr int OP = HDP + 8;
    static_assert(NWA * 32 * OP * 2 <= NS * 2 * TILE_B, "output staging fits in the stages");
    __syncthreads();   // every wave has finished reading the K/V stages
    uint16_t *stg = reinterpret_cast<uint16_t *>(stage_mem) + wave * 32 * OP;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int col = 32 * nb + 8 * jj + 4 * hl;
        if (HDP == HD || col < HD) {
          // partials travel in bf16: the merge rescales and sums them in
          // fp32 and rounds the result to bf16 anyway; half the bytes of fp32
          uint2 v;
          v.x = pack_bf16x2(oacc[nb][4 * jj] * sc, oacc[nb][4 * jj + 1] * sc);
          v.y = pack_bf16x2(oacc[nb][4 * jj + 2] * sc, oacc[nb][4 * jj + 3] * sc);
          *reinterpret_cast<uint2 *>(stg + (lane & 31) * OP + col) = v;
        }
      }
    const int row0 = qb * BQ + wave * 32;
    constexpr int PPR = HD / 8;   // 16-byte pieces per row
    for (int e = lane; e < 32 * PPR; e += 64) {
      const int q = e / PPR, pc = e - q * PPR;
      const int row = row0 + q;
      if (row < GC) {
        const int h = g * a.G + row / a.C, ii = row % a.C;
        const int64_t r = static_cast<int64_t>(b) * a.C + ii;
        uint16_t *dst = whole ? a.o + r * qcols + h * HD
                              : a.opart + ((split * (static_cast<int64_t>(a.B) * a.C) + r) * a.Hq + h) * HD;
        *reinterpret_cast<uint4 *>(dst + 8 * pc) = *reinterpret_cast<const uint4 *>(stg + q * OP + 8 * pc);
      }
    }
    const int row = row0 + (lane & 31);
    if (!whole && hl == 0 && row < GC) {
      const int h = g * a.G + row / a.C, ii = row % a.C;
      const int64_t r = static_cast<int64_t>(b) * a.C + ii;
      a.ml[(split * (static_cast<int64_t>(a.B) * a.C) + r) * a.Hq + h] = make_float2(m_ref, l_q);
    }
  }
}

// o[r, h, e] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s. One thread
// per four consecutive columns of a row (hd % 4 == 0), looping over the
// splits: the general case (more than 16 splits, head dims that are not a
// multiple of 8, or partials of 2 GiB and more).
__global__ void __launch_bounds__(256) attn_combine_kernel(const uint16_t *__restrict__ opart,
                                                           const float2 *__restrict__ ml,
                                                           int splits, int64_t rows, int hd,
                                                           uint16_t *__restrict__ o) {
  const int q4 = hd / 4;
  const int64_t total = rows * hd, total4 = rows * q4;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < total4;
       t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t row = t / q4;
    const int64_t idx = row * hd + 4 * (t - row * q4);
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, ml[s * rows + row].x);
    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
    float den = 0.f;
    for (int s = 0; s < splits; ++s) {
      const float2 v = ml[s * rows + row];
      const float w = exp2f(v.x - M);
      const uint2 xb = *reinterpret_cast<const uint2 *>(opart + s * total + idx);
      num.x += w * __uint_as_float(xb.x << 16);
      num.y += w * __uint_as_float(xb.x & 0xFFFF0000u);
      num.z += w * __uint_as_float(xb.y << 16);
      num.w += w * __uint_as_float(xb.y & 0xFFFF0000u);
      den += w * v.y;
    }
    const float inv = 1.f / den;
    uint2 out;
    out.x = pack_bf16x2(num.x * inv, num.y * inv);
    out.y = pack_bf16x2(num.z * inv, num.w * inv);
    *reinterpret_cast<uint2 *>(o + idx) = out;
  }
}

// hd % 8 == 0, at most 16 splits: one thread per 8 consecutive columns of a
// (row, head) pair, NP == splits (exact instantiations). The (m, l) records
// are requested first, then the partials as 16-byte buffer loads (one
// resource, the split offset in a scalar register), all before the maximum;
// up to 128 registers per lane keep every load in flight.
template <int NP>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 4))) attn_combine_wide_kernel(const uint16_t *__restrict__ opart,
                                                                const float2 *__restrict__ ml,
                                                                int64_t rows, int hd,
                                                                uint16_t *__restrict__ o) {
  // rows * hd < 2^30 (the launch checks that all splits hold < 2^31 bytes)
  const int q8 = hd / 8;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= static_cast<int>(rows) * q8) return;
  const int row = t / q8;
  const int idx = row * hd + 8 * (t - row * q8);
  const int sbytes = static_cast<int>(rows) * hd * 2;
  const __amdgpu_buffer_rsrc_t pr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(opart), 0, NP * sbytes, kBufferFlags);
  float2 mr[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) mr[k] = ml[k * rows + row];   // < 2^31 records
  uint32_t xr[NP][4];
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(pr, idx * 2, k * sbytes, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) xr[k][i] = v[i];
  }
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < NP; ++k) M = fmaxf(M, mr[k].x);
  float num[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) num[i] = 0.f;
  float den = 0.f;
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const float w = exp2f(mr[k].x - M);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      num[2 * i] += w * __uint_as_float(xr[k][i] << 16);
      num[2 * i + 1] += w * __uint_as_float(xr[k][i] & 0xFFFF0000u);
    }
    den += w * mr[k].y;
  }
  const float inv = 1.f / den;
  uint4 out;
  out.x = pack_bf16x2(num[0] * inv, num[1] * inv);
  out.y = pack_bf16x2(num[2] * inv, num[3] * inv);
  out.z = pack_bf16x2(num[4] * inv, num[5] * inv);
  out.w = pack_bf16x2(num[6] * inv, num[7] * inv);
  *reinterpret_cast<uint4 *>(o + idx) = out;
}

void plan_waves(const Shape &s, int nwa, int &splits, int &tps) {
  const int bq = nwa * 32;
  const int tiles = (s.P + s.C + BK - 1) / BK;
  const int base = ((s.G() * s.C + bq - 1) / bq) * s.Hkv * s.B;
  int want = (256 + base - 1) / base;   // one block per CU fills the chip
  if (want < 1) want = 1;
  if (want > tiles) want = tiles;
  tps = (tiles + want - 1) / want;
  // a one-tile split costs more in partials (and their merge) than it gains
  if (tps < 2) tps = 2;
  splits = (tiles + tps - 1) / tps;
}

// 8-wave blocks unless they leave half the CUs idle; then 4-wave blocks
void plan(const Shape &s, int &nwa, int &splits, int &tps) {
  nwa = 8;
  plan_waves(s, 8, splits, tps);
  const int blocks = ((s.G() * s.C + 255) / 256) * s.Hkv * s.B * splits;
  if (blocks <= 128) {
    nwa = 4;
    plan_waves(s, 4, splits, tps);
  }
}

}  // namespace

int attention_splits(const Shape &s) {
  int nwa, sp, tps;
  plan(s, nwa, sp, tps);
  return sp;
}

size_t attention_workspace_bytes(const Shape &s) {
  const int sp = attention_splits(s);
  if (sp <= 1) return 0;
  const size_t rows = static_cast<size_t>(s.R()) * s.Hq;
  return sp * rows * (s.hd * sizeof(uint16_t) + sizeof(float2));
}

hipError_t launch_attention_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                 const uint16_t *Kp, const uint16_t *Vp, const Shape &s,
                                 void *work, uint16_t *o, hipStream_t st) {
  if (s.R() == 0) return hipSuccess;
  AttnArgs a;
  a.q = q; a.k = k; a.v = v; a.Kp = Kp; a.Vp = Vp; a.o = o;
  a.B = s.B; a.C = s.C; a.P = s.P; a.Pst = s.pstride(); a.Hq = s.Hq; a.Hkv = s.Hkv; a.G = s.G();
  a.causal = s.causal;
  int nwa = 8;
  plan(s, nwa, a.splits, a.tiles_per_split);
  const size_t rows = static_cast<size_t>(s.R()) * s.Hq;
  a.opart = static_cast<uint16_t *>(work);
  a.ml = reinterpret_cast<float2 *>(static_cast<char *>(work) +
                                    static_cast<size_t>(a.splits) * rows * s.hd * sizeof(uint16_t));
  a.scale_log2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(s.hd)));
  const int bq = nwa * 32;
  a.qblocks = (s.G() * s.C + bq - 1) / bq;
  const int64_t nblocks = static_cast<int64_t>(a.qblocks) * s.Hkv * s.B * a.splits;
  if (nblocks > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid(static_cast<uint32_t>(nblocks));
#define DG_ATT(HD_)                                                                       \
  case HD_:                                                                               \
    if (s.causal) {                                                                       \
      if (nwa == 8)                                                                       \
        hipLaunchKernelGGL((attn_fwd_kernel<HD_, 8, true>), grid, dim3(512), 0, st, a);   \
      else                                                                                \
        hipLaunchKernelGGL((attn_fwd_kernel<HD_, 4, true>), grid, dim3(256), 0, st, a);   \
    } else if (nwa == 8) {                                                                \
      hipLaunchKernelGGL((attn_fwd_kernel<HD_, 8, false>), grid, dim3(512), 0, st, a);    \
    } else {                                                                              \
      hipLaunchKernelGGL((attn_fwd_kernel<HD_, 4, false>), grid, dim3(256), 0, st, a);    \
    }                                                                                     \
    break;
  switch (s.hd) {
    DG_ATT(64) DG_ATT(128) DG_ATT(176)
    default: return hipErrorInvalidValue;
  }
#undef DG_ATT
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  const bool fits31 = static_cast<int64_t>(a.splits) * rows * s.hd * 2 < (int64_t{1} << 31);
  const bool aligned16 = ((reinterpret_cast<uintptr_t>(a.opart) | reinterpret_cast<uintptr_t>(o)) & 15) == 0;
  if (s.hd % 8 == 0 && a.splits <= 16 && fits31 && aligned16) {
    const int64_t total8 = static_cast<int64_t>(rows) * (s.hd / 8);
    const dim3 wgrid(static_cast<uint32_t>((total8 + 255) / 256));
#define DG_ACW(NP_)                                                                              \
  case NP_:                                                                                      \
    hipLaunchKernelGGL(attn_combine_wide_kernel<NP_>, wgrid, dim3(256), 0, st, a.opart, a.ml,    \
                       static_cast<int64_t>(rows), s.hd, o);                                     \
    return hipGetLastError();
    switch (a.splits) {
      DG_ACW(2) DG_ACW(3) DG_ACW(4) DG_ACW(5) DG_ACW(6) DG_ACW(7) DG_ACW(8) DG_ACW(9) DG_ACW(10)
      DG_ACW(11) DG_ACW(12) DG_ACW(13) DG_ACW(14) DG_ACW(15) DG_ACW(16)
      default: break;
    }
#undef DG_ACW
  }
  const int64_t total4 = static_cast<int64_t>(rows) * (s.hd / 4);
  int64_t blocks = (total4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  const dim3 cgrid(static_cast<uint32_t>(blocks));
  hipLaunchKernelGGL(attn_combine_kernel, cgrid, dim3(256), 0, st, a.opart, a.ml, a.splits,
                     static_cast<int64_t>(rows), s.hd, o);
  return hipGetLastError();
}

}  // namespace dg
