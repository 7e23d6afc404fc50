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

struct Plan {
  int MT, DW, splits, tps;
};

bool plan(const Shape &s, Plan &p) {
  if (s.V % VT != 0 || s.d % (NW * 32) != 0) return false;
  p.DW = s.d / NW;
  if (p.DW != 32 && p.DW != 64 && p.DW != 128 && p.DW != 256 && p.DW != 352) return false;
  p.MT = (p.DW <= 256) ? 32 : 16;
  const int rblocks = (s.R() + p.MT - 1) / p.MT;
  const int tiles = s.V / VT;
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
  dim3 grid((s.R() + p.MT - 1) / p.MT, p.splits);
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
