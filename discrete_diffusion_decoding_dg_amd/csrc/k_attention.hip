// Fused prefix + canvas attention on bf16 MFMA (flash style, split-KV).
//
// DiffusionGemma Technical Report (hyper.ai summary), Method, three-stage
// generation pipeline and decoder equation: the canvas attends
// bidirectionally to itself and cross-attends to the prompt KV cache. Read
// here as one joint, unmasked softmax over [prefix ; canvas] keys, scale
// 1/sqrt(hd), query head h using kv head h / G.
//
// One block = 64 query rows of one kv head (the G query heads of a kv head
// share its K/V, so their rows are stacked: row qr = (h - g G) C + i), 4 waves
// of 16 rows. K/V tiles of 64 keys are staged in LDS: K row-major, V
// transposed ([e][key]) so both MFMA operands read contiguous 8-byte runs.
// Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_bf16:
// a lane then owns one query row and 4 consecutive keys per 16-key block,
// which is exactly the A-operand layout of O += P V (keys as K dimension), so
// P never leaves registers. The online softmax runs in log2 units.
// Long key ranges are split across blocks; partial (m, l, O) are merged by a
// second kernel.
#include "dg_device.hpp"
#include "dg_kernels.hpp"

namespace dg {
namespace {

constexpr int BQ = 64;     // query rows per block
constexpr int BKV = 64;    // keys per tile
constexpr int VT_PITCH = BKV + 8;

constexpr int round_up32(int x) { return (x + 31) / 32 * 32; }

struct AttnArgs {
  const uint16_t *q, *k, *v, *Kp, *Vp;
  uint16_t *o;
  float *opart;   // [splits][R][Hq][hd] unnormalised, when splits > 1
  float2 *ml;     // [splits][R][Hq] (m, l), log2 units
  int B, C, P, Hq, Hkv, G, splits, tiles_per_split;
  float scale_log2;   // log2(e) / sqrt(hd)
};

template <int HD>
__global__ void __launch_bounds__(256) attn_fwd_kernel(AttnArgs a) {
  constexpr int HDP = round_up32(HD);
  constexpr int KPITCH = HDP + 8;
  constexpr int NKS = HDP / 32;     // k-steps of the score contraction
  constexpr int NB = HD / 16;       // 16-wide column blocks of O
  constexpr int CH = HD / 8;        // 16-byte chunks per key row

  __shared__ __attribute__((aligned(16))) uint16_t Ks[BKV * KPITCH];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[HD * VT_PITCH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qb = blockIdx.x, g = blockIdx.y;
  const int b = blockIdx.z / a.splits, split = blockIdx.z - b * a.splits;
  const int GC = a.G * a.C;
  const int Lk = a.P + a.C;
  const int64_t hd_stride = HD;
  const int qcols = a.Hq * HD;

  // zero the score padding columns once (never written by tile loads)
  if (HDP > HD) {
    for (int c = tid; c < BKV * (HDP - HD); c += 256) {
      const int key = c / (HDP - HD), col = HD + c % (HDP - HD);
      Ks[key * KPITCH + col] = 0;
    }
  }

  // this lane's query row in the S^T layout
  const int qr = qb * BQ + wave * 16 + (lane & 15);
  const bool qvalid = qr < GC;
  const int qh = qvalid ? g * a.G + qr / a.C : 0;
  const int qi = qvalid ? qr % a.C : 0;
  bf16x8 qreg[NKS];
  {
    const uint16_t *qrow = a.q + (static_cast<int64_t>(b) * a.C + qi) * qcols + qh * hd_stride;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int e = ks * 32 + (lane >> 4) * 8;
      if (qvalid && e < HD)
        qreg[ks] = *reinterpret_cast<const bf16x8 *>(qrow + e);
      else
        qreg[ks] = bf16x8{};
    }
  }

  f32x4 oacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int64_t kvp_base = (static_cast<int64_t>(b) * a.Hkv + g) * a.P * hd_stride;
  const int64_t kvc_base = (static_cast<int64_t>(b) * a.Hkv + g) * a.C * hd_stride;
  const int tile0 = split * a.tiles_per_split;
  const int total_tiles = (Lk + BKV - 1) / BKV;
  int tile_end = tile0 + a.tiles_per_split;
  if (tile_end > total_tiles) tile_end = total_tiles;

  for (int tile = tile0; tile < tile_end; ++tile) {
    const int kv0 = tile * BKV;
    __syncthreads();   // previous tile fully consumed
    for (int c = tid; c < BKV * CH; c += 256) {
      const int key = c / CH, col = (c - key * CH) * 8;
      const int j = kv0 + key;
      uint4 kk = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (j < a.P) {
        kk = *reinterpret_cast<const uint4 *>(a.Kp + kvp_base + j * hd_stride + col);
        vv = *reinterpret_cast<const uint4 *>(a.Vp + kvp_base + j * hd_stride + col);
      } else if (j < Lk) {
        kk = *reinterpret_cast<const uint4 *>(a.k + kvc_base + (j - a.P) * hd_stride + col);
        vv = *reinterpret_cast<const uint4 *>(a.v + kvc_base + (j - a.P) * hd_stride + col);
      }
      *reinterpret_cast<uint4 *>(&Ks[key * KPITCH + col]) = kk;
      const uint32_t w4[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        Vt[(col + 2 * t) * VT_PITCH + key] = static_cast<uint16_t>(w4[t] & 0xFFFFu);
        Vt[(col + 2 * t + 1) * VT_PITCH + key] = static_cast<uint16_t>(w4[t] >> 16);
      }
    }
    __syncthreads();

    // S^T for 4 blocks of 16 keys: lane owns query row (lane & 15) and keys
    // 16 kb + 4 (lane >> 4) + [0, 4)
    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t *krow = &Ks[(kb * 16 + (lane & 15)) * KPITCH + (lane >> 4) * 8];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(krow + ks * 32);
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qreg[ks], s[kb], 0, 0, 0);
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = kv0 + kb * 16 + (lane >> 4) * 4 + r;
        const float val = (j < Lk) ? s[kb][r] * a.scale_log2 : -INFINITY;
        s[kb][r] = val;
        tmax = fmaxf(tmax, val);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = exp2f(m_run - m_new);   // 0 on the first tile
    float psum = 0.f;
    bf16x8 pa[2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = exp2f(s[kb][r] - m_new);
        psum += p[r];
      }
      // keys 16 kb + 4 (lane>>4) + r map to k-slots 8 (lane>>4) + 4 (kb & 1) + r
#pragma unroll
      for (int r = 0; r < 4; ++r) pa[kb >> 1][(kb & 1) * 4 + r] = static_cast<__bf16>(p[r]);
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;

    // O rows in the C layout are 4 (lane >> 4) + i; their alpha lives in lane row
    float arow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) arow[i] = __shfl(alpha, (lane >> 4) * 4 + i, 64);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[nb][i] *= arow[i];
      const uint16_t *vrow = &Vt[(nb * 16 + (lane & 15)) * VT_PITCH + (lane >> 4) * 4];
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const uint2 lo = *reinterpret_cast<const uint2 *>(vrow + ks2 * 32);
        const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + ks2 * 32 + 16);
        const uint4 w = make_uint4(lo.x, lo.y, hi.x, hi.y);
        const bf16x8 vb = *reinterpret_cast<const bf16x8 *>(&w);
        oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[ks2], vb, oacc[nb], 0, 0, 0);
      }
    }
  }

  // epilogue: lane holds O[row 4 (lane>>4) + i][col 16 nb + (lane & 15)]
  float lrow[4], mrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lrow[i] = __shfl(l_run, (lane >> 4) * 4 + i, 64);
    mrow[i] = __shfl(m_run, (lane >> 4) * 4 + i, 64);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = qb * BQ + wave * 16 + (lane >> 4) * 4 + i;
    if (row >= GC) continue;
    const int h = g * a.G + row / a.C, ii = row % a.C;
    const int64_t r = static_cast<int64_t>(b) * a.C + ii;
    if (a.splits == 1) {
      const float inv = 1.f / lrow[i];
      uint16_t *orow = a.o + r * qcols + h * hd_stride;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) orow[nb * 16 + (lane & 15)] = f32_to_bf16(oacc[nb][i] * inv);
    } else {
      const int64_t R = static_cast<int64_t>(a.B) * a.C;
      float *prow = a.opart + ((split * R + r) * a.Hq + h) * hd_stride;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) prow[nb * 16 + (lane & 15)] = oacc[nb][i];
      if ((lane & 15) == 0) a.ml[(split * R + r) * a.Hq + h] = make_float2(mrow[i], lrow[i]);
    }
  }
}

// ---------------------------------------------------------------------------
// Second version: K and V tiles stay row-major in LDS (rows padded so that the
// 16-row operand reads of K and the 4-row transposed reads of V hit distinct
// banks), V reaches the O contraction through ds_read_b64_tr_b16, and the
// next tile is fetched into registers while the current one is computed.
template <int HD> struct AttnPitch;
template <> struct AttnPitch<64> { static constexpr int K = 72, V = 80; };
template <> struct AttnPitch<128> { static constexpr int K = 136, V = 144; };
template <> struct AttnPitch<176> { static constexpr int K = 200, V = 208; };

template <int HD>
__global__ void __launch_bounds__(256) attn_fwd_v2_kernel(AttnArgs a) {
  constexpr int HDP = round_up32(HD);
  constexpr int KP = AttnPitch<HD>::K, VP = AttnPitch<HD>::V;
  static_assert(KP >= HDP, "score operand reads stay inside a K row");
  constexpr int NKS = HDP / 32;
  constexpr int NB = HD / 16;
  constexpr int CH = HD / 8;                       // 16-byte chunks per key row
  constexpr int PER = (BKV * CH + 255) / 256;      // chunks per thread per tile and tensor
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BKV * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[BKV * VP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qb = blockIdx.x, g = blockIdx.y;
  const int b = blockIdx.z / a.splits, split = blockIdx.z - b * a.splits;
  const int GC = a.G * a.C;
  const int Lk = a.P + a.C;
  const int64_t hd_stride = HD;
  const int qcols = a.Hq * HD;

  if (KP > HD)   // pad columns of K are read (against zero q) and must be finite
    for (int c = tid; c < BKV * (KP - HD); c += 256)
      Ks[(c / (KP - HD)) * KP + HD + c % (KP - HD)] = 0;

  const int qr = qb * BQ + wave * 16 + (lane & 15);
  const bool qvalid = qr < GC;
  const int qh = qvalid ? g * a.G + qr / a.C : 0;
  const int qi = qvalid ? qr % a.C : 0;
  bf16x8 qreg[NKS];
  {
    const uint16_t *qrow = a.q + (static_cast<int64_t>(b) * a.C + qi) * qcols + qh * hd_stride;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int e = ks * 32 + (lane >> 4) * 8;
      qreg[ks] = (qvalid && e < HD) ? *reinterpret_cast<const bf16x8 *>(qrow + e) : bf16x8{};
    }
  }

  f32x4 oacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int64_t kvp_base = (static_cast<int64_t>(b) * a.Hkv + g) * a.P * hd_stride;
  const int64_t kvc_base = (static_cast<int64_t>(b) * a.Hkv + g) * a.C * hd_stride;
  const int tile0 = split * a.tiles_per_split;
  const int total_tiles = (Lk + BKV - 1) / BKV;
  int tile_end = tile0 + a.tiles_per_split;
  if (tile_end > total_tiles) tile_end = total_tiles;

  uint4 kreg[PER], vreg[PER];
  auto fetch = [&](int tile) {
    const int kv0 = tile * BKV;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + 256 * u;
      uint4 kk = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (c < BKV * CH) {
        const int key = c / CH, col = (c - key * CH) * 8;
        const int j = kv0 + key;
        if (j < a.P) {
          kk = *reinterpret_cast<const uint4 *>(a.Kp + kvp_base + j * hd_stride + col);
          vv = *reinterpret_cast<const uint4 *>(a.Vp + kvp_base + j * hd_stride + col);
        } else if (j < Lk) {
          kk = *reinterpret_cast<const uint4 *>(a.k + kvc_base + (j - a.P) * hd_stride + col);
          vv = *reinterpret_cast<const uint4 *>(a.v + kvc_base + (j - a.P) * hd_stride + col);
        }
      }
      kreg[u] = kk;
      vreg[u] = vv;
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + 256 * u;
      if (c < BKV * CH) {
        const int key = c / CH, col = (c - key * CH) * 8;
        *reinterpret_cast<uint4 *>(&Ks[key * KP + col]) = kreg[u];
        *reinterpret_cast<uint4 *>(&Vs[key * VP + col]) = vreg[u];
      }
    }
  };

  if (tile0 < tile_end) {
    fetch(tile0);
    __syncthreads();            // pad zeroing done before rows land
    stash();
    if (tile0 + 1 < tile_end) fetch(tile0 + 1);
    __syncthreads();
  }
  // transposed-read source address of this lane (see the LM head for the
  // lane mapping of ds_read_b64_tr_b16)
  const int tr_row = 4 * (lane >> 4) + ((lane & 15) >> 2);
  const int tr_col = 4 * (lane & 3);

  for (int tile = tile0; tile < tile_end; ++tile) {
    const int kv0 = tile * BKV;
    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t *krow = &Ks[(kb * 16 + (lane & 15)) * KP + (lane >> 4) * 8];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(krow + ks * 32);
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qreg[ks], s[kb], 0, 0, 0);
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = kv0 + kb * 16 + (lane >> 4) * 4 + r;
        const float val = (j < Lk) ? s[kb][r] * a.scale_log2 : -INFINITY;
        s[kb][r] = val;
        tmax = fmaxf(tmax, val);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = exp2f(m_run - m_new);
    float psum = 0.f;
    bf16x8 pa[2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2f(s[kb][r] - m_new);
        psum += p;
        pa[kb >> 1][(kb & 1) * 4 + r] = static_cast<__bf16>(p);
      }
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    float arow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) arow[i] = __shfl(alpha, (lane >> 4) * 4 + i, 64);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[nb][i] *= arow[i];
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const int col = nb * 16 + tr_col;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)&Vs[(ks2 * 32 + tr_row) * VP + col]);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)&Vs[(ks2 * 32 + 16 + tr_row) * VP + col]);
        const uint16_t w8[8] = {(uint16_t)lo[0], (uint16_t)lo[1], (uint16_t)lo[2], (uint16_t)lo[3],
                                (uint16_t)hi[0], (uint16_t)hi[1], (uint16_t)hi[2], (uint16_t)hi[3]};
        const bf16x8 vb = *reinterpret_cast<const bf16x8 *>(w8);
        oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[ks2], vb, oacc[nb], 0, 0, 0);
      }
    }
    if (tile + 1 < tile_end) {
      __syncthreads();          // everyone is done with this tile's K and V
      stash();                  // the next tile, fetched during this one
      if (tile + 2 < tile_end) fetch(tile + 2);
      __syncthreads();
    }
  }

  float lrow[4], mrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lrow[i] = __shfl(l_run, (lane >> 4) * 4 + i, 64);
    mrow[i] = __shfl(m_run, (lane >> 4) * 4 + i, 64);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = qb * BQ + wave * 16 + (lane >> 4) * 4 + i;
    if (row >= GC) continue;
    const int h = g * a.G + row / a.C, ii = row % a.C;
    const int64_t r = static_cast<int64_t>(b) * a.C + ii;
    if (a.splits == 1) {
      const float inv = 1.f / lrow[i];
      uint16_t *orow = a.o + r * qcols + h * hd_stride;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) orow[nb * 16 + (lane & 15)] = f32_to_bf16(oacc[nb][i] * inv);
    } else {
      const int64_t R = static_cast<int64_t>(a.B) * a.C;
      float *prow = a.opart + ((split * R + r) * a.Hq + h) * hd_stride;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) prow[nb * 16 + (lane & 15)] = oacc[nb][i];
      if ((lane & 15) == 0) a.ml[(split * R + r) * a.Hq + h] = make_float2(mrow[i], lrow[i]);
    }
  }
}

// o[r, h, e] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s
__global__ void __launch_bounds__(256) attn_combine_kernel(const float *__restrict__ opart,
                                                           const float2 *__restrict__ ml,
                                                           int splits, int64_t rows, int hd,
                                                           uint16_t *__restrict__ o) {
  const int64_t total = rows * hd;   // rows = R * Hq
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t row = idx / hd;
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, ml[s * rows + row].x);
    float num = 0.f, den = 0.f;
    for (int s = 0; s < splits; ++s) {
      const float2 v = ml[s * rows + row];
      const float w = exp2f(v.x - M);
      num += w * opart[s * total + idx];
      den += w * v.y;
    }
    o[idx] = f32_to_bf16(num / den);
  }
}

void plan(const Shape &s, int &splits, int &tps) {
  const int tiles = (s.P + s.C + BKV - 1) / BKV;
  const int base = ((s.G() * s.C + BQ - 1) / BQ) * s.Hkv * s.B;
  int want = (512 + base - 1) / base;
  if (want < 1) want = 1;
  if (want > tiles) want = tiles;
  tps = (tiles + want - 1) / want;
  splits = (tiles + tps - 1) / tps;
}

}  // namespace

int attention_splits(const Shape &s) {
  int sp, tps;
  plan(s, sp, tps);
  return sp;
}

size_t attention_workspace_bytes(const Shape &s) {
  const int sp = attention_splits(s);
  if (sp <= 1) return 0;
  const size_t rows = static_cast<size_t>(s.R()) * s.Hq;
  return sp * rows * (s.hd * sizeof(float) + sizeof(float2));
}

hipError_t launch_attention_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                 const uint16_t *Kp, const uint16_t *Vp, const Shape &s,
                                 void *work, uint16_t *o, hipStream_t st) {
  if (s.R() == 0) return hipSuccess;
  AttnArgs a;
  a.q = q; a.k = k; a.v = v; a.Kp = Kp; a.Vp = Vp; a.o = o;
  a.B = s.B; a.C = s.C; a.P = s.P; a.Hq = s.Hq; a.Hkv = s.Hkv; a.G = s.G();
  plan(s, a.splits, a.tiles_per_split);
  const size_t rows = static_cast<size_t>(s.R()) * s.Hq;
  a.opart = static_cast<float *>(work);
  a.ml = reinterpret_cast<float2 *>(static_cast<char *>(work) +
                                    static_cast<size_t>(a.splits) * rows * s.hd * sizeof(float));
  a.scale_log2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(s.hd)));
  dim3 grid((s.G() * s.C + BQ - 1) / BQ, s.Hkv, s.B * a.splits);
  switch (s.hd) {
    case 64: hipLaunchKernelGGL(attn_fwd_v2_kernel<64>, grid, dim3(256), 0, st, a); break;
    case 128: hipLaunchKernelGGL(attn_fwd_v2_kernel<128>, grid, dim3(256), 0, st, a); break;
    case 176: hipLaunchKernelGGL(attn_fwd_v2_kernel<176>, grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  const int64_t total = static_cast<int64_t>(rows) * s.hd;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st,
                     a.opart, a.ml, a.splits, static_cast<int64_t>(rows), s.hd, o);
  return hipGetLastError();
}

}  // namespace dg
