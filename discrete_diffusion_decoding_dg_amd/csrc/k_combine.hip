// Merge of the vocabulary-split partials and the Step select.
//
// DiffusionGemma Technical Report (hyper.ai summary), Method, three-line
// update. Per row: lse = logsumexp of the scaled logits, z = p0 E from the
// unnormalised split sums, and the Step draw (our Euler reading of Step):
// keep x_t unless the row's Bernoulli u < lambda_b, in which case take the
// Gumbel argmax over the whole vocabulary (ties: lowest id, i.e. the lowest
// split wins an exact tie between splits).
//
// Entropy-bounded step: every row keeps its Gumbel draw, and the merge also
// yields the row's entropy H = ln 2 (log2 L - S1 / L), with L the merged sum
// of exp2(t - M) and S1 the merged sum of exp2(t - M) (t - M) (t the scaled
// logits in log2 units, M the merged reference), and the plain argmax; the
// select kernel then decides which draws to keep.
//
// Grid: (row, strip of columns). Every wave merges the row's split
// statistics itself (one split per lane: wave-wide max / sum); the first wave
// of the first strip also takes the argmax and writes the per-row results.
// Every thread then streams 8 consecutive columns (16 bytes of bf16) of a
// group of splits, with the split weights read back from the owning lane.
// With many splits the block's 256 threads form four groups (splits q, q + 4,
// ...) over a strip of 512 columns, whose sums meet in LDS; with few, one
// group over 2048 columns.
// z partials are bf16 from the MFMA LM head and fp32 from the fp32 path.
//
// Up to 32 bf16 splits (every MFMA workload here) take a second kernel: each
// lane merges all splits of its 8 columns, so the partial sums never meet in
// LDS and no barrier is needed; the split statistics are reduced with DPP
// and lane-swap instructions instead of LDS permutes, and an exact tie of
// the Gumbel maxima is resolved with one ballot.
#include "dg_device.hpp"
#include "dg_kernels.hpp"

namespace dg {
namespace {

constexpr int kMaxSplits = 64;
constexpr int kCols = 8;   // columns per thread

__device__ __forceinline__ void load8(const uint16_t *p, float (&v)[kCols]) {
  const uint4 q = *reinterpret_cast<const uint4 *>(p);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const float *p, float (&v)[kCols]) {
  const float4 a = reinterpret_cast<const float4 *>(p)[0], b = reinterpret_cast<const float4 *>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(uint16_t *p, const float (&v)[kCols]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = static_cast<uint32_t>(f32_to_bf16(v[2 * i])) | (static_cast<uint32_t>(f32_to_bf16(v[2 * i + 1])) << 16);
  *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ void store8(float *p, const float (&v)[kCols]) {
  reinterpret_cast<float4 *>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4 *>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ float load1(const float *p) { return *p; }
__device__ __forceinline__ float load1(const uint16_t *p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float lane_value(float v, int s) {   // s wave-uniform
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), s));
}

// ---- wave-wide reductions without LDS: DPP within rows of 16 lanes (quad
// swaps, then the half-row and row mirrors), then the gfx950 row and half
// swaps (v_permlane16_swap, v_permlane32_swap); every lane gets the result
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1, 0, 3, 2]
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2, 3, 0, 1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
__device__ __forceinline__ float swap_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float swap_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float wave_max_x(float v) {
  v = fmaxf(v, dpp<kQuadSwap1>(v));
  v = fmaxf(v, dpp<kQuadSwap2>(v));
  v = fmaxf(v, dpp<kRowHalfMirror>(v));
  v = fmaxf(v, dpp<kRowMirror>(v));
  return swap_max(v);
}
__device__ __forceinline__ float wave_sum_x(float v) {
  v += dpp<kQuadSwap1>(v);
  v += dpp<kQuadSwap2>(v);
  v += dpp<kRowHalfMirror>(v);
  v += dpp<kRowMirror>(v);
  return swap_sum(v);
}
// id of the lowest lane whose candidate (valid, value) attains the wave's
// maximum value, read from `id` on that lane; -1 if no lane is valid
__device__ __forceinline__ int wave_argmax_lowest(bool valid, float value, int id) {
  const float v = valid ? value : -INFINITY;
  const float mx = wave_max_x(v);
  const uint64_t hit = __ballot(valid && v == mx);
  if (hit == 0) return -1;
  return __builtin_amdgcn_readlane(id, static_cast<int>(__builtin_ctzll(hit)));
}

// NPRE: bf16 partial loads per thread issued before the split statistics are
// reduced (at least ceil(splits / groups); the surplus re-read the last
// split and are not summed), so that their latency overlaps the reductions.
template <typename T, typename ZP, int NPRE>
__global__ void __launch_bounds__(256) combine_kernel(const RowPartial *__restrict__ part,
                                                      const ZP *__restrict__ zpart, int splits,
                                                      const int32_t *__restrict__ x_t,
                                                      const StepParams *__restrict__ prm, int R,
                                                      int C, int d, uint32_t k0, uint32_t k1,
                                                      int32_t *__restrict__ x_out,
                                                      T *__restrict__ z_out,
                                                      float *__restrict__ lse,
                                                      int32_t *__restrict__ best, EntropyRows ent,
                                                      const int32_t *__restrict__ frozen,
                                                      const T *__restrict__ z_t, int groups) {
  __shared__ __attribute__((aligned(16))) float gsum[3 * 64 * kCols];
  const int r = blockIdx.x;
  const int s = threadIdx.x & 63;
  const int tpg = 256 / groups;                    // threads per split group
  const int q = threadIdx.x / tpg, t = threadIdx.x - q * tpg;
  const int c0 = (blockIdx.y * tpg + t) * kCols;
  const int64_t rowoff = static_cast<int64_t>(r) * d;
  if (frozen && frozen[r / C]) {
    // a stopped canvas keeps its self-conditioning signal
    if (q == 0)
      for (int c = c0; c < c0 + kCols && c < d; ++c) z_out[rowoff + c] = z_t[rowoff + c];
    return;
  }
  const int64_t sstride = static_cast<int64_t>(R) * d;
  constexpr bool kPrefetch = NPRE > 0;
  uint4 raw[kPrefetch ? NPRE : 1];
  if constexpr (kPrefetch) {
    // split q + k groups of this thread's 8 columns (clamped to valid
    // addresses; only the splits below `splits` are summed further down)
    const int cc = (c0 + kCols <= d) ? c0 : 0;
    const uint16_t *zp = reinterpret_cast<const uint16_t *>(zpart) + rowoff + cc;
#pragma unroll
    for (int k = 0; k < NPRE; ++k) {
      int sp = q + k * groups;
      if (sp > splits - 1) sp = splits - 1;
      raw[k] = *reinterpret_cast<const uint4 *>(zp + sp * sstride);
    }
  }
  RowPartial p;
  p.m = -INFINITY;
  p.l = 0.f;
  p.best = -INFINITY;
  p.arg = -1;
  p.s1 = 0.f;
  p.dbest = -INFINITY;
  p.darg = -1;
  p.pad = 0;
  if (s < splits) p = part[static_cast<int64_t>(s) * R + r];
  const float M = wave_max(p.m);
  const float w = (s < splits) ? exp2f(p.m - M) : 0.f;
  const float L = wave_sum(w * p.l);
  if (blockIdx.y == 0 && threadIdx.x < 64) {
    // argmax of the best draw over splits; an exact tie goes to the lower split
    float bv = p.arg >= 0 ? p.best : -INFINITY;
    int bs = p.arg >= 0 ? s : kMaxSplits;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int os = __shfl_xor(bs, o, 64);
      if (ov > bv || (ov == bv && os < bs)) { bv = ov; bs = os; }
    }
    const int bi = __shfl(p.arg, bs < kMaxSplits ? bs : 0, 64);
    if (ent.H) {
      // entropy and plain argmax of the row (exact ties: the lower split)
      const float S1 = wave_sum((s < splits && p.l > 0.f) ? w * (p.s1 + (p.m - M) * p.l) : 0.f);
      float dv = (s < splits && p.darg >= 0) ? p.dbest : -INFINITY;
      int ds = (s < splits && p.darg >= 0) ? s : kMaxSplits;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(dv, o, 64);
        const int os = __shfl_xor(ds, o, 64);
        if (ov > dv || (ov == dv && os < ds)) { dv = ov; ds = os; }
      }
      const int di = __shfl(p.darg, ds < kMaxSplits ? ds : 0, 64);
      if (s == 0) {
        ent.H[r] = 0.6931471805599453f * (log2f(L) - S1 / L);
        ent.y[r] = bs < kMaxSplits ? bi : -1;
        ent.det[r] = ds < kMaxSplits ? di : -1;
        if (lse) lse[r] = (M + log2f(L)) * 0.6931471805599453f;
        if (best) best[r] = bs < kMaxSplits ? bi : -1;
      }
    } else if (s == 0) {
      const int b = r / C, i = r - b * C;
      const u32x4 u = philox4x32_10(0u, static_cast<uint32_t>(i), static_cast<uint32_t>(b),
                                    kStreamBernoulli, k0, k1);
      const bool rs = u01(u.x) < prm[b].lam;
      const int y = bs < kMaxSplits ? bi : -1;
      x_out[r] = rs ? y : x_t[r];
      if (lse) lse[r] = (M + log2f(L)) * 0.6931471805599453f;
      if (best) best[r] = rs ? y : -1;
    }
  }
  const float il = 1.f / L;
  if ((d % kCols) == 0) {
    // group q sums splits q, q + groups, ...; the groups meet in LDS
    const bool active = c0 + kCols <= d;
    float acc[kCols];
#pragma unroll
    for (int i = 0; i < kCols; ++i) acc[i] = 0.f;
    if constexpr (kPrefetch) {
#pragma unroll
      for (int k = 0; k < NPRE; ++k) {
        const int sp = q + k * groups;   // wave-uniform
        if (sp < splits) {
          const float ws = lane_value(w, sp);
          const uint32_t wd[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] += ws * __uint_as_float(wd[i] << 16);
            acc[2 * i + 1] += ws * __uint_as_float(wd[i] & 0xFFFF0000u);
          }
        }
      }
    } else if (active) {
      const ZP *zp = zpart + rowoff + c0;
      for (int sp = q; sp < splits; sp += groups) {
        float v[kCols];
        load8(zp + sp * sstride, v);
        const float ws = lane_value(w, sp);
#pragma unroll
        for (int i = 0; i < kCols; ++i) acc[i] += ws * v[i];
      }
    }
    if (groups > 1) {
      if (q > 0)
#pragma unroll
        for (int i = 0; i < kCols; ++i) gsum[((q - 1) * tpg + t) * kCols + i] = acc[i];
      __syncthreads();
      if (q > 0) return;
      for (int g = 0; g < groups - 1; ++g)
#pragma unroll
        for (int i = 0; i < kCols; ++i) acc[i] += gsum[(g * tpg + t) * kCols + i];
    }
    if (!active) return;
#pragma unroll
    for (int i = 0; i < kCols; ++i) acc[i] *= il;
    if ((reinterpret_cast<uintptr_t>(z_out) & 15) == 0) {
      store8(z_out + rowoff + c0, acc);
    } else {
#pragma unroll
      for (int i = 0; i < kCols; ++i) Act<T>::store(z_out, rowoff + c0 + i, acc[i]);
    }
  } else {
    if (q > 0) return;
    for (int c = c0; c < d && c < c0 + kCols; ++c) {
      float acc = 0.f;
      for (int sp = 0; sp < splits; ++sp) acc += lane_value(w, sp) * load1(zpart + sp * sstride + rowoff + c);
      Act<T>::store(z_out, rowoff + c, acc * il);
    }
  }
}


// At most 32 bf16 splits, d % 8 == 0. Grid (row, group of 2048 columns);
// lane (wave w, l) of block (r, y) owns columns 8 (64 (4 y + w) + l) + [0, 8)
// of row r and sums every split of them in split order. Every wave reduces
// the row's split statistics itself (lane s holds split s); wave 0 of the
// first column group also writes the per-row results. NP >= splits: the
// row records are requested first and then NP partial loads (the surplus
// ones re-read the last split and are not summed), so the statistics are
// reduced while the partials are in flight. With h0n every wave also settles
// the row's token and writes its columns of the next step's embedding.
template <int NP>
__global__ void __launch_bounds__(256) combine_wide_kernel(const RowPartial *__restrict__ part,
                                                           const uint16_t *__restrict__ zpart, int splits,
                                                           const int32_t *__restrict__ x_t,
                                                           const StepParams *__restrict__ prm, int R,
                                                           int C, int d, uint32_t k0, uint32_t k1,
                                                           int32_t *__restrict__ x_out,
                                                           uint16_t *__restrict__ z_out,
                                                           float *__restrict__ lse,
                                                           int32_t *__restrict__ best, EntropyRows ent,
                                                           const int32_t *__restrict__ frozen,
                                                           const uint16_t *__restrict__ z_t,
                                                           const uint16_t *__restrict__ E, int V,
                                                           uint16_t *__restrict__ h0n) {
  const int r = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cr = ((blockIdx.y * 4 + wave) * 64 + lane) * kCols;
  const bool active = cr + kCols <= d;
  const int c0 = active ? cr : 0;   // inactive lanes read valid addresses and store nothing
  const int64_t rowoff = static_cast<int64_t>(r) * d;
  RowPartial p;
  p.m = -INFINITY;
  p.l = 0.f;
  p.best = -INFINITY;
  p.arg = -1;
  p.s1 = 0.f;
  p.dbest = -INFINITY;
  p.darg = -1;
  p.pad = 0;
  const bool has = lane < splits;
  if (has) p = part[static_cast<int64_t>(lane) * R + r];
  // buffer loads: the partials as one buffer resource (all splits hold fewer
  // than 2^31 bytes), the split's byte offset in a scalar register and the
  // lane's in a vector register, so no 64-bit address is formed per load
  const int sbytes = R * d * 2;
  const __amdgpu_buffer_rsrc_t zr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(zpart), 0, splits * sbytes, kBufferFlags);
  const int loff = static_cast<int>((rowoff + c0) * 2);
  uint4 raw[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int sp = k < splits ? k : splits - 1;
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(zr, loff, sp * sbytes, 0);
    raw[k] = make_uint4(v[0], v[1], v[2], v[3]);
  }
  if (frozen && frozen[r / C]) {
    // a stopped canvas keeps its self-conditioning signal
    if (active)
      *reinterpret_cast<uint4 *>(z_out + rowoff + c0) = *reinterpret_cast<const uint4 *>(z_t + rowoff + c0);
    return;
  }
  // the row's Bernoulli decision while the loads are in flight
  const bool head = blockIdx.y == 0 && wave == 0;
  const bool need_tok = head || h0n != nullptr;   // wave-uniform
  bool rs = false;
  if (need_tok && !ent.H) {
    const int b = r / C, i = r - b * C;
    const u32x4 u = philox4x32_10(0u, static_cast<uint32_t>(i), static_cast<uint32_t>(b),
                                  kStreamBernoulli, k0, k1);
    rs = u01(u.x) < prm[b].lam;
  }
  const float M = wave_max_x(p.m);
  const float w = has ? exp2f(p.m - M) : 0.f;
  const float L = wave_sum_x(w * p.l);
  // the Gumbel draw over splits (an exact tie goes to the lower split)
  const int y = need_tok ? wave_argmax_lowest(has && p.arg >= 0, p.best, p.arg) : -1;
  if (head) {
    if (ent.H) {
      const float S1 = wave_sum_x((has && p.l > 0.f) ? w * (p.s1 + (p.m - M) * p.l) : 0.f);
      const int det = wave_argmax_lowest(has && p.darg >= 0, p.dbest, p.darg);
      if (lane == 0) {
        ent.H[r] = 0.6931471805599453f * (log2f(L) - S1 / L);
        ent.y[r] = y;
        ent.det[r] = det;
        if (lse) lse[r] = (M + log2f(L)) * 0.6931471805599453f;
        if (best) best[r] = y;
      }
    } else if (lane == 0) {
      x_out[r] = rs ? y : x_t[r];
      if (lse) lse[r] = (M + log2f(L)) * 0.6931471805599453f;
      if (best) best[r] = rs ? y : -1;
    }
  }
  if (!active) return;
  // the next step's embedding row piece, requested before the sums
  uint4 e = make_uint4(0, 0, 0, 0);
  if (h0n) {
    const int tok = rs ? y : x_t[r];
    if (tok >= 0 && tok < V) e = *reinterpret_cast<const uint4 *>(E + static_cast<int64_t>(tok) * d + c0);
  }
  float acc[kCols];
#pragma unroll
  for (int i = 0; i < kCols; ++i) acc[i] = 0.f;
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    if (k < splits) {
      const float ws = lane_value(w, k);
      const uint32_t wd[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += ws * __uint_as_float(wd[i] << 16);
        acc[2 * i + 1] += ws * __uint_as_float(wd[i] & 0xFFFF0000u);
      }
    }
  }
  const float il = 1.f / L;
#pragma unroll
  for (int i = 0; i < kCols; ++i) acc[i] *= il;
  store8(z_out + rowoff + c0, acc);
  if (h0n) {
    // h0 = round(E[token] + z), z as stored (bf16), as the embedding pass
    const uint32_t ew[4] = {e.x, e.y, e.z, e.w};
    uint32_t hw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = bf16_to_f32(static_cast<uint16_t>(ew[i] & 0xFFFFu)) + bf16_to_f32(f32_to_bf16(acc[2 * i]));
      const float hi = bf16_to_f32(static_cast<uint16_t>(ew[i] >> 16)) + bf16_to_f32(f32_to_bf16(acc[2 * i + 1]));
      hw[i] = pack_bf16x2(lo, hi);
    }
    *reinterpret_cast<uint4 *>(h0n + rowoff + c0) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
  }
}

}  // namespace

namespace {
// the many-lane merge applies: bf16 partials, at most 32 splits, whole
// 16-byte column groups, aligned buffers, all splits below 2^31 bytes
bool wide_merge(bool bf16, const void *work, int splits, const Shape &s, const void *z_out,
                const void *z_t) {
  const int R = s.R();
  const char *zbase = static_cast<const char *>(work) + static_cast<size_t>(splits) * R * sizeof(RowPartial);
  const bool aligned16 = ((reinterpret_cast<uintptr_t>(z_out) | reinterpret_cast<uintptr_t>(z_t) |
                           reinterpret_cast<uintptr_t>(zbase)) & 15) == 0;
  const bool fits31 = static_cast<int64_t>(splits) * R * s.d * 2 < (int64_t{1} << 31);
  return bf16 && s.d % kCols == 0 && splits >= 1 && splits <= 32 && aligned16 && fits31;
}
}  // namespace

bool combine_embeds_next(bool bf16, const void *work, int splits, const Shape &s, const void *z_out) {
  return wide_merge(bf16, work, splits, s, z_out, nullptr);
}

hipError_t launch_combine(bool bf16, const void *work, int splits, const int32_t *x_t,
                          const StepParams *prm, const Shape &s, uint64_t seed, int32_t *x_out,
                          void *z_out, float *lse, int32_t *best, const EntropyRows *ent,
                          const int32_t *frozen, const void *z_t, hipStream_t st, const void *E,
                          void *h0_next) {
  const int R = s.R();
  if (R == 0) return hipSuccess;
  if (splits < 1 || splits > kMaxSplits) return hipErrorInvalidValue;
  const RowPartial *part = static_cast<const RowPartial *>(work);
  const char *zbase = static_cast<const char *>(work) + static_cast<size_t>(splits) * R * sizeof(RowPartial);
  const uint32_t k0 = static_cast<uint32_t>(seed), k1 = static_cast<uint32_t>(seed >> 32);
  // four split groups when there are many splits and d fills the strips
  const int groups = (splits >= 8 && s.d % kCols == 0) ? 4 : 1;
  const int strip = 256 / groups * kCols;
  const dim3 grid(R, (s.d + strip - 1) / strip);
  const EntropyRows er = ent ? *ent : EntropyRows{nullptr, nullptr, nullptr};
  if (frozen && !z_t) return hipErrorInvalidValue;
  if (h0_next && (ent || frozen || !E || (reinterpret_cast<uintptr_t>(E) & 15) ||
                  (reinterpret_cast<uintptr_t>(h0_next) & 15) || !wide_merge(bf16, work, splits, s, z_out, z_t)))
    return hipErrorInvalidValue;
  // 16-byte rows: z_out and z_t (and the partials, carved at 256-byte
  // offsets of the workspace) take 16-byte accesses at every 8th column
  if (wide_merge(bf16, work, splits, s, z_out, z_t)) {
    const dim3 wgrid(R, (s.d + 4 * 64 * kCols - 1) / (4 * 64 * kCols));
#define DG_WIDE(NP)                                                                                   \
  hipLaunchKernelGGL((combine_wide_kernel<NP>), wgrid, dim3(256), 0, st, part,                        \
                     reinterpret_cast<const uint16_t *>(zbase), splits, x_t, prm, R, s.C, s.d, k0, k1, \
                     x_out, static_cast<uint16_t *>(z_out), lse, best, er, frozen,                    \
                     static_cast<const uint16_t *>(z_t), static_cast<const uint16_t *>(E), s.V,       \
                     static_cast<uint16_t *>(h0_next))
    if (splits <= 1)
      DG_WIDE(1);
    else if (splits <= 2)
      DG_WIDE(2);
    else if (splits <= 4)
      DG_WIDE(4);
    else if (splits <= 8)
      DG_WIDE(8);
    else if (splits <= 16)
      DG_WIDE(16);
    else
      DG_WIDE(32);
#undef DG_WIDE
    return hipGetLastError();
  }
  // bf16 partials with d % 8 == 0 are prefetched: 8 or 16 loads per thread
  const int per_group = (splits + groups - 1) / groups;
  const bool pre = bf16 && s.d % kCols == 0 && per_group <= 16;
#define DG_COMB(NP)                                                                              \
  hipLaunchKernelGGL((combine_kernel<uint16_t, uint16_t, NP>), grid, dim3(256), 0, st, part,     \
                     reinterpret_cast<const uint16_t *>(zbase), splits, x_t, prm, R, s.C, s.d, k0, \
                     k1, x_out, static_cast<uint16_t *>(z_out), lse, best, er, frozen,            \
                     static_cast<const uint16_t *>(z_t), groups)
  if (pre && per_group <= 8)
    DG_COMB(8);
  else if (pre)
    DG_COMB(16);
  else if (bf16)
    DG_COMB(0);
  else
    hipLaunchKernelGGL((combine_kernel<float, float, 0>), grid, dim3(256), 0, st, part,
                       reinterpret_cast<const float *>(zbase), splits, x_t,
                       prm, R, s.C, s.d, k0, k1, x_out, static_cast<float *>(z_out), lse, best,
                       er, frozen, static_cast<const float *>(z_t), groups);
#undef DG_COMB
  return hipGetLastError();
}

}  // namespace dg
