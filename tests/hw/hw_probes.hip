// Hardware probes behind the kernel designs (MI355X, gfx950): the issue cost
// of vector-memory loads per CU, the MFMA instruction rates, LDS read
// bandwidth, the back-to-back launch interval, and how MFMAs and VALU
// instructions share a SIMD. Every access stays inside
// its buffer; every loop has a fixed trip count. Times in shader clocks come
// from s_memtime, wall times from HIP events.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

#define CHECK(x)                                                               \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));             \
      std::exit(1);                                                            \
    }                                                                          \
  } while (0)

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;

// ---- A: vector-memory issue. Every wave of a 512-thread block issues NL
// loads of 16 bytes per lane (1 KB per instruction) back to back, either
// straight into LDS (global_load_lds_dwordx4) or into registers; the wave's
// clocks from the first issue to the last, and to all data landed, are kept.
constexpr int NL = 8, NWV = 8;
template <bool DIRECT>
__global__ void __launch_bounds__(512) vmem_issue(const unsigned char *buf, unsigned long long *out,
                                                  unsigned *sink) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[NWV * NL * 1024];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)lds;
  const unsigned char *src = buf + ((size_t)(blockIdx.x * NWV + wave) * NL) * 1024 + lane * 16;
  u32x4 r[NL];
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int n = 0; n < NL; ++n) {
    if (DIRECT) {
      const unsigned m0 = __builtin_amdgcn_readfirstlane(base + (wave * NL + n) * 1024);
      // M0 is reserved by the compiler: keep its value across the block
      unsigned saved;
      asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                   "global_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
                   : "=&s"(saved) : "s"(m0), "v"(src + n * 1024) : "memory");
    } else {
      r[n] = *(const u32x4 *)(src + n * 1024);
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  const unsigned long long t2 = __builtin_amdgcn_s_memtime();
  __syncthreads();
  unsigned acc = 0;
  if (DIRECT) {
    acc = lds[threadIdx.x * 16];
  } else {
#pragma unroll
    for (int n = 0; n < NL; ++n) acc ^= r[n].x ^ r[n].w;
  }
  if (acc == 0xdeadbeefu) sink[0] = acc;
  if (lane == 0 && blockIdx.x == 0) {
    out[wave * 2] = t1 - t0;
    out[wave * 2 + 1] = t2 - t0;
  }
}

// ---- B: MFMA rate. Each wave runs ITER rounds of 4 independent accumulator
// chains of one MFMA shape with register operands.
constexpr int MITER = 2048;
template <int SHAPE>   // 0: 32x32x16 bf16, 1: 16x16x32 bf16, 2: 16x16x16 bf16 (1k)
__global__ void __launch_bounds__(256) mfma_rate(const float *in, float *out) {
  const int lane = threadIdx.x & 63;
  const float x = in[lane];
  bf16x8 a8, b8;
  bf16x4 a4, b4;
  for (int i = 0; i < 8; ++i) {
    a8[i] = (__bf16)(x + i);
    b8[i] = (__bf16)(x - i);
  }
  for (int i = 0; i < 4; ++i) {
    a4[i] = (__bf16)(x + i);
    b4[i] = (__bf16)(x - i);
  }
  float s = 0.f;
  if constexpr (SHAPE == 0) {
    f32x16 c0{}, c1{}, c2{}, c3{};
    for (int it = 0; it < MITER; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a8, b8, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a8, b8, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a8, b8, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a8, b8, c3, 0, 0, 0);
    }
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  } else if constexpr (SHAPE == 1) {
    f32x4 c0{}, c1{}, c2{}, c3{};
    for (int it = 0; it < MITER; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, c3, 0, 0, 0);
    }
    for (int i = 0; i < 4; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  } else {
    f32x4 c0{}, c1{}, c2{}, c3{};
    for (int it = 0; it < MITER; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a4, b4, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a4, b4, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a4, b4, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a4, b4, c3, 0, 0, 0);
    }
    for (int i = 0; i < 4; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// ---- C: LDS read bandwidth. 8 waves read a 64 KB LDS array LITER times per
// instruction kind: 16-byte reads (1 KB per instruction, consecutive lanes on
// consecutive 16-byte pieces) or transposing 8-byte reads (512 B). Clocks of
// the whole block from one barrier to the next.
constexpr int LITER = 1024, LDS_B = 64 * 1024;
template <bool TR>
__global__ void __launch_bounds__(512) lds_rate(unsigned long long *out, unsigned *sink) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_B];
  for (int i = threadIdx.x; i < LDS_B / 4; i += blockDim.x) reinterpret_cast<unsigned *>(lds)[i] = i * 2654435761u;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  unsigned acc = 0;
  if (TR) {
    for (int it = 0; it < LITER; ++it) {
      const unsigned off = ((wave * 8 + it) * 512 + lane * 8) & (LDS_B - 1);
      const bf16x4 v = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4 *)(lds + off)));
      acc ^= __builtin_bit_cast(unsigned, __builtin_shufflevector(v, v, 0, 1));
    }
  } else {
    for (int it = 0; it < LITER; ++it) {
      const unsigned off = ((wave * 8 + it) * 1024 + lane * 16) & (LDS_B - 1);
      const u32x4 v = *reinterpret_cast<const u32x4 *>(lds + off);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  __syncthreads();
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if (acc == 0xdeadbeefu) sink[0] = acc;
  if (threadIdx.x == 0) out[blockIdx.x] = t1 - t0;
}

__global__ void empty_kernel() {}

// ---- E: MFMA and VALU sharing a SIMD. Each wave runs EITER rounds of 4
// independent v_mfma_f32_32x32x16_bf16 chains with NV independent v_fma_f32
// after each MFMA (the order pinned by scheduling groups). ROLES: the four
// older waves (one per SIMD) issue only the MFMAs and the four younger only the
// FMAs. Clocks per round over each CU, from the first wave's start to the last
// wave's end, averaged over the blocks.
constexpr int EITER = 2000;
template <int NV, bool ROLES>
__global__ void __launch_bounds__(512) mfma_valu(float *out, unsigned long long *stamps) {
  const int tid = threadIdx.x, wave = tid >> 6;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (tid + i));
    b[i] = (__bf16)(0.002f * (tid - i));
  }
  f32x16 c0{}, c1{}, c2{}, c3{};
  float x[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) x[k] = tid * 0.01f + k;
  const bool mf = !ROLES || wave < 4, va = !ROLES || wave >= 4;
  const unsigned long long t0 = __builtin_readcyclecounter();
  if (mf && va) {
    for (int it = 0; it < EITER; ++it) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        f32x16 &c = m == 0 ? c0 : m == 1 ? c1 : m == 2 ? c2 : c3;
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
#pragma unroll
        for (int k = 0; k < NV; ++k) x[(m * NV + k) & 31] = fmaf(x[(m * NV + k) & 31], 1.0001f, 0.5f);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
      }
    }
  } else if (mf) {
    for (int it = 0; it < EITER; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
  } else {
    for (int it = 0; it < EITER; ++it) {
#pragma unroll
      for (int k = 0; k < 4 * NV; ++k) x[k & 31] = fmaf(x[k & 31], 1.0001f, 0.5f);
    }
  }
  const unsigned long long t1 = __builtin_readcyclecounter();
  float s = 0.f;
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  for (int k = 0; k < 32; ++k) s += x[k];
  out[blockIdx.x * blockDim.x + tid] = s;
  if ((tid & 63) == 0) {
    stamps[(blockIdx.x * 8 + wave) * 2] = t0;
    stamps[(blockIdx.x * 8 + wave) * 2 + 1] = t1;
  }
}

// one E configuration: 256 blocks of `threads` (one block per CU: 100 KB of
// dynamic LDS each), clocks per round over the CU
template <int NV, bool ROLES>
static double mfma_valu_span(int threads, float *out, unsigned long long *stamps) {
  const int blocks = 256;
  for (int rep = 0; rep < 2; ++rep) {
    hipLaunchKernelGGL((mfma_valu<NV, ROLES>), dim3(blocks), dim3(threads), 100 * 1024, 0, out, stamps);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
  }
  std::vector<unsigned long long> h(blocks * 16);
  CHECK(hipMemcpy(h.data(), stamps, h.size() * 8, hipMemcpyDeviceToHost));
  double span = 0;
  for (int b = 0; b < blocks; ++b) {
    unsigned long long lo = ~0ull, hi = 0;
    for (int w = 0; w < threads / 64; ++w) {
      lo = h[(b * 8 + w) * 2] < lo ? h[(b * 8 + w) * 2] : lo;
      hi = h[(b * 8 + w) * 2 + 1] > hi ? h[(b * 8 + w) * 2 + 1] : hi;
    }
    span += static_cast<double>(hi - lo);
  }
  return span / blocks / EITER;
}

int main() {
  unsigned *sink;
  CHECK(hipMalloc(&sink, 4));
  // A
  {
    const int blocks = 256;
    const size_t bytes = (size_t)blocks * NWV * NL * 1024;
    unsigned char *buf;
    unsigned long long *out;
    CHECK(hipMalloc(&buf, bytes));
    CHECK(hipMemset(buf, 1, bytes));
    CHECK(hipMalloc(&out, NWV * 2 * 8));
    for (int direct = 1; direct >= 0; --direct) {
      for (int rep = 0; rep < 3; ++rep) {
        if (direct)
          hipLaunchKernelGGL(vmem_issue<true>, dim3(blocks), dim3(512), 0, 0, buf, out, sink);
        else
          hipLaunchKernelGGL(vmem_issue<false>, dim3(blocks), dim3(512), 0, 0, buf, out, sink);
        CHECK(hipGetLastError());
        CHECK(hipDeviceSynchronize());
      }
      std::vector<unsigned long long> h(NWV * 2);
      CHECK(hipMemcpy(h.data(), out, h.size() * 8, hipMemcpyDeviceToHost));
      std::printf("vmem_issue %-6s 8 waves x %d loads x 1 KB, clocks to issue per wave:", direct ? "direct" : "vgpr",
                  NL);
      for (int w = 0; w < NWV; ++w) std::printf(" %llu", h[w * 2]);
      std::printf(" | to landed:");
      for (int w = 0; w < NWV; ++w) std::printf(" %llu", h[w * 2 + 1]);
      std::printf("\n");
    }
    CHECK(hipFree(buf));
    CHECK(hipFree(out));
  }
  // B
  {
    const int blocks = 4096, threads = 256;
    float *in, *out;
    CHECK(hipMalloc(&in, 64 * 4));
    CHECK(hipMemset(in, 0, 64 * 4));
    CHECK(hipMalloc(&out, (size_t)blocks * threads * 4));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    const char *names[3] = {"v_mfma_f32_32x32x16_bf16", "v_mfma_f32_16x16x32_bf16", "v_mfma_f32_16x16x16_bf16"};
    const double flop[3] = {32.0 * 32 * 16 * 2, 16.0 * 16 * 32 * 2, 16.0 * 16 * 16 * 2};
    for (int shp = 0; shp < 3; ++shp) {
      float best = 1e30f;
      for (int rep = 0; rep < 3; ++rep) {
        CHECK(hipEventRecord(e0));
        if (shp == 0) hipLaunchKernelGGL(mfma_rate<0>, dim3(blocks), dim3(threads), 0, 0, in, out);
        if (shp == 1) hipLaunchKernelGGL(mfma_rate<1>, dim3(blocks), dim3(threads), 0, 0, in, out);
        if (shp == 2) hipLaunchKernelGGL(mfma_rate<2>, dim3(blocks), dim3(threads), 0, 0, in, out);
        CHECK(hipGetLastError());
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        float ms;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        if (ms < best) best = ms;
      }
      const double total = flop[shp] * 4.0 * MITER * (blocks * threads / 64);
      std::printf("mfma_rate %-26s %8.1f TFLOP/s (%.3f of 2500)\n", names[shp], total / (best * 1e-3) / 1e12,
                  total / (best * 1e-3) / 1e12 / 2500.0);
    }
    CHECK(hipFree(in));
    CHECK(hipFree(out));
    // D
    for (int i = 0; i < 100; ++i) hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, 0);
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    const int nl = 2000;
    for (int i = 0; i < nl; ++i) hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, 0);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    std::printf("launch_interval empty kernels back to back: %.2f us each\n", ms * 1e3 / nl);
  }
  // C
  {
    const int blocks = 256;
    unsigned long long *out;
    CHECK(hipMalloc(&out, blocks * 8));
    for (int tr = 0; tr < 2; ++tr) {
      for (int rep = 0; rep < 3; ++rep) {
        if (tr)
          hipLaunchKernelGGL(lds_rate<true>, dim3(blocks), dim3(512), 0, 0, out, sink);
        else
          hipLaunchKernelGGL(lds_rate<false>, dim3(blocks), dim3(512), 0, 0, out, sink);
        CHECK(hipGetLastError());
        CHECK(hipDeviceSynchronize());
      }
      std::vector<unsigned long long> h(blocks);
      CHECK(hipMemcpy(h.data(), out, blocks * 8, hipMemcpyDeviceToHost));
      unsigned long long mn = ~0ull, mx = 0;
      for (auto v : h) {
        mn = v < mn ? v : mn;
        mx = v > mx ? v : mx;
      }
      const double bytes = 8.0 * LITER * (tr ? 512 : 1024);
      std::printf("lds_rate %-13s 8 waves: %.1f-%.1f bytes/clock per CU\n", tr ? "ds_read_tr_b64" : "ds_read_b128",
                  bytes / mx, bytes / mn);
    }
    CHECK(hipFree(out));
  }
  // E
  {
    float *out;
    unsigned long long *stamps;
    CHECK(hipMalloc(&out, 256 * 512 * 4));
    CHECK(hipMalloc(&stamps, 256 * 16 * 8));
    for (int threads : {256, 512}) {
      std::printf("mfma_valu %d wave(s)/SIMD, 4 MFMA 32x32x16 + 4 NV FMA per wave and round, CU clocks per round:",
                  threads / 256);
      std::printf(" NV=0 %.0f", mfma_valu_span<0, false>(threads, out, stamps));
      std::printf(" NV=4 %.0f", mfma_valu_span<4, false>(threads, out, stamps));
      std::printf(" NV=8 %.0f", mfma_valu_span<8, false>(threads, out, stamps));
      std::printf(" NV=16 %.0f\n", mfma_valu_span<16, false>(threads, out, stamps));
    }
    std::printf("mfma_valu split roles (per SIMD one wave 4 MFMA, one wave 4 NV FMA per round), CU clocks per round:");
    std::printf(" NV=4 %.0f", mfma_valu_span<4, true>(512, out, stamps));
    std::printf(" NV=8 %.0f", mfma_valu_span<8, true>(512, out, stamps));
    std::printf(" NV=16 %.0f\n", mfma_valu_span<16, true>(512, out, stamps));
    CHECK(hipFree(out));
    CHECK(hipFree(stamps));
  }
  CHECK(hipFree(sink));
  return 0;
}
