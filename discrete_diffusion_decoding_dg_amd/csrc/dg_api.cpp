// libdg C ABI: argument checking, workspace ownership and launch order of the
// denoising step. Declarations and the contract live in include/dg.h.
#include "dg.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "dg_kernels.hpp"

namespace {

thread_local std::string g_err;

dg_status fail(dg_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

dg_status hip_fail(hipError_t e, const char *what) {
  return fail(DG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define DG_HIP(call, what)                  \
  do {                                      \
    hipError_t e_ = (call);                 \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

constexpr int kMaxSteps = 4096;
constexpr float kRmsEps = 1e-6f;   // RMSNorm epsilon of the decoder stack
constexpr int kMaxLayers = 256;
constexpr int kPoll = 4;   // adaptive generation tests for early termination every kPoll steps
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void *a, size_t an, const void *b, size_t bn) {
  const char *pa = static_cast<const char *>(a), *pb = static_cast<const char *>(b);
  return pa < pb + bn && pb < pa + an;
}

dg::Shape shape_of(const dg_config &c) {
  return dg::Shape{c.B, c.C, c.P, c.d, c.n_q_heads, c.n_kv_heads, c.head_dim, c.V};
}

// Workspace layout, in carve order.
struct Layout {
  size_t h0, q, k, v, o, h1, attn, lm, etm, prm, kappa, genx, genz, ent, gendet, flags, blkx, blksteps, total;
};

Layout layout_of(const dg_config &c) {
  const dg::Shape s = shape_of(c);
  const size_t es = c.dtype == DG_DTYPE_BF16 ? 2 : 4;
  const size_t R = static_cast<size_t>(s.R());
  Layout L;
  L.h0 = align_up(R * s.d * es);
  L.q = align_up(R * s.Hq * s.hd * es);
  L.k = align_up(R * s.Hkv * s.hd * es);
  L.v = L.k;
  L.o = L.q;
  L.h1 = L.h0;
  if (c.dtype == DG_DTYPE_BF16) {
    // attention partials for any prefix length up to P (block generation
    // attends to a growing prefix; the split count is not monotone in it)
    size_t attn = 0;
    dg::Shape sp = s;
    for (int p = 0;; p += 64) {
      sp.P = p < s.P ? p : s.P;
      const size_t a = dg::attention_workspace_bytes(sp);
      if (a > attn) attn = a;
      if (sp.P == s.P) break;
    }
    L.attn = align_up(attn);
    L.lm = align_up(dg::lmhead_workspace_bytes(s));
    L.etm = align_up(dg::lmhead_copy_bytes(s));      // the LM head's tile-major copy of E
  } else {
    L.attn = 0;
    L.lm = align_up(dg::lmhead_f32_workspace_bytes(s));
    L.etm = 0;
  }
  L.prm = align_up(static_cast<size_t>(kMaxSteps) * s.B * sizeof(dg::StepParams));
  L.kappa = align_up(static_cast<size_t>(s.B) * sizeof(float));
  L.genx = align_up(2 * R * sizeof(int32_t));
  L.genz = align_up(2 * R * s.d * es);
  L.ent = align_up(3 * R * sizeof(int32_t));        // entropy step: H, draw, argmax per row
  L.gendet = align_up(2 * R * sizeof(int32_t));     // generation: argmax predictions, ping-pong
  L.flags = align_up(2 * static_cast<size_t>(s.B) * sizeof(int32_t));   // stopped, stop
  L.blkx = align_up(R * sizeof(int32_t));           // block generation: the canvas being committed
  L.blksteps = align_up(static_cast<size_t>(s.B) * sizeof(int32_t));
  L.total = L.h0 + L.q + L.k + L.v + L.o + L.h1 + L.attn + L.lm + L.etm + L.prm + L.kappa + L.genx +
            L.genz + L.ent + L.gendet + L.flags + L.blkx + L.blksteps;
  return L;
}

dg_status check_config(const dg_config *c) {
  if (!c) return fail(DG_ERR_INVALID_ARG, "config is NULL");
  if (c->B < 1 || c->C < 1 || c->P < 0 || c->d < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 ||
      c->head_dim < 1 || c->V < 2)
    return fail(DG_ERR_INVALID_ARG,
                "sizes must be positive (B=%d C=%d P=%d d=%d Hq=%d Hkv=%d hd=%d V=%d; P may be 0, V >= 2)",
                c->B, c->C, c->P, c->d, c->n_q_heads, c->n_kv_heads, c->head_dim, c->V);
  if (c->n_q_heads % c->n_kv_heads != 0)
    return fail(DG_ERR_INVALID_ARG, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)",
                c->n_q_heads, c->n_kv_heads);
  if (c->dtype != DG_DTYPE_F32 && c->dtype != DG_DTYPE_BF16)
    return fail(DG_ERR_INVALID_ARG, "dtype %d is neither DG_DTYPE_F32 nor DG_DTYPE_BF16", c->dtype);
  if (c->schedule != DG_SCHEDULE_LINEAR && c->schedule != DG_SCHEDULE_COSINE)
    return fail(DG_ERR_INVALID_ARG, "schedule %d is unknown", c->schedule);
  const int64_t R = static_cast<int64_t>(c->B) * c->C;
  const int64_t lim = int64_t(1) << 31;
  if (R * c->d >= lim || R * c->n_q_heads * c->head_dim >= lim ||
      static_cast<int64_t>(c->V) * c->d >= (int64_t(1) << 40) ||
      static_cast<int64_t>(c->P) + c->C >= lim)
    return fail(DG_ERR_INVALID_ARG, "sizes overflow the 32-bit row indexing (B*C*d must be < 2^31)");
  const dg::Shape s = shape_of(*c);
  if (c->dtype == DG_DTYPE_BF16) {
    if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 176)
      return fail(DG_ERR_UNSUPPORTED, "bf16 kernels support head_dim 64, 128, 176 (got %d)",
                  c->head_dim);
    if (!dg::lmhead_supported(s))
      return fail(DG_ERR_UNSUPPORTED,
                  "bf16 LM head supports d in {256, 512, 1024, 2048, 2816} and V %% 16 == 0 "
                  "(got d=%d V=%d)", c->d, c->V);
  } else {
    if (c->d > 4096)
      return fail(DG_ERR_UNSUPPORTED, "fp32 kernels support d <= 4096 (got %d)", c->d);
    if (static_cast<int64_t>(c->P) + c->C > 16384)
      return fail(DG_ERR_UNSUPPORTED, "fp32 attention supports P + C <= 16384 (got %d)",
                  c->P + c->C);
  }
  return DG_OK;
}

// Per-canvas step constants, fp64 on the host, rounded to fp32.
// Schedules: linear kappa = 1 - t; cosine kappa = cos^2(pi t / 2). The Step
// weight is lambda = dt (-dkappa/dt) / (1 - kappa) clamped to [0, 1]; the
// temperature is tau = 0.4 + 0.4 t (linear anneal 0.8 -> 0.4).
dg::StepParams step_params(double t, double dt, int schedule) {
  double rate, one_minus;
  if (schedule == DG_SCHEDULE_LINEAR) {
    rate = 1.0;
    one_minus = t;
  } else {
    const double c = std::cos(0.5 * M_PI * t), s = std::sin(0.5 * M_PI * t);
    rate = M_PI * s * c;
    one_minus = s * s;
  }
  double lam = one_minus > 0.0 ? dt * rate / one_minus : 1.0;
  lam = lam < 0.0 ? 0.0 : (lam > 1.0 ? 1.0 : lam);
  dg::StepParams p;
  p.lam = static_cast<float>(lam);
  p.inv_tau = static_cast<float>(1.0 / (0.4 + 0.4 * t));
  return p;
}

}  // namespace

// ----------------------------------------------------------- model state --
struct dg_model {
  dg_config cfg;
  dg_weights w;
  dg::Shape s;
  int device;
  Layout L;
  char *ws;
  void *h0, *q, *k, *v, *o, *h1, *attn, *lm, *etm;
  dg::StepParams *prm;
  float *kappa;
  int32_t *genx;
  char *genz;
  dg::EntropyRows ent;      // per-row entropy-step results
  int32_t *gendet;          // [2][R] argmax predictions during generation
  int32_t *stopped, *stopbuf;   // [B] each
  int32_t *blkx;                // [B, C] canvas being committed (block generation)
  int32_t *blksteps;            // [B] its step counts (adaptive block generation)
  int32_t *host_stopped = nullptr;   // pinned [B], allocated on first use
  // gated self-conditioning block (dg_set_ffw); ffw_F == 0 is the identity
  int ffw_F = 0;
  const void *ffw_wg = nullptr, *ffw_wu = nullptr, *ffw_wd = nullptr;
  char *ffw_mem = nullptr;   // owned: packed gate/up rows (bf16), u [R, d], hid [R, F]
  void *ffw_gu = nullptr, *ffw_u = nullptr, *ffw_hid = nullptr;
  // decoder stack (dg_set_stack); st_L == 0 is the single attention block
  int st_L = 0, st_F = 0;
  std::vector<dg_layer_weights> st_w;
  const void *st_gfinal = nullptr;
  char *st_mem = nullptr;   // owned: packed gate/up rows (bf16), a, h_attn, two h [R, d], hid [R, F]
  void *st_gu = nullptr, *st_a = nullptr, *st_ha = nullptr, *st_hb = nullptr, *st_hc = nullptr,
       *st_hid = nullptr;
  // mixture of experts in the stack's MLPs (st_X == 0: dense)
  int st_X = 0, st_k = 0;
  std::vector<const void *> st_wr;   // routers [X, d] per layer
  int32_t *st_sel = nullptr, *st_list = nullptr, *st_offs = nullptr, *st_toff = nullptr;
  float *st_wts = nullptr, *st_y = nullptr;
  // profiling: event pairs recorded around stage launches while enabled
  int prof_mask = 0;
  struct Mark {
    int stage;
    hipEvent_t a, b;
  };
  std::vector<Mark> marks;
};

namespace {

// Records an event pair around one stage when profiling is on.
struct StageTimer {
  dg_model *m;
  int stage;
  hipStream_t st;
  hipEvent_t a = nullptr, b = nullptr;
  StageTimer(dg_model *m_, int stage_, hipStream_t st_) : m(m_), stage(stage_), st(st_) {
    if (((m->prof_mask >> stage) & 1) && hipEventCreate(&a) == hipSuccess && hipEventCreate(&b) == hipSuccess)
      (void)hipEventRecord(a, st);
  }
  ~StageTimer() {
    if (a && b) {
      (void)hipEventRecord(b, st);
      m->marks.push_back({stage, a, b});
    }
  }
};

// z = FFW(u) through the attached block; rows of canvases marked in `frozen`
// (nullable) take z_t instead.
dg_status run_ffw(dg_model *m, const void *u, void *z, const int32_t *frozen, const void *z_t,
                  hipStream_t st) {
  const dg::Shape &s = m->s;
  const int F = m->ffw_F;
  StageTimer tm(m, 7, st);
  if (m->cfg.dtype == DG_DTYPE_BF16) {
    using u16 = uint16_t;
    DG_HIP(dg::launch_ffw_gate_up_bf16(static_cast<const u16 *>(u), static_cast<const u16 *>(m->ffw_gu),
                                       s.R(), s.d, F, static_cast<u16 *>(m->ffw_hid), st),
           "feed-forward gate/up launch");
    DG_HIP(dg::launch_ffw_down_bf16(static_cast<const u16 *>(m->ffw_hid),
                                    static_cast<const u16 *>(m->ffw_wd), s.R(), s.d, F, s.C, frozen,
                                    static_cast<const u16 *>(z_t), static_cast<u16 *>(z), st),
           "feed-forward down launch");
  } else {
    DG_HIP(dg::launch_ffw_gate_up_f32(static_cast<const float *>(u), static_cast<const float *>(m->ffw_wg),
                                      static_cast<const float *>(m->ffw_wu), s.R(), s.d, F,
                                      static_cast<float *>(m->ffw_hid), st),
           "feed-forward gate/up launch");
    DG_HIP(dg::launch_ffw_down_f32(static_cast<const float *>(m->ffw_hid),
                                   static_cast<const float *>(m->ffw_wd), s.R(), s.d, F, s.C, frozen,
                                   static_cast<const float *>(z_t), static_cast<float *>(z), st),
           "feed-forward down launch");
  }
  return DG_OK;
}

// The pieces of one attention block over the rows of shape sa (B canvases of
// sa.C rows): q, k, v = x W^T (stage 1), attention over [prefix ; canvas]
// (stage 2), out = res + o Wo^T (stage 3; res may equal x).
dg_status qkv_part(dg_model *m, const void *x, const void *Wq, const void *Wk, const void *Wv,
                   const dg::Shape &sa, void *q, void *k, void *v, hipStream_t st) {
  StageTimer tm(m, 1, st);
  if (m->cfg.dtype == DG_DTYPE_BF16) {
    using u16 = uint16_t;
    DG_HIP(dg::launch_qkv_bf16(static_cast<const u16 *>(x), static_cast<const u16 *>(Wq),
                               static_cast<const u16 *>(Wk), static_cast<const u16 *>(Wv), sa,
                               static_cast<u16 *>(q), static_cast<u16 *>(k), static_cast<u16 *>(v), st),
           "qkv launch");
  } else {
    DG_HIP(dg::launch_qkv_f32(static_cast<const float *>(x), static_cast<const float *>(Wq),
                              static_cast<const float *>(Wk), static_cast<const float *>(Wv), sa,
                              static_cast<float *>(q), static_cast<float *>(k), static_cast<float *>(v), st),
           "qkv launch");
  }
  return DG_OK;
}

dg_status attend_part(dg_model *m, const void *q, const void *k, const void *v, const void *Kp,
                      const void *Vp, const dg::Shape &sa, void *o, hipStream_t st) {
  StageTimer tm(m, 2, st);
  if (m->cfg.dtype == DG_DTYPE_BF16) {
    using u16 = uint16_t;
    DG_HIP(dg::launch_attention_bf16(static_cast<const u16 *>(q), static_cast<const u16 *>(k),
                                     static_cast<const u16 *>(v), static_cast<const u16 *>(Kp),
                                     static_cast<const u16 *>(Vp), sa, m->attn, static_cast<u16 *>(o), st),
           "attention launch");
  } else {
    DG_HIP(dg::launch_attention_f32(static_cast<const float *>(q), static_cast<const float *>(k),
                                    static_cast<const float *>(v), static_cast<const float *>(Kp),
                                    static_cast<const float *>(Vp), sa, static_cast<float *>(o), st),
           "attention launch");
  }
  return DG_OK;
}

dg_status oproj_part(dg_model *m, const void *o, const void *Wo, const void *res, const dg::Shape &sa,
                     void *out, hipStream_t st) {
  StageTimer tm(m, 3, st);
  if (m->cfg.dtype == DG_DTYPE_BF16) {
    using u16 = uint16_t;
    DG_HIP(dg::launch_residual_gemm_bf16(static_cast<const u16 *>(o), static_cast<const u16 *>(Wo),
                                         static_cast<const u16 *>(res), sa.R(), sa.d, sa.Hq * sa.hd,
                                         static_cast<u16 *>(out), st),
           "out-projection launch");
  } else {
    DG_HIP(dg::launch_oproj_f32(static_cast<const float *>(o), static_cast<const float *>(Wo),
                                static_cast<const float *>(res), sa, static_cast<float *>(out), st),
           "out-projection launch");
  }
  return DG_OK;
}

// One attention block: q, k, v = x W^T; attention over [prefix ; canvas];
// out = res + o Wo^T (res may equal x). Stages 1-3 of the profile.
dg_status attn_block(dg_model *m, const void *x, const void *res, const void *Wq, const void *Wk,
                     const void *Wv, const void *Wo, const void *Kp, const void *Vp,
                     const dg::Shape &sa, void *q, void *k, void *v, void *o, void *out,
                     hipStream_t st) {
  if (dg_status e = qkv_part(m, x, Wq, Wk, Wv, sa, q, k, v, st)) return e;
  if (dg_status e = attend_part(m, q, k, v, Kp, Vp, sa, o, st)) return e;
  return oproj_part(m, o, Wo, res, sa, out, st);
}

// The MLP of stack layer l on R rows (canvases of C rows): out = hin +
// MLP(rmsnorm(hin) g_mlp), dense gated or routed experts; the norm goes
// through st_a. Stage 9 of the profile.
dg_status stack_mlp(dg_model *m, int l, int R, int C, const void *hin, void *out, hipStream_t st) {
  const bool bf16 = m->cfg.dtype == DG_DTYPE_BF16;
  const int d = m->s.d, F = m->st_F;
  const dg_layer_weights &lw = m->st_w[l];
  StageTimer tm(m, 9, st);
  DG_HIP(dg::launch_rmsnorm(bf16, hin, lw.g_mlp, R, d, kRmsEps, m->st_a, st), "norm launch");
  if (m->st_X) {
    // mixture of experts: route, group, expert GEMMs, weighted combine
    const int X = m->st_X, K = m->st_k;
    DG_HIP(dg::launch_moe_route(bf16, m->st_a, m->st_wr[l], R, d, X, K, m->st_sel, m->st_wts,
                                bf16 ? m->st_list : nullptr, m->st_offs, m->st_toff, st),
           "router launch");
    if (bf16) {
      using u16 = uint16_t;
      const u16 *gu = static_cast<const u16 *>(m->st_gu) + static_cast<size_t>(l) * X * 2 * F * d;
      DG_HIP(dg::launch_moe_experts_bf16(static_cast<const u16 *>(m->st_a), gu,
                                         static_cast<const u16 *>(lw.W_down), m->st_list, m->st_offs,
                                         m->st_toff, R, K, X, d, F, static_cast<u16 *>(m->st_hid),
                                         m->st_y, st),
             "expert GEMM launch");
    } else {
      DG_HIP(dg::launch_moe_experts_f32(static_cast<const float *>(m->st_a), m->st_sel,
                                        static_cast<const float *>(lw.W_gate),
                                        static_cast<const float *>(lw.W_up),
                                        static_cast<const float *>(lw.W_down), R * K, K, d, F,
                                        static_cast<float *>(m->st_hid), m->st_y, st),
             "expert launch");
    }
    DG_HIP(dg::launch_moe_combine(bf16, hin, m->st_y, m->st_wts, R, d, K, out, st), "combine launch");
  } else if (bf16) {
    using u16 = uint16_t;
    const u16 *gu = static_cast<const u16 *>(m->st_gu) + static_cast<size_t>(l) * 2 * F * d;
    DG_HIP(dg::launch_ffw_gate_up_bf16(static_cast<const u16 *>(m->st_a), gu, R, d, F,
                                       static_cast<u16 *>(m->st_hid), st),
           "MLP gate/up launch");
    DG_HIP(dg::launch_residual_gemm_bf16(static_cast<const u16 *>(m->st_hid),
                                         static_cast<const u16 *>(lw.W_down),
                                         static_cast<const u16 *>(hin), R, d, F, static_cast<u16 *>(out), st),
           "MLP down launch");
  } else {
    DG_HIP(dg::launch_ffw_gate_up_f32(static_cast<const float *>(m->st_a),
                                      static_cast<const float *>(lw.W_gate),
                                      static_cast<const float *>(lw.W_up), R, d, F,
                                      static_cast<float *>(m->st_hid), st),
           "MLP gate/up launch");
    DG_HIP(dg::launch_ffw_down_f32(static_cast<const float *>(m->st_hid),
                                   static_cast<const float *>(lw.W_down), R, d, F, C, nullptr,
                                   nullptr, static_cast<float *>(out), st,
                                   static_cast<const float *>(hin)),
           "MLP down launch");
  }
  return DG_OK;
}

// The decoder stack from h0 (embedding + z) to the LM head's input hf:
// per layer a = rmsnorm(h) g_attn; h = h + attention block(a); a =
// rmsnorm(h) g_mlp; h = h + MLP(a); then hf = rmsnorm(h) g_final. Layer l
// reads cache slice l of Kp, Vp ([L, B, Hkv, P, hd]). Stage 9 of the profile
// covers the norms and the MLP.
dg_status run_stack(dg_model *m, const void *h0, const void *Kp, const void *Vp, const dg::Shape &sa,
                    void *q, void *k, void *v, void *o, void *hf, hipStream_t st) {
  const dg::Shape &s = m->s;
  const bool bf16 = m->cfg.dtype == DG_DTYPE_BF16;
  const size_t es = bf16 ? 2 : 4;
  const size_t cache = static_cast<size_t>(s.B) * s.Hkv * s.P * s.hd * es;
  const int R = s.R(), d = s.d;
  const void *h = h0;
  void *hb[2] = {m->st_hb, m->st_hc};
  for (int l = 0; l < m->st_L; ++l) {
    const dg_layer_weights &lw = m->st_w[l];
    {
      StageTimer tm(m, 9, st);
      DG_HIP(dg::launch_rmsnorm(bf16, h, lw.g_attn, R, d, kRmsEps, m->st_a, st), "norm launch");
    }
    if (dg_status e = attn_block(m, m->st_a, h, lw.Wq, lw.Wk, lw.Wv, lw.Wo,
                                 static_cast<const char *>(Kp) + l * cache,
                                 static_cast<const char *>(Vp) + l * cache, sa, q, k, v, o, m->st_ha, st))
      return e;
    void *hn = hb[l & 1];
    if (dg_status e = stack_mlp(m, l, R, s.C, m->st_ha, hn, st)) return e;
    h = hn;
  }
  StageTimer tm(m, 9, st);
  DG_HIP(dg::launch_rmsnorm(bf16, h, m->st_gfinal, R, d, kRmsEps, hf, st), "norm launch");
  return DG_OK;
}

// Causal encoder pass of the stack (prefill / commit with a stack attached):
// tokens [B, ld] (columns [0, n)) into cache rows [pos, pos + n) of every
// layer's slice of K, V ([L, B, Hkv, P, hd]). Chunks of at most C tokens;
// per chunk h = E[x]; per layer a = rmsnorm(h) g_attn, q, k, v = a W^T, k and
// v copied into the layer's cache rows, then (all but the last layer)
// attention of the chunk over the cache rows before it and, causally, over
// its own keys, h += o Wo^T and h += MLP. Stage 8 covers the embedding and
// the copies; the layers' kernels count under stages 1-3 and 9.
dg_status encode_stack(dg_model *m, const int32_t *tokens, int n, int ld, int pos, void *K, void *V,
                       hipStream_t st) {
  const dg::Shape &s = m->s;
  const bool bf16 = m->cfg.dtype == DG_DTYPE_BF16;
  const size_t es = bf16 ? 2 : 4;
  const size_t cache = static_cast<size_t>(s.B) * s.Hkv * s.P * s.hd * es;
  const int d = s.d, L = m->st_L;
  for (int c0 = 0; c0 < n; c0 += s.C) {
    const int nc = n - c0 < s.C ? n - c0 : s.C;
    dg::Shape sc = s;      // the chunk as a canvas of nc rows over cache rows [0, pos + c0)
    sc.C = nc;
    sc.P = pos + c0;
    sc.Pst = s.P;
    sc.causal = 1;
    if (bf16 && dg::attention_workspace_bytes(sc) > m->L.attn)
      return fail(DG_ERR_UNSUPPORTED, "internal: encoder attention partials exceed the workspace");
    const int R = sc.R();
    {
      StageTimer tm(m, 8, st);
      DG_HIP(dg::launch_embed_tokens(bf16, m->w.E, tokens + c0, ld, s.B, nc, d, s.V, m->h0, st),
             "encoder embedding launch");
    }
    const void *h = m->h0;
    void *hb[2] = {m->st_hb, m->st_hc};
    for (int l = 0; l < L; ++l) {
      const dg_layer_weights &lw = m->st_w[l];
      char *Kl = static_cast<char *>(K) + l * cache;
      char *Vl = static_cast<char *>(V) + l * cache;
      {
        StageTimer tm(m, 9, st);
        DG_HIP(dg::launch_rmsnorm(bf16, h, lw.g_attn, R, d, kRmsEps, m->st_a, st), "norm launch");
      }
      if (dg_status e = qkv_part(m, m->st_a, lw.Wq, lw.Wk, lw.Wv, sc, m->q, m->k, m->v, st)) return e;
      {
        StageTimer tm(m, 8, st);
        DG_HIP(dg::launch_kv_to_cache(bf16, m->k, m->v, sc, pos + c0, Kl, Vl, st), "cache copy launch");
      }
      if (l == L - 1) break;   // the last layer's output feeds no cache entry
      if (dg_status e = attend_part(m, m->q, m->k, m->v, Kl, Vl, sc, m->o, st)) return e;
      if (dg_status e = oproj_part(m, m->o, lw.Wo, h, sc, m->st_ha, st)) return e;
      void *hn = hb[l & 1];
      if (dg_status e = stack_mlp(m, l, R, nc, m->st_ha, hn, st)) return e;
      h = hn;
    }
  }
  return DG_OK;
}

// prm: device step constants of every canvas; when n_inline > 0 the embedding
// launch first stores them there from the host array `inline_prm`.
// With `ent` the step is the entropy-bounded one: every row draws and the
// merge writes per-row entropy, draw and argmax to *ent (the select kernel
// then produces the tokens); rows of canvases marked in `frozen` keep z_t.
// With a decoder stack attached the body between the embedding and the LM
// head is the stack, and h1 holds the final normalised activation.
dg_status run_step(dg_model *m, const int32_t *x_t, const void *z_t, const void *Kp,
                   const void *Vp, dg::StepParams *prm, const dg::StepParams *inline_prm,
                   int n_inline, uint64_t seed, int32_t *x_out, void *z_out,
                   const dg_taps *taps, float *lse, float *p0, hipStream_t st,
                   const dg::EntropyRows *ent = nullptr, const int32_t *frozen = nullptr,
                   int P_cur = -1, bool h0_ready = false, void *h0_next = nullptr) {
  const dg::Shape &s = m->s;
  // attention over the first P_cur rows of caches with s.P rows per slice
  dg::Shape sa = s;
  if (P_cur >= 0) {
    sa.P = P_cur;
    sa.Pst = s.P;
  }
  const bool bf16 = m->cfg.dtype == DG_DTYPE_BF16;
  void *h0 = taps && taps->h0 ? taps->h0 : m->h0;
  void *q = taps && taps->q ? taps->q : m->q;
  void *k = taps && taps->k ? taps->k : m->k;
  void *v = taps && taps->v ? taps->v : m->v;
  void *o = taps && taps->o ? taps->o : m->o;
  void *h1 = taps && taps->h1 ? taps->h1 : m->h1;
  int32_t *best = taps ? taps->best : nullptr;
  // with a feed-forward block the merge writes its input p0 E, and the block
  // takes care of frozen canvases
  void *zc = z_out;
  const int32_t *frozen_c = frozen;
  if (m->ffw_F) {
    zc = taps && taps->p0E ? taps->p0E : m->ffw_u;
    frozen_c = nullptr;
  }
  if (h0_ready) {
    // the previous step's merge already wrote this step's embedding
    if (n_inline || taps) return fail(DG_ERR_INVALID_ARG, "internal: a precomputed embedding with inline parameters or taps");
  } else {
    StageTimer tm(m, 0, st);
    DG_HIP(dg::launch_embed(bf16, m->w.E, x_t, z_t, s.R(), s.d, s.V, h0, prm, inline_prm, n_inline,
                            st),
           "embed launch");
  }
  if (m->st_L) {
    if (dg_status e = run_stack(m, h0, Kp, Vp, sa, q, k, v, o, h1, st)) return e;
  } else {
    if (dg_status e = attn_block(m, h0, h0, m->w.Wq, m->w.Wk, m->w.Wv, m->w.Wo, Kp, Vp, sa, q, k, v, o,
                                 h1, st))
      return e;
  }
  if (bf16) {
    using u16 = uint16_t;
    {
      StageTimer tm(m, 4, st);
      DG_HIP(dg::launch_lmhead_bf16(static_cast<const u16 *>(h1), static_cast<const u16 *>(m->etm),
                                  x_t, prm, s, seed, m->lm, p0, ent != nullptr, st),
           "LM head launch");
    }
    {
      StageTimer tm(m, 5, st);
      DG_HIP(dg::launch_combine(true, m->lm, dg::lmhead_splits(s), x_t, prm, s, seed, x_out, zc,
                              lse, best, ent, frozen_c, z_t, st, m->w.E, h0_next),
           "combine launch");
    }
  } else {
    {
      StageTimer tm(m, 4, st);
      DG_HIP(dg::launch_lmhead_f32(static_cast<const float *>(h1), static_cast<const float *>(m->w.E),
                                 prm, s, seed, m->lm, p0, ent != nullptr, st),
           "LM head launch");
    }
    {
      StageTimer tm(m, 5, st);
      DG_HIP(dg::launch_combine(false, m->lm, 1, x_t, prm, s, seed, x_out, zc, lse, best, ent,
                              frozen_c, z_t, st),
           "combine launch");
    }
  }
  if (m->ffw_F)
    if (dg_status e = run_ffw(m, zc, z_out, frozen, z_t, st)) return e;
  if (p0) {
    if (!lse) return fail(DG_ERR_INVALID_ARG, "internal: p0 requires lse");
    DG_HIP(dg::launch_p0_from_logits(p0, lse, s.R(), s.V, st), "p0 launch");
  }
  return DG_OK;
}

dg_status check_model(const dg_model *m) {
  if (!m) return fail(DG_ERR_INVALID_ARG, "model is NULL");
  int dev = -1;
  if (hipGetDevice(&dev) == hipSuccess && dev != m->device)
    return fail(DG_ERR_INVALID_ARG, "current device %d is not the model's device %d", dev, m->device);
  return DG_OK;
}

dg_status check_times(const float *t, int B, float dt) {
  if (!t) return fail(DG_ERR_INVALID_ARG, "t is NULL");
  if (!std::isfinite(dt) || !(dt > 0.f) || dt > 1.f)
    return fail(DG_ERR_INVALID_ARG, "dt must be in (0, 1] (got %g)", static_cast<double>(dt));
  for (int b = 0; b < B; ++b)
    if (!std::isfinite(t[b]) || !(t[b] > 0.f) || t[b] > 1.f)
      return fail(DG_ERR_INVALID_ARG, "t[%d] must be in (0, 1] (got %g)", b, static_cast<double>(t[b]));
  return DG_OK;
}

dg_status upload_params(dg_model *m, dg::StepParams *dst, const std::vector<dg::StepParams> &p,
                        hipStream_t st) {
  DG_HIP(dg::launch_set_params(dst, p.data(), static_cast<int>(p.size()), st), "parameter upload");
  return DG_OK;
}

// Step-sampler generation of one batch of canvases from noise (see
// dg_generate_canvas), attending to the first P_cur cache rows (-1: all P).
dg_status generate_steps(dg_model *m, const void *K_pre, const void *V_pre, int P_cur, int steps,
                         uint64_t seed, int32_t *x_out, void *z_out, hipStream_t st) {
  const dg::Shape &s = m->s;
  const bool bf16 = m->cfg.dtype == DG_DTYPE_BF16;
  const size_t es = bf16 ? 2 : 4;
  const size_t R = static_cast<size_t>(s.R());
  const size_t nz = R * s.d * es;

  // per-step constants for every canvas, uploaded once
  std::vector<dg::StepParams> prm(static_cast<size_t>(steps) * s.B);
  const float dt = static_cast<float>(1.0 / steps);
  for (int k = 0; k < steps; ++k) {
    const float tk = static_cast<float>(1.0 - static_cast<double>(k) / steps);
    const dg::StepParams p = step_params(tk, dt, m->cfg.schedule);
    for (int b = 0; b < s.B; ++b) prm[static_cast<size_t>(k) * s.B + b] = p;
  }
  if (dg_status e = upload_params(m, m->prm, prm, st)) return e;

  int32_t *xb[2] = {m->genx, m->genx + R};
  char *zb[2] = {m->genz, m->genz + nz};
  // x_init: corruption of a zero canvas at kappa = 0 (every token uniform)
  DG_HIP(dg::launch_fill_zero(m->kappa, align_up(s.B * sizeof(float)), st), "fill");
  DG_HIP(dg::launch_fill_zero(xb[0], R * sizeof(int32_t), st), "fill");
  DG_HIP(dg::launch_corrupt(xb[0], m->kappa, s.B, s.C, s.V, seed, xb[0], st), "corrupt launch");
  DG_HIP(dg::launch_fill_zero(zb[0], nz, st), "fill");
  // Every step's constants are uploaded above, so the embedding pass only
  // computes h0 = round(E[x] + z) from the previous step's outputs: where the
  // merge can, it writes that for the next step itself (one pass fewer per
  // step; the bf16 Step sampler without a feed-forward block, whose output
  // z only exists after the merge).
  bool h0_ready = false;
  for (int k = 0; k < steps; ++k) {
    const int cur = k & 1, nxt = cur ^ 1;
    const bool last = k == steps - 1;
    int32_t *xo = last ? x_out : xb[nxt];
    void *zo = (last && z_out) ? z_out : zb[nxt];
    const bool fuse = !last && bf16 && !m->ffw_F &&
                      dg::combine_embeds_next(true, m->lm, dg::lmhead_splits(s), s, zo);
    if (dg_status e = run_step(m, xb[cur], zb[cur], K_pre, V_pre, m->prm + static_cast<size_t>(k) * s.B,
                               nullptr, 0, seed + static_cast<uint64_t>(k), xo, zo, nullptr, nullptr,
                               nullptr, st, nullptr, nullptr, P_cur, h0_ready, fuse ? m->h0 : nullptr))
      return e;
    h0_ready = fuse;
  }
  return DG_OK;
}

// Adaptive generation with the entropy-bounded step (see
// dg_generate_canvas_entropy), attending to the first P_cur cache rows (-1:
// all P).
dg_status generate_entropy(dg_model *m, const void *K_pre, const void *V_pre, int P_cur, int max_steps,
                           uint64_t seed, float eps_accept, float eps_stop, int32_t *x_out, void *z_out,
                           int32_t *steps_out, hipStream_t st) {
  const dg::Shape &s = m->s;
  const bool bf16 = m->cfg.dtype == DG_DTYPE_BF16;
  if (!m->host_stopped) {
    void *h = nullptr;
    DG_HIP(hipHostMalloc(&h, static_cast<size_t>(s.B) * sizeof(int32_t), hipHostMallocDefault),
           "hipHostMalloc");
    m->host_stopped = static_cast<int32_t *>(h);
  }
  const size_t es = bf16 ? 2 : 4;
  const size_t R = static_cast<size_t>(s.R());
  const size_t nz = R * s.d * es;

  // temperatures of the whole grid t_k = 1 - k / max_steps, uploaded once
  std::vector<dg::StepParams> prm(static_cast<size_t>(max_steps) * s.B);
  for (int k = 0; k < max_steps; ++k) {
    const float tk = static_cast<float>(1.0 - static_cast<double>(k) / max_steps);
    const dg::StepParams p = step_params(tk, 1.0, m->cfg.schedule);
    for (int b = 0; b < s.B; ++b) prm[static_cast<size_t>(k) * s.B + b] = p;
  }
  if (dg_status e = upload_params(m, m->prm, prm, st)) return e;

  int32_t *xb[2] = {m->genx, m->genx + R};
  char *zb[2] = {m->genz, m->genz + nz};
  int32_t *db[2] = {m->gendet, m->gendet + R};
  DG_HIP(dg::launch_fill_zero(m->kappa, align_up(s.B * sizeof(float)), st), "fill");
  DG_HIP(dg::launch_fill_zero(xb[0], R * sizeof(int32_t), st), "fill");
  DG_HIP(dg::launch_corrupt(xb[0], m->kappa, s.B, s.C, s.V, seed, xb[0], st), "corrupt launch");
  DG_HIP(dg::launch_fill_zero(zb[0], nz, st), "fill");
  DG_HIP(dg::launch_fill_zero(m->stopped, static_cast<size_t>(s.B) * sizeof(int32_t), st), "fill");
  DG_HIP(dg::launch_fill_i32(steps_out, static_cast<size_t>(s.B), max_steps, st), "fill");
  int cur = 0;
  for (int k = 0; k < max_steps; ++k) {
    const int nxt = cur ^ 1;
    if (dg_status e = run_step(m, xb[cur], zb[cur], K_pre, V_pre, m->prm + static_cast<size_t>(k) * s.B,
                               nullptr, 0, seed + static_cast<uint64_t>(k), xb[nxt], zb[nxt], nullptr,
                               nullptr, nullptr, st, &m->ent, m->stopped, P_cur))
      return e;
    DG_HIP(dg::launch_entropy_select(m->ent, xb[cur], k ? db[cur] : nullptr, s.B, s.C, s.V,
                                     eps_accept, eps_stop, seed + static_cast<uint64_t>(k), k,
                                     xb[nxt], db[nxt], nullptr, m->stopbuf, m->stopped, steps_out, st),
           "select launch");
    cur = nxt;
    // every kPoll steps, end early once every canvas has stopped
    if ((k + 1) % kPoll == 0 && k + 1 < max_steps) {
      DG_HIP(hipMemcpyAsync(m->host_stopped, m->stopped, static_cast<size_t>(s.B) * sizeof(int32_t),
                            hipMemcpyDeviceToHost, st), "stop flags copy");
      DG_HIP(hipStreamSynchronize(st), "stop flags sync");
      bool all = true;
      for (int b = 0; b < s.B && all; ++b) all = m->host_stopped[b] != 0;
      if (all) break;
    }
  }
  DG_HIP(hipMemcpyAsync(x_out, xb[cur], R * sizeof(int32_t), hipMemcpyDeviceToDevice, st), "x copy");
  if (z_out) DG_HIP(hipMemcpyAsync(z_out, zb[cur], nz, hipMemcpyDeviceToDevice, st), "z copy");
  return DG_OK;
}


// Encoder cache entries of tokens [B, ld] (columns [0, n)) into cache rows
// [pos, pos + n): key and value projections of the token embeddings.
dg_status encode_kv(dg_model *m, const int32_t *tokens, int n, int ld, int pos, void *K, void *V,
                    hipStream_t st) {
  if (m->st_L) return encode_stack(m, tokens, n, ld, pos, K, V, st);
  const dg::Shape &s = m->s;
  StageTimer tm(m, 8, st);
  if (m->cfg.dtype == DG_DTYPE_BF16) {
    using u16 = uint16_t;
    // chunks of at most C tokens per canvas fit the step's h0 buffer
    for (int c0 = 0; c0 < n; c0 += s.C) {
      const int nc = n - c0 < s.C ? n - c0 : s.C;
      DG_HIP(dg::launch_embed_tokens(true, m->w.E, tokens + c0, ld, s.B, nc, s.d, s.V, m->h0, st),
             "encoder embedding launch");
      DG_HIP(dg::launch_kv_encode_bf16(static_cast<const u16 *>(m->h0), static_cast<const u16 *>(m->w.Wk),
                                       static_cast<const u16 *>(m->w.Wv), s, nc, pos + c0, s.P,
                                       static_cast<u16 *>(K), static_cast<u16 *>(V), st),
             "encoder projection launch");
    }
  } else {
    DG_HIP(dg::launch_kv_encode_f32(static_cast<const float *>(m->w.E), tokens, ld,
                                    static_cast<const float *>(m->w.Wk), static_cast<const float *>(m->w.Wv),
                                    s, n, pos, s.P, static_cast<float *>(K), static_cast<float *>(V), st),
           "encoder projection launch");
  }
  return DG_OK;
}

// Argument checks of one denoising step of model m (after the model check).
dg_status check_step_args(const dg_model *m, const int32_t *x_t, const void *z_t, const void *K_pre,
                          const void *V_pre, const float *t, float dt, const int32_t *x_out,
                          const void *z_out, const dg_taps *taps) {
  const dg::Shape &s = m->s;
  if (!x_t || !z_t || !x_out || !z_out) return fail(DG_ERR_INVALID_ARG, "x_t, z_t, x_out and z_out must be non-NULL");
  if (s.P > 0 && (!K_pre || !V_pre)) return fail(DG_ERR_INVALID_ARG, "K_pre and V_pre must be non-NULL when P > 0");
  if (dg_status e = check_times(t, s.B, dt)) return e;
  const bool bf16 = m->cfg.dtype == DG_DTYPE_BF16;
  const size_t es = bf16 ? 2 : 4;
  const size_t nx = static_cast<size_t>(s.R()) * sizeof(int32_t);
  const size_t nz = static_cast<size_t>(s.R()) * s.d * es;
  if (overlap(x_out, nx, x_t, nx)) return fail(DG_ERR_INVALID_ARG, "x_out overlaps x_t");
  if (overlap(z_out, nz, z_t, nz)) return fail(DG_ERR_INVALID_ARG, "z_out overlaps z_t");
  if (bf16 && (!aligned16(z_t) || !aligned16(z_out) || (K_pre && !aligned16(K_pre)) ||
               (V_pre && !aligned16(V_pre))))
    return fail(DG_ERR_INVALID_ARG, "bf16 tensors must be 16-byte aligned");
  if (taps && taps->p0 && !taps->lse)
    return fail(DG_ERR_INVALID_ARG, "taps->p0 requires taps->lse");
  if (taps && bf16) {
    const void *tp[7] = {taps->h0, taps->q, taps->k, taps->v, taps->o, taps->h1, taps->p0E};
    for (const void *p : tp)
      if (p && !aligned16(p)) return fail(DG_ERR_INVALID_ARG, "bf16 taps must be 16-byte aligned");
  }
  return DG_OK;
}

// The launches of one checked step: step constants (host storage prm_host of
// B entries, supplied by the caller), then the kernels.
dg_status launch_step(dg_model *m, const int32_t *x_t, const void *z_t, const void *K_pre,
                      const void *V_pre, const float *t, float dt, uint64_t seed, int32_t *x_out,
                      void *z_out, const dg_taps *taps, void *stream, dg::StepParams *prm_host) {
  const dg::Shape &s = m->s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int b = 0; b < s.B; ++b) prm_host[b] = step_params(t[b], dt, m->cfg.schedule);
  // a few canvases: the constants ride along with the embedding launch
  const int n_inline = s.B <= dg::kInlineParams ? s.B : 0;
  if (!n_inline)
    DG_HIP(dg::launch_set_params(m->prm, prm_host, s.B, st), "parameter upload");
  return run_step(m, x_t, z_t, K_pre, V_pre, m->prm, prm_host, n_inline, seed, x_out, z_out,
                  taps, taps ? taps->lse : nullptr, taps ? taps->p0 : nullptr, st);
}

// ---- the step without allocation (dg_denoise_step_static) ----
// Its whole workspace lives in one file-scope device array per GPU. In host
// code `scratch` names a host-side stand-in; its device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
constexpr int kStaticMaxB = 256;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Workspace of one step in carve order: activations, attention and LM-head
// split partials, the LM head's tile-major copy of E, step constants.
struct StaticLayout {
  size_t h0, q, k, v, o, h1, attn, lm, etm, prm, total;
};

StaticLayout static_layout_of(const dg_config &c) {
  const Layout L = layout_of(c);
  StaticLayout S;
  S.h0 = L.h0; S.q = L.q; S.k = L.k; S.v = L.v; S.o = L.o; S.h1 = L.h1;
  S.attn = L.attn; S.lm = L.lm; S.etm = L.etm;
  S.prm = align_up(static_cast<size_t>(c.B) * sizeof(dg::StepParams));
  S.total = S.h0 + S.q + S.k + S.v + S.o + S.h1 + S.attn + S.lm + S.etm + S.prm;
  return S;
}

// Device address of this device's scratch array (looked up on the device's
// first call).
dg_status scratch_address(int dev, char **out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(DG_ERR_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(DG_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<char *>(g_scratch_ptr[dev]);
  return DG_OK;
}

}  // namespace

extern "C" {

const char *dg_status_string(dg_status s) {
  // C callers may pass any int: read the raw value (loading a value outside
  // the enumerators as the C++ enum type is undefined behaviour)
  int v;
  std::memcpy(&v, &s, sizeof(v));
  switch (v) {
    case DG_OK: return "DG_OK";
    case DG_ERR_INVALID_ARG: return "DG_ERR_INVALID_ARG";
    case DG_ERR_UNSUPPORTED: return "DG_ERR_UNSUPPORTED";
    case DG_ERR_HIP: return "DG_ERR_HIP";
    case DG_ERR_OOM: return "DG_ERR_OOM";
  }
  return "DG_ERR_UNKNOWN";
}

const char *dg_last_error(void) { return g_err.c_str(); }

dg_status dg_workspace_bytes(const dg_config *cfg, size_t *bytes) {
  g_err.clear();
  if (dg_status s = check_config(cfg)) return s;
  if (!bytes) return fail(DG_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = layout_of(*cfg).total;
  return DG_OK;
}

dg_status dg_create(const dg_config *cfg, const dg_weights *w, dg_model **out) {
  g_err.clear();
  if (dg_status s = check_config(cfg)) return s;
  if (!w) return fail(DG_ERR_INVALID_ARG, "weights is NULL");
  if (!out) return fail(DG_ERR_INVALID_ARG, "out is NULL");
  if (!w->E || !w->Wq || !w->Wk || !w->Wv || !w->Wo)
    return fail(DG_ERR_INVALID_ARG, "a weight pointer is NULL");
  if (!aligned16(w->E) || !aligned16(w->Wq) || !aligned16(w->Wk) || !aligned16(w->Wv) ||
      !aligned16(w->Wo))
    return fail(DG_ERR_INVALID_ARG, "weight pointers must be 16-byte aligned");
  int dev = 0;
  DG_HIP(hipGetDevice(&dev), "hipGetDevice");
  const Layout L = layout_of(*cfg);
  char *ws = nullptr;
  hipError_t e = hipMalloc(&ws, L.total);
  if (e != hipSuccess) return fail(DG_ERR_OOM, "workspace of %zu bytes: %s", L.total, hipGetErrorString(e));
  dg_model *m = new dg_model;
  m->cfg = *cfg;
  m->w = *w;
  m->s = shape_of(*cfg);
  m->device = dev;
  m->L = L;
  m->ws = ws;
  char *p = ws;
  m->h0 = p; p += L.h0;
  m->q = p; p += L.q;
  m->k = p; p += L.k;
  m->v = p; p += L.v;
  m->o = p; p += L.o;
  m->h1 = p; p += L.h1;
  m->attn = p; p += L.attn;
  m->lm = p; p += L.lm;
  m->etm = p; p += L.etm;
  m->prm = reinterpret_cast<dg::StepParams *>(p); p += L.prm;
  m->kappa = reinterpret_cast<float *>(p); p += L.kappa;
  m->genx = reinterpret_cast<int32_t *>(p); p += L.genx;
  m->genz = p; p += L.genz;
  {
    const size_t R = static_cast<size_t>(m->s.R());
    m->ent.H = reinterpret_cast<float *>(p);
    m->ent.y = reinterpret_cast<int32_t *>(p) + R;
    m->ent.det = reinterpret_cast<int32_t *>(p) + 2 * R;
    p += L.ent;
  }
  m->gendet = reinterpret_cast<int32_t *>(p); p += L.gendet;
  m->stopped = reinterpret_cast<int32_t *>(p);
  m->stopbuf = m->stopped + m->s.B;
  p += L.flags;
  m->blkx = reinterpret_cast<int32_t *>(p); p += L.blkx;
  m->blksteps = reinterpret_cast<int32_t *>(p); p += L.blksteps;
  if (cfg->dtype == DG_DTYPE_BF16) {
    // the LM head's tile-major copy of E, made once (E must not change while
    // the model lives)
    hipError_t re = dg::launch_lmhead_relayout(static_cast<const uint16_t *>(w->E), m->s,
                                               static_cast<uint16_t *>(m->etm), nullptr);
    if (re == hipSuccess) re = hipDeviceSynchronize();
    if (re != hipSuccess) {
      (void)hipFree(ws);
      delete m;
      return hip_fail(re, "copy of E for the LM head");
    }
  }
  *out = m;
  return DG_OK;
}

dg_status dg_profile_enable(dg_model *m, int mask) {
  g_err.clear();
  if (!m) return fail(DG_ERR_INVALID_ARG, "model is NULL");
  m->prof_mask = mask & ((1 << DG_NUM_STAGES) - 1);
  return DG_OK;
}

dg_status dg_profile_read(dg_model *m, dg_profile *out) {
  g_err.clear();
  if (!m || !out) return fail(DG_ERR_INVALID_ARG, "model or out is NULL");
  std::memset(out, 0, sizeof(*out));
  dg_status st = DG_OK;
  for (auto &mk : m->marks) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(mk.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, mk.a, mk.b);
    if (e != hipSuccess && st == DG_OK) st = hip_fail(e, "profile event");
    if (mk.stage >= 0 && mk.stage < DG_NUM_STAGES) {
      out->ms[mk.stage] += ms;
      out->count[mk.stage] += 1;
    }
    (void)hipEventDestroy(mk.a);
    (void)hipEventDestroy(mk.b);
  }
  m->marks.clear();
  return st;
}

dg_status dg_destroy(dg_model *m) {
  g_err.clear();
  if (!m) return DG_OK;
  hipError_t e = hipDeviceSynchronize();
  for (auto &mk : m->marks) {
    (void)hipEventDestroy(mk.a);
    (void)hipEventDestroy(mk.b);
  }
  hipError_t f = hipFree(m->ws);
  if (m->ffw_mem) (void)hipFree(m->ffw_mem);
  if (m->st_mem) (void)hipFree(m->st_mem);
  if (m->host_stopped) (void)hipHostFree(m->host_stopped);
  delete m;
  if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
  if (f != hipSuccess) return hip_fail(f, "hipFree");
  return DG_OK;
}

dg_status dg_corrupt_batch(const int32_t *x0, const float *kappa_dev, int32_t B, int32_t C,
                           int32_t V, uint64_t seed, int32_t *xt_out, void *stream) {
  g_err.clear();
  if (!x0 || !kappa_dev || !xt_out) return fail(DG_ERR_INVALID_ARG, "a pointer is NULL");
  if (B < 0 || C < 0 || V < 1) return fail(DG_ERR_INVALID_ARG, "B, C >= 0 and V >= 1 required");
  const size_t n = static_cast<size_t>(B) * C * sizeof(int32_t);
  if (x0 != xt_out && overlap(x0, n, xt_out, n))
    return fail(DG_ERR_INVALID_ARG, "xt_out partially overlaps x0");
  DG_HIP(dg::launch_corrupt(x0, kappa_dev, B, C, V, seed, xt_out, static_cast<hipStream_t>(stream)),
         "corrupt launch");
  return DG_OK;
}

dg_status dg_corrupt(dg_model *m, const int32_t *x0, const float *kappa, uint64_t seed,
                     int32_t *xt_out, void *stream) {
  g_err.clear();
  if (dg_status s = check_model(m)) return s;
  if (!x0 || !kappa || !xt_out) return fail(DG_ERR_INVALID_ARG, "a pointer is NULL");
  const int B = m->s.B, C = m->s.C;
  for (int b = 0; b < B; ++b)
    if (!std::isfinite(kappa[b]) || kappa[b] < 0.f || kappa[b] > 1.f)
      return fail(DG_ERR_INVALID_ARG, "kappa[%d] must be in [0, 1] (got %g)", b,
                  static_cast<double>(kappa[b]));
  const size_t n = static_cast<size_t>(B) * C * sizeof(int32_t);
  if (overlap(x0, n, xt_out, n)) return fail(DG_ERR_INVALID_ARG, "xt_out overlaps x0");
  hipStream_t st = static_cast<hipStream_t>(stream);
  DG_HIP(dg::launch_set_floats(m->kappa, kappa, B, st), "kappa upload");
  {
    StageTimer tm(m, 6, st);
    DG_HIP(dg::launch_corrupt(x0, m->kappa, B, C, m->s.V, seed, xt_out, st), "corrupt launch");
  }
  return DG_OK;
}

dg_status dg_denoise_step_taps(dg_model *m, const int32_t *x_t, const void *z_t,
                               const void *K_pre, const void *V_pre, const float *t, float dt,
                               uint64_t seed, int32_t *x_out, void *z_out, const dg_taps *taps,
                               void *stream) {
  g_err.clear();
  if (dg_status s = check_model(m)) return s;
  if (dg_status e = check_step_args(m, x_t, z_t, K_pre, V_pre, t, dt, x_out, z_out, taps)) return e;
  std::vector<dg::StepParams> prm(m->s.B);
  return launch_step(m, x_t, z_t, K_pre, V_pre, t, dt, seed, x_out, z_out, taps, stream, prm.data());
}

dg_status dg_set_ffw(dg_model *m, int32_t hidden, const void *W_gate, const void *W_up,
                     const void *W_down) {
  g_err.clear();
  if (dg_status s = check_model(m)) return s;
  const dg::Shape &s = m->s;
  const bool bf16 = m->cfg.dtype == DG_DTYPE_BF16;
  if (hidden < 0) return fail(DG_ERR_INVALID_ARG, "hidden must be >= 0 (got %d)", hidden);
  if (hidden > 0) {
    if (!W_gate || !W_up || !W_down) return fail(DG_ERR_INVALID_ARG, "a feed-forward weight pointer is NULL");
    if (!aligned16(W_gate) || !aligned16(W_up) || !aligned16(W_down))
      return fail(DG_ERR_INVALID_ARG, "feed-forward weight pointers must be 16-byte aligned");
    if (static_cast<int64_t>(s.R()) * hidden >= (int64_t(1) << 31) ||
        static_cast<int64_t>(hidden) * s.d >= (int64_t(1) << 31))
      return fail(DG_ERR_INVALID_ARG, "B*C*hidden and hidden*d must be < 2^31");
    if (bf16 && (hidden % 64 != 0 || s.d % 64 != 0))
      return fail(DG_ERR_UNSUPPORTED, "the bf16 feed-forward kernels need hidden %% 64 == 0 (got %d)", hidden);
  }
  // queued steps may still read the old block
  DG_HIP(hipDeviceSynchronize(), "hipDeviceSynchronize");
  if (m->ffw_mem) {
    DG_HIP(hipFree(m->ffw_mem), "hipFree");
    m->ffw_mem = nullptr;
  }
  m->ffw_F = 0;
  m->ffw_wg = m->ffw_wu = m->ffw_wd = nullptr;
  m->ffw_gu = m->ffw_u = m->ffw_hid = nullptr;
  if (hidden == 0) return DG_OK;

  const size_t es = bf16 ? 2 : 4;
  const size_t R = static_cast<size_t>(s.R()), F = static_cast<size_t>(hidden), d = static_cast<size_t>(s.d);
  const size_t n_gu = bf16 ? align_up(2 * F * d * es) : 0;
  const size_t n_u = align_up(R * d * es), n_hid = align_up(R * F * es);
  char *mem = nullptr;
  hipError_t e = hipMalloc(&mem, n_gu + n_u + n_hid);
  if (e != hipSuccess)
    return fail(DG_ERR_OOM, "feed-forward buffers of %zu bytes: %s", n_gu + n_u + n_hid, hipGetErrorString(e));
  if (bf16) {
    // gate/up rows interleaved in groups of 32: rows 64 j + [0, 32) are gate
    // rows 32 j + [0, 32), rows 64 j + 32 + [0, 32) the up rows of the same units
    const size_t grp = 32 * d * es;
    e = hipMemcpy2D(mem, 2 * grp, W_gate, grp, grp, F / 32, hipMemcpyDeviceToDevice);
    if (e == hipSuccess) e = hipMemcpy2D(mem + grp, 2 * grp, W_up, grp, grp, F / 32, hipMemcpyDeviceToDevice);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
      (void)hipFree(mem);
      return hip_fail(e, "feed-forward weight packing");
    }
  }
  m->ffw_mem = mem;
  m->ffw_F = hidden;
  m->ffw_wg = W_gate;
  m->ffw_wu = W_up;
  m->ffw_wd = W_down;
  m->ffw_gu = bf16 ? mem : nullptr;
  m->ffw_u = mem + n_gu;
  m->ffw_hid = mem + n_gu + n_u;
  return DG_OK;
}

dg_status dg_set_stack(dg_model *m, int32_t n_layers, int32_t mlp_hidden,
                       const dg_layer_weights *layers, const void *g_final) {
  return dg_set_stack_moe(m, n_layers, mlp_hidden, 0, 0, layers, nullptr, g_final);
}

dg_status dg_set_stack_moe(dg_model *m, int32_t n_layers, int32_t mlp_hidden, int32_t n_experts,
                           int32_t top_k, const dg_layer_weights *layers,
                           const void *const *W_router, const void *g_final) {
  g_err.clear();
  if (dg_status s = check_model(m)) return s;
  const dg::Shape &s = m->s;
  const bool bf16 = m->cfg.dtype == DG_DTYPE_BF16;
  if (n_experts < 0 || n_experts > dg::kMoeMaxExperts)
    return fail(DG_ERR_INVALID_ARG, "n_experts must be in [0, %d] (got %d)", dg::kMoeMaxExperts, n_experts);
  if (n_experts > 0 && (top_k < 1 || top_k > n_experts))
    return fail(DG_ERR_INVALID_ARG, "top_k must be in [1, n_experts] (got %d)", top_k);
  if (n_layers > 0 && n_experts > 0) {
    if (!W_router) return fail(DG_ERR_INVALID_ARG, "W_router is NULL");
    for (int l = 0; l < n_layers; ++l)
      if (!W_router[l] || !aligned16(W_router[l]))
        return fail(DG_ERR_INVALID_ARG, "router of layer %d is NULL or not 16-byte aligned", l);
    if (bf16 && (mlp_hidden % 128 != 0 || s.d % 128 != 0))
      return fail(DG_ERR_UNSUPPORTED, "the bf16 expert kernels need mlp_hidden %% 128 == 0 (got %d)", mlp_hidden);
    if (static_cast<int64_t>(s.R()) * top_k * (mlp_hidden > s.d ? mlp_hidden : s.d) >= (int64_t(1) << 31))
      return fail(DG_ERR_INVALID_ARG, "B*C*top_k*max(mlp_hidden, d) must be < 2^31");
  }
  if (n_layers < 0 || n_layers > kMaxLayers)
    return fail(DG_ERR_INVALID_ARG, "n_layers must be in [0, %d] (got %d)", kMaxLayers, n_layers);
  if (n_layers > 0) {
    if (!layers || !g_final) return fail(DG_ERR_INVALID_ARG, "layers and g_final must be non-NULL");
    if (mlp_hidden < 1) return fail(DG_ERR_INVALID_ARG, "mlp_hidden must be >= 1 (got %d)", mlp_hidden);
    if (static_cast<int64_t>(s.R()) * mlp_hidden >= (int64_t(1) << 31) ||
        static_cast<int64_t>(mlp_hidden) * s.d >= (int64_t(1) << 31))
      return fail(DG_ERR_INVALID_ARG, "B*C*mlp_hidden and mlp_hidden*d must be < 2^31");
    if (bf16 && (mlp_hidden % 64 != 0 || s.d % 64 != 0))
      return fail(DG_ERR_UNSUPPORTED, "the bf16 MLP kernels need mlp_hidden %% 64 == 0 (got %d)", mlp_hidden);
    if (!aligned16(g_final)) return fail(DG_ERR_INVALID_ARG, "g_final must be 16-byte aligned");
    for (int l = 0; l < n_layers; ++l) {
      const dg_layer_weights &w = layers[l];
      const void *p[9] = {w.Wq, w.Wk, w.Wv, w.Wo, w.g_attn, w.g_mlp, w.W_gate, w.W_up, w.W_down};
      for (const void *x : p) {
        if (!x) return fail(DG_ERR_INVALID_ARG, "a weight pointer of layer %d is NULL", l);
        if (!aligned16(x)) return fail(DG_ERR_INVALID_ARG, "weight pointers of layer %d must be 16-byte aligned", l);
      }
    }
  }
  // queued steps may still read the old stack
  DG_HIP(hipDeviceSynchronize(), "hipDeviceSynchronize");
  if (m->st_mem) {
    DG_HIP(hipFree(m->st_mem), "hipFree");
    m->st_mem = nullptr;
  }
  m->st_L = m->st_F = m->st_X = m->st_k = 0;
  m->st_w.clear();
  m->st_wr.clear();
  m->st_gfinal = nullptr;
  m->st_gu = m->st_a = m->st_ha = m->st_hb = m->st_hc = m->st_hid = nullptr;
  m->st_sel = m->st_list = m->st_offs = m->st_toff = nullptr;
  m->st_wts = m->st_y = nullptr;
  if (n_layers == 0) return DG_OK;

  const size_t es = bf16 ? 2 : 4;
  const size_t R = static_cast<size_t>(s.R()), F = static_cast<size_t>(mlp_hidden), d = static_cast<size_t>(s.d);
  const size_t X = static_cast<size_t>(n_experts), NX = n_experts ? X : 1;   // MLPs per layer
  const size_t Q = n_experts ? R * static_cast<size_t>(top_k) : R;            // rows of the hidden activations
  const size_t n_gu = bf16 ? align_up(static_cast<size_t>(n_layers) * NX * 2 * F * d * es) : 0;
  const size_t n_act = align_up(R * d * es), n_hid = align_up(Q * F * es);
  const size_t n_moe = n_experts ? align_up(Q * 4) * 3 + align_up((X + 1) * 4) * 2 + align_up(Q * d * 4) : 0;
  const size_t total = n_gu + 4 * n_act + n_hid + n_moe;
  char *mem = nullptr;
  hipError_t e = hipMalloc(&mem, total);
  if (e != hipSuccess)
    return fail(DG_ERR_OOM, "decoder stack buffers of %zu bytes: %s", total, hipGetErrorString(e));
  if (bf16) {
    // per layer and expert, gate/up rows interleaved in groups of 32 (the
    // GEGLU GEMM's layout); experts' matrices follow each other
    const size_t grp = 32 * d * es, mat = F * d * es;
    for (int l = 0; l < n_layers && e == hipSuccess; ++l)
      for (size_t x = 0; x < NX && e == hipSuccess; ++x) {
        char *dst = mem + (static_cast<size_t>(l) * NX + x) * 2 * mat;
        const char *wg = static_cast<const char *>(layers[l].W_gate) + x * mat;
        const char *wu = static_cast<const char *>(layers[l].W_up) + x * mat;
        e = hipMemcpy2D(dst, 2 * grp, wg, grp, grp, F / 32, hipMemcpyDeviceToDevice);
        if (e == hipSuccess) e = hipMemcpy2D(dst + grp, 2 * grp, wu, grp, grp, F / 32, hipMemcpyDeviceToDevice);
      }
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
      (void)hipFree(mem);
      return hip_fail(e, "MLP weight packing");
    }
  }
  m->st_mem = mem;
  m->st_L = n_layers;
  m->st_F = mlp_hidden;
  m->st_w.assign(layers, layers + n_layers);
  m->st_gfinal = g_final;
  m->st_gu = bf16 ? mem : nullptr;
  m->st_a = mem + n_gu;
  m->st_ha = mem + n_gu + n_act;
  m->st_hb = mem + n_gu + 2 * n_act;
  m->st_hc = mem + n_gu + 3 * n_act;
  m->st_hid = mem + n_gu + 4 * n_act;
  if (n_experts) {
    char *p = mem + n_gu + 4 * n_act + n_hid;
    m->st_sel = reinterpret_cast<int32_t *>(p); p += align_up(Q * 4);
    m->st_list = reinterpret_cast<int32_t *>(p); p += align_up(Q * 4);
    m->st_wts = reinterpret_cast<float *>(p); p += align_up(Q * 4);
    m->st_offs = reinterpret_cast<int32_t *>(p); p += align_up((X + 1) * 4);
    m->st_toff = reinterpret_cast<int32_t *>(p); p += align_up((X + 1) * 4);
    m->st_y = reinterpret_cast<float *>(p);
    m->st_X = n_experts;
    m->st_k = top_k;
    m->st_wr.assign(W_router, W_router + n_layers);
  }
  return DG_OK;
}

dg_status dg_ffw(dg_model *m, const void *u, void *z_out, void *stream) {
  g_err.clear();
  if (dg_status s = check_model(m)) return s;
  if (!m->ffw_F) return fail(DG_ERR_INVALID_ARG, "no feed-forward block is attached (dg_set_ffw)");
  if (!u || !z_out) return fail(DG_ERR_INVALID_ARG, "u and z_out must be non-NULL");
  const bool bf16 = m->cfg.dtype == DG_DTYPE_BF16;
  const size_t nz = static_cast<size_t>(m->s.R()) * m->s.d * (bf16 ? 2 : 4);
  if (overlap(u, nz, z_out, nz)) return fail(DG_ERR_INVALID_ARG, "z_out overlaps u");
  if (bf16 && (!aligned16(u) || !aligned16(z_out)))
    return fail(DG_ERR_INVALID_ARG, "bf16 tensors must be 16-byte aligned");
  return run_ffw(m, u, z_out, nullptr, nullptr, static_cast<hipStream_t>(stream));
}

dg_status dg_denoise_step(dg_model *m, const int32_t *x_t, const void *z_t, const void *K_pre,
                          const void *V_pre, const float *t, float dt, uint64_t seed,
                          int32_t *x_out, void *z_out, float *lse_out, float *p0_out,
                          void *stream) {
  g_err.clear();
  if (p0_out && !lse_out) return fail(DG_ERR_INVALID_ARG, "p0_out requires lse_out");
  dg_taps taps;
  std::memset(&taps, 0, sizeof(taps));
  taps.lse = lse_out;
  taps.p0 = p0_out;
  return dg_denoise_step_taps(m, x_t, z_t, K_pre, V_pre, t, dt, seed, x_out, z_out, &taps, stream);
}

dg_status dg_denoise_step_static(const dg_config *cfg, const dg_weights *w, const int32_t *x_t,
                                 const void *z_t, const void *K_pre, const void *V_pre,
                                 const float *t, float dt, uint64_t seed, int32_t *x_out,
                                 void *z_out, float *lse_out, float *p0_out, void *stream) {
  g_err.clear();
  if (dg_status s = check_config(cfg)) return s;
  if (!w) return fail(DG_ERR_INVALID_ARG, "weights is NULL");
  if (!w->E || !w->Wq || !w->Wk || !w->Wv || !w->Wo)
    return fail(DG_ERR_INVALID_ARG, "a weight pointer is NULL");
  if (!aligned16(w->E) || !aligned16(w->Wq) || !aligned16(w->Wk) || !aligned16(w->Wv) ||
      !aligned16(w->Wo))
    return fail(DG_ERR_INVALID_ARG, "weight pointers must be 16-byte aligned");
  if (p0_out && !lse_out) return fail(DG_ERR_INVALID_ARG, "p0_out requires lse_out");
  if (cfg->B > kStaticMaxB)
    return fail(DG_ERR_UNSUPPORTED, "dg_denoise_step_static supports B <= %d (got %d)", kStaticMaxB, cfg->B);
  const StaticLayout S = static_layout_of(*cfg);
  if (S.total > kStaticScratchBytes)
    return fail(DG_ERR_UNSUPPORTED,
                "the step needs %zu bytes of workspace; dg_denoise_step_static has %zu bytes of static "
                "scratch per device (use dg_create and dg_denoise_step)", S.total, kStaticScratchBytes);
  int dev = 0;
  DG_HIP(hipGetDevice(&dev), "hipGetDevice");
  char *p = nullptr;
  if (dg_status e = scratch_address(dev, &p)) return e;
  // a model on the stack that owns nothing: every buffer is carved from the
  // scratch array; generation, entropy and block buffers stay NULL
  dg_model m{};
  m.cfg = *cfg;
  m.w = *w;
  m.s = shape_of(*cfg);
  m.device = dev;
  m.h0 = p; p += S.h0;
  m.q = p; p += S.q;
  m.k = p; p += S.k;
  m.v = p; p += S.v;
  m.o = p; p += S.o;
  m.h1 = p; p += S.h1;
  m.attn = p; p += S.attn;
  m.lm = p; p += S.lm;
  m.etm = p; p += S.etm;
  m.prm = reinterpret_cast<dg::StepParams *>(p);
  dg_taps taps;
  std::memset(&taps, 0, sizeof(taps));
  taps.lse = lse_out;
  taps.p0 = p0_out;
  if (dg_status e = check_step_args(&m, x_t, z_t, K_pre, V_pre, t, dt, x_out, z_out, &taps)) return e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (cfg->dtype == DG_DTYPE_BF16)
    DG_HIP(dg::launch_lmhead_relayout(static_cast<const uint16_t *>(w->E), m.s,
                                      static_cast<uint16_t *>(m.etm), st),
           "copy of E for the LM head");
  dg::StepParams prm_host[kStaticMaxB];
  return launch_step(&m, x_t, z_t, K_pre, V_pre, t, dt, seed, x_out, z_out, &taps, stream, prm_host);
}

dg_status dg_generate_canvas(dg_model *m, const void *K_pre, const void *V_pre, int32_t steps,
                             uint64_t seed, int32_t *x_out, void *z_out, void *stream) {
  g_err.clear();
  if (dg_status s = check_model(m)) return s;
  const dg::Shape &s = m->s;
  if (!x_out) return fail(DG_ERR_INVALID_ARG, "x_out is NULL");
  if (s.P > 0 && (!K_pre || !V_pre)) return fail(DG_ERR_INVALID_ARG, "K_pre and V_pre must be non-NULL when P > 0");
  if (steps < 1 || steps > kMaxSteps)
    return fail(DG_ERR_INVALID_ARG, "steps must be in [1, %d] (got %d)", kMaxSteps, steps);
  const bool bf16 = m->cfg.dtype == DG_DTYPE_BF16;
  if (bf16 && ((K_pre && !aligned16(K_pre)) || (V_pre && !aligned16(V_pre)) ||
               (z_out && !aligned16(z_out))))
    return fail(DG_ERR_INVALID_ARG, "bf16 tensors must be 16-byte aligned");
  return generate_steps(m, K_pre, V_pre, -1, steps, seed, x_out, z_out, static_cast<hipStream_t>(stream));
}

dg_status dg_encode_kv(dg_model *m, const int32_t *tokens, int32_t n, int32_t pos, void *K_cache,
                       void *V_cache, void *stream) {
  g_err.clear();
  if (dg_status s = check_model(m)) return s;
  const dg::Shape &s = m->s;
  if (n < 0 || pos < 0 || static_cast<int64_t>(pos) + n > s.P)
    return fail(DG_ERR_INVALID_ARG, "need n >= 0, pos >= 0 and pos + n <= P (n=%d pos=%d P=%d)", n, pos, s.P);
  if (n == 0) return DG_OK;
  if (!tokens || !K_cache || !V_cache) return fail(DG_ERR_INVALID_ARG, "tokens, K_cache and V_cache must be non-NULL");
  const bool bf16 = m->cfg.dtype == DG_DTYPE_BF16;
  if (bf16 && (!aligned16(K_cache) || !aligned16(V_cache)))
    return fail(DG_ERR_INVALID_ARG, "bf16 tensors must be 16-byte aligned");
  return encode_kv(m, tokens, n, n, pos, K_cache, V_cache, static_cast<hipStream_t>(stream));
}

dg_status dg_generate_blocks(dg_model *m, void *K_cache, void *V_cache, int32_t P0,
                             int32_t n_canvases, int32_t steps, uint64_t seed, int32_t *x_out,
                             void *stream) {
  g_err.clear();
  if (dg_status s = check_model(m)) return s;
  const dg::Shape &s = m->s;
  if (!x_out) return fail(DG_ERR_INVALID_ARG, "x_out is NULL");
  if (n_canvases < 1 || P0 < 0 || static_cast<int64_t>(P0) + static_cast<int64_t>(n_canvases) * s.C > s.P)
    return fail(DG_ERR_INVALID_ARG, "need n_canvases >= 1, P0 >= 0 and P0 + n_canvases * C <= P "
                "(P0=%d n_canvases=%d C=%d P=%d)", P0, n_canvases, s.C, s.P);
  if (!K_cache || !V_cache) return fail(DG_ERR_INVALID_ARG, "K_cache and V_cache must be non-NULL");
  if (steps < 1 || steps > kMaxSteps)
    return fail(DG_ERR_INVALID_ARG, "steps must be in [1, %d] (got %d)", kMaxSteps, steps);
  const bool bf16 = m->cfg.dtype == DG_DTYPE_BF16;
  if (bf16 && (!aligned16(K_cache) || !aligned16(V_cache)))
    return fail(DG_ERR_INVALID_ARG, "bf16 tensors must be 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t row = static_cast<size_t>(s.C) * sizeof(int32_t);
  for (int j = 0; j < n_canvases; ++j) {
    const int Pj = P0 + j * s.C;
    // canvas j: a whole generation against the first Pj cache rows
    if (dg_status e = generate_steps(m, K_cache, V_cache, Pj, steps,
                                     seed + static_cast<uint64_t>(j) * static_cast<uint64_t>(steps),
                                     m->blkx, nullptr, st))
      return e;
    // commit: its clean tokens through the encoder into rows [Pj, Pj + C)
    if (dg_status e = encode_kv(m, m->blkx, s.C, s.C, Pj, K_cache, V_cache, st)) return e;
    DG_HIP(hipMemcpy2DAsync(x_out + static_cast<size_t>(j) * s.C, row * n_canvases, m->blkx, row, row,
                            s.B, hipMemcpyDeviceToDevice, st),
           "canvas copy");
  }
  return DG_OK;
}


dg_status dg_denoise_step_entropy(dg_model *m, const int32_t *x_t, const void *z_t,
                                  const void *K_pre, const void *V_pre, const float *t,
                                  uint64_t seed, float eps_accept, float eps_stop,
                                  const int32_t *det_prev, int32_t *x_out, void *z_out,
                                  int32_t *det_out, float *entropy_out, int32_t *stop_out,
                                  void *stream) {
  g_err.clear();
  if (dg_status s = check_model(m)) return s;
  const dg::Shape &s = m->s;
  if (!x_t || !z_t || !x_out || !z_out || !det_out || !stop_out)
    return fail(DG_ERR_INVALID_ARG, "x_t, z_t, x_out, z_out, det_out and stop_out must be non-NULL");
  if (s.P > 0 && (!K_pre || !V_pre)) return fail(DG_ERR_INVALID_ARG, "K_pre and V_pre must be non-NULL when P > 0");
  if (s.C > dg::kSelectMaxC)
    return fail(DG_ERR_UNSUPPORTED, "the entropy-bounded step supports C <= %d (got %d)", dg::kSelectMaxC, s.C);
  if (!std::isfinite(eps_accept) || !std::isfinite(eps_stop))
    return fail(DG_ERR_INVALID_ARG, "eps_accept and eps_stop must be finite");
  if (dg_status e = check_times(t, s.B, 1.0f)) return e;
  const bool bf16 = m->cfg.dtype == DG_DTYPE_BF16;
  const size_t es = bf16 ? 2 : 4;
  const size_t nx = static_cast<size_t>(s.R()) * sizeof(int32_t);
  const size_t nz = static_cast<size_t>(s.R()) * s.d * es;
  if (overlap(x_out, nx, x_t, nx)) return fail(DG_ERR_INVALID_ARG, "x_out overlaps x_t");
  if (overlap(z_out, nz, z_t, nz)) return fail(DG_ERR_INVALID_ARG, "z_out overlaps z_t");
  if (det_prev && overlap(det_out, nx, det_prev, nx)) return fail(DG_ERR_INVALID_ARG, "det_out overlaps det_prev");
  if (bf16 && (!aligned16(z_t) || !aligned16(z_out) || (K_pre && !aligned16(K_pre)) ||
               (V_pre && !aligned16(V_pre))))
    return fail(DG_ERR_INVALID_ARG, "bf16 tensors must be 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  // only the temperature of the step constants is used here
  std::vector<dg::StepParams> prm(s.B);
  for (int b = 0; b < s.B; ++b) prm[b] = step_params(t[b], 1.0, m->cfg.schedule);
  const int n_inline = s.B <= dg::kInlineParams ? s.B : 0;
  if (!n_inline)
    if (dg_status e = upload_params(m, m->prm, prm, st)) return e;
  if (dg_status e = run_step(m, x_t, z_t, K_pre, V_pre, m->prm, prm.data(), n_inline, seed, x_out,
                             z_out, nullptr, nullptr, nullptr, st, &m->ent, nullptr))
    return e;
  DG_HIP(dg::launch_entropy_select(m->ent, x_t, det_prev, s.B, s.C, s.V, eps_accept, eps_stop, seed,
                                   0, x_out, det_out, entropy_out, stop_out, nullptr, nullptr, st),
         "select launch");
  return DG_OK;
}

dg_status dg_generate_canvas_entropy(dg_model *m, const void *K_pre, const void *V_pre,
                                     int32_t max_steps, uint64_t seed, float eps_accept,
                                     float eps_stop, int32_t *x_out, void *z_out,
                                     int32_t *steps_out, void *stream) {
  g_err.clear();
  if (dg_status s = check_model(m)) return s;
  const dg::Shape &s = m->s;
  if (!x_out || !steps_out) return fail(DG_ERR_INVALID_ARG, "x_out and steps_out must be non-NULL");
  if (s.P > 0 && (!K_pre || !V_pre)) return fail(DG_ERR_INVALID_ARG, "K_pre and V_pre must be non-NULL when P > 0");
  if (max_steps < 1 || max_steps > kMaxSteps)
    return fail(DG_ERR_INVALID_ARG, "max_steps must be in [1, %d] (got %d)", kMaxSteps, max_steps);
  if (s.C > dg::kSelectMaxC)
    return fail(DG_ERR_UNSUPPORTED, "the entropy-bounded step supports C <= %d (got %d)", dg::kSelectMaxC, s.C);
  if (!std::isfinite(eps_accept) || !std::isfinite(eps_stop))
    return fail(DG_ERR_INVALID_ARG, "eps_accept and eps_stop must be finite");
  const bool bf16 = m->cfg.dtype == DG_DTYPE_BF16;
  if (bf16 && ((K_pre && !aligned16(K_pre)) || (V_pre && !aligned16(V_pre)) ||
               (z_out && !aligned16(z_out))))
    return fail(DG_ERR_INVALID_ARG, "bf16 tensors must be 16-byte aligned");
  return generate_entropy(m, K_pre, V_pre, -1, max_steps, seed, eps_accept, eps_stop, x_out, z_out,
                          steps_out, static_cast<hipStream_t>(stream));
}

dg_status dg_generate_blocks_entropy(dg_model *m, void *K_cache, void *V_cache, int32_t P0,
                                     int32_t n_canvases, int32_t max_steps, uint64_t seed,
                                     float eps_accept, float eps_stop, int32_t *x_out,
                                     int32_t *steps_out, void *stream) {
  g_err.clear();
  if (dg_status s = check_model(m)) return s;
  const dg::Shape &s = m->s;
  if (!x_out || !steps_out) return fail(DG_ERR_INVALID_ARG, "x_out and steps_out must be non-NULL");
  if (n_canvases < 1 || P0 < 0 || static_cast<int64_t>(P0) + static_cast<int64_t>(n_canvases) * s.C > s.P)
    return fail(DG_ERR_INVALID_ARG, "need n_canvases >= 1, P0 >= 0 and P0 + n_canvases * C <= P "
                "(P0=%d n_canvases=%d C=%d P=%d)", P0, n_canvases, s.C, s.P);
  if (!K_cache || !V_cache) return fail(DG_ERR_INVALID_ARG, "K_cache and V_cache must be non-NULL");
  if (max_steps < 1 || max_steps > kMaxSteps)
    return fail(DG_ERR_INVALID_ARG, "max_steps must be in [1, %d] (got %d)", kMaxSteps, max_steps);
  if (s.C > dg::kSelectMaxC)
    return fail(DG_ERR_UNSUPPORTED, "the entropy-bounded step supports C <= %d (got %d)", dg::kSelectMaxC, s.C);
  if (!std::isfinite(eps_accept) || !std::isfinite(eps_stop))
    return fail(DG_ERR_INVALID_ARG, "eps_accept and eps_stop must be finite");
  const bool bf16 = m->cfg.dtype == DG_DTYPE_BF16;
  if (bf16 && (!aligned16(K_cache) || !aligned16(V_cache)))
    return fail(DG_ERR_INVALID_ARG, "bf16 tensors must be 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t row = static_cast<size_t>(s.C) * sizeof(int32_t);
  for (int j = 0; j < n_canvases; ++j) {
    const int Pj = P0 + j * s.C;
    // canvas j: adaptive generation against the first Pj cache rows; its step
    // count goes to column j of steps_out [B, n_canvases]
    if (dg_status e = generate_entropy(m, K_cache, V_cache, Pj, max_steps,
                                       seed + static_cast<uint64_t>(j) * static_cast<uint64_t>(max_steps),
                                       eps_accept, eps_stop, m->blkx, nullptr, m->blksteps, st))
      return e;
    if (dg_status e = encode_kv(m, m->blkx, s.C, s.C, Pj, K_cache, V_cache, st)) return e;
    DG_HIP(hipMemcpy2DAsync(x_out + static_cast<size_t>(j) * s.C, row * n_canvases, m->blkx, row, row,
                            s.B, hipMemcpyDeviceToDevice, st),
           "canvas copy");
    DG_HIP(hipMemcpy2DAsync(steps_out + j, sizeof(int32_t) * n_canvases, m->blksteps, sizeof(int32_t),
                            sizeof(int32_t), s.B, hipMemcpyDeviceToDevice, st),
           "step count copy");
  }
  return DG_OK;
}

}  // extern "C"
