// Host-side launchers of the gfx950 kernels (internal to libdg).
// Every launcher checks nothing: dg_api.cpp validates shapes and pointers
// before calling them. All pointers are device pointers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

// Per-canvas constants of one step, computed on the host in fp64 and rounded
// to fp32: lambda_b (Step mixing weight) and 1/tau_b (logit scale).
struct StepParams {
  float lam;
  float inv_tau;
};

// Shapes of the decoder stand-in. The prefix cache of canvas b and kv head g
// holds P keys (and values) at rows [0, P) of a slice of pstride() rows.
struct Shape {
  int B, C, P, d, Hq, Hkv, hd, V;
  int Pst = 0;   // cache rows per (canvas, kv head) slice; 0: P
  // attention: canvas query i sees the P prefix keys and canvas keys 0..i
  // only (the causal encoder pass); 0: every canvas key (the decoder)
  int causal = 0;
  int R() const { return B * C; }
  int G() const { return Hq / Hkv; }
  int pstride() const { return Pst ? Pst : P; }
};

// Partial results of the split-V LM head, one record per (split, row).
struct RowPartial {
  float m;        // reference max of the scaled logits in log2 units
  float l;        // sum of exp2(t - m) over the split, t = s*log2e
  float best;     // best Gumbel-perturbed logit (natural units), -inf if none
  int32_t arg;    // its vocab id (lowest on ties), -1 if none
  // entropy statistics (entropy-bounded step only)
  float s1;       // sum of exp2(t - m) (t - m) over the split
  float dbest;    // largest t (log2 units), -inf if none
  int32_t darg;   // its vocab id (lowest on ties), -1 if none
  int32_t pad;
};

// Per-row results of the entropy-bounded step's merge, for the select kernel.
struct EntropyRows {
  float *H;        // [R] entropy of p0 in nats
  int32_t *y;      // [R] Gumbel-max draw from p0
  int32_t *det;    // [R] argmax of the scaled logits
};

// ---- k_elementwise.hip ----
hipError_t launch_corrupt(const int32_t *x0, const float *kappa, int B, int C, int V,
                          uint64_t seed, int32_t *out, hipStream_t st);
// h0 = round(E[x] + z); z may be null (treated as 0); tokens outside [0, V)
// embed as a zero row.
// h0 = E[x] + z; also stores `np` (<= kInlineParams) step constants from host
// memory into prm (they travel as a kernel argument)
constexpr int kInlineParams = 32;
hipError_t launch_embed(bool bf16, const void *E, const int32_t *x, const void *z, int R, int d,
                        int V, void *h0, StepParams *prm, const StepParams *prm_src, int np,
                        hipStream_t st);
// h [B * n, d] = E[x[b * ld + i]] for i < n (no self-conditioning input).
hipError_t launch_embed_tokens(bool bf16, const void *E, const int32_t *x, int ld, int B, int n,
                               int d, int V, void *h, hipStream_t st);
// y [R, d] = round(x / sqrt(mean(x^2) + eps) * g) per row.
hipError_t launch_rmsnorm(bool bf16, const void *x, const void *g, int R, int d, float eps, void *y,
                          hipStream_t st);
// p0[r, v] = exp(p0[r, v] - lse[r]) in place (p0 holds scaled logits on entry).
hipError_t launch_p0_from_logits(float *p0, const float *lse, int R, int V, hipStream_t st);
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t st);
// Canvas-layout k, v [B, Hkv, C, hd] (act) into rows [row0, row0 + C) of
// caches [B, Hkv, Pst, hd] (C, Pst from s; the encoder pass of a stack).
hipError_t launch_kv_to_cache(bool bf16, const void *k, const void *v, const Shape &s, int row0,
                              void *K, void *V, hipStream_t st);
// Copy small host arrays to device memory through kernel arguments.
hipError_t launch_set_params(StepParams *dst, const StepParams *src, int n, hipStream_t st);
hipError_t launch_fill_i32(int32_t *p, size_t n, int32_t v, hipStream_t st);
hipError_t launch_set_floats(float *dst, const float *src, int n, hipStream_t st);

// ---- k_gemm.hip (bf16 MFMA) ----
// q [R, Hq*hd], k/v [B, Hkv, C, hd] = h0 W^T for the three weights.
hipError_t launch_qkv_bf16(const uint16_t *h0, const uint16_t *Wq, const uint16_t *Wk,
                           const uint16_t *Wv, const Shape &s, uint16_t *q, uint16_t *k,
                           uint16_t *v, hipStream_t st);
// out [M, N] = res + A W^T (A [M, K], W [N, K]).
hipError_t launch_residual_gemm_bf16(const uint16_t *A, const uint16_t *W, const uint16_t *res, int M,
                                    int N, int K, uint16_t *out, hipStream_t st);

// ---- gated self-conditioning block z = FFW(u) (k_gemm.hip bf16 MFMA) ----
// hid [M, F] = round(gelu(u Wg^T) * (u Wu^T)) from the packed gate/up matrix
// Wgu [2F, d] (rows 64 j + [0, 32): gate rows 32 j + [0, 32); rows
// 64 j + 32 + [0, 32): the up rows of the same units). Needs d % 64 == 0 and
// F % 32 == 0 (hipErrorInvalidValue otherwise).
hipError_t launch_ffw_gate_up_bf16(const uint16_t *u, const uint16_t *Wgu, int M, int d, int F,
                                   uint16_t *hid, hipStream_t st);
// z [M, d] = hid Wd^T, Wd [d, F]; rows m of canvases m / C marked in `frozen`
// (nullable) copy z_t. Needs F % 64 == 0 and d % 64 == 0.
hipError_t launch_ffw_down_bf16(const uint16_t *hid, const uint16_t *Wd, int M, int d, int F, int C,
                                const int32_t *frozen, const uint16_t *z_t, uint16_t *z,
                                hipStream_t st);

// Encoder cache entries: for rows m = b * n + i of h [B * n, d], k = h Wk^T
// and v = h Wv^T go to rows pos + i of the (b, kv head) slices of the caches
// K, V [B, Hkv, Pst, hd].
hipError_t launch_kv_encode_bf16(const uint16_t *h, const uint16_t *Wk, const uint16_t *Wv,
                                 const Shape &s, int n, int pos, int Pst, uint16_t *K, uint16_t *V,
                                 hipStream_t st);

// ---- mixture-of-experts MLP (k_moe.hip; expert GEMMs in k_gemm.hip) ----
constexpr int kMoeMaxExperts = 64;
constexpr int kMoeTile = 64;   // rows per expert tile of the grouped GEMMs
// Router logits of m [R, d] against Wr [X, d], top_k experts per token (ties
// to the lower expert) with softmax weights: sel, wts [R * top_k]. With list
// non-null, also the entries q = token * top_k + slot grouped by expert
// (list [R * top_k]), entry offsets offs [X + 1] and kMoeTile-row tile
// offsets toff [X + 1].
hipError_t launch_moe_route(bool bf16, const void *m, const void *Wr, int R, int d, int X, int top_k,
                            int32_t *sel, float *wts, int32_t *list, int32_t *offs, int32_t *toff,
                            hipStream_t st);
// Expert GEMMs over the grouped entries: hid [R * top_k, F] = round(gelu(.) *
// (.)) from the packed gate/up rows of each expert (Wgu [X, 2F, d]), and
// y [R * top_k, d] = hid Wd_e^T in fp32 (Wd [X, d, F]). d, F % 128 == 0.
hipError_t launch_moe_experts_bf16(const uint16_t *m, const uint16_t *Wgu, const uint16_t *Wd,
                                   const int32_t *list, const int32_t *offs, const int32_t *toff,
                                   int R, int top_k, int X, int d, int F, uint16_t *hid, float *y,
                                   hipStream_t st);
// fp32 experts directly from sel (no grouping): hid [n, F], y [n, d].
hipError_t launch_moe_experts_f32(const float *m, const int32_t *sel, const float *Wg, const float *Wu,
                                  const float *Wd, int n, int top_k, int d, int F, float *hid, float *y,
                                  hipStream_t st);
// out [R, d] = round(h + sum_j wts[r, j] y[r * top_k + j]).
hipError_t launch_moe_combine(bool bf16, const void *h, const float *y, const float *wts, int R, int d,
                              int top_k, void *out, hipStream_t st);

// ---- k_attention.hip (bf16 MFMA) ----
int attention_splits(const Shape &s);
size_t attention_workspace_bytes(const Shape &s);
hipError_t launch_attention_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                 const uint16_t *Kp, const uint16_t *Vp, const Shape &s,
                                 void *work, uint16_t *o, hipStream_t st);

// ---- k_lmhead.hip (bf16 MFMA) ----
bool lmhead_supported(const Shape &s);
int lmhead_splits(const Shape &s);
size_t lmhead_workspace_bytes(const Shape &s);
// The LM head reads E from a tile-major copy (lmhead_copy_bytes, filled once
// by launch_lmhead_relayout from the row-major [V, d] matrix).
size_t lmhead_copy_bytes(const Shape &s);
hipError_t launch_lmhead_relayout(const uint16_t *E, const Shape &s, uint16_t *Et, hipStream_t st);
// Fused LM head over V splits (E: the tile-major copy); writes RowPartial
// [splits, R] and z partials [splits, R, d] bf16 into `work`, and raw scaled
// logits into p0 when non-null. With `entropy` every row draws (no
// Bernoulli) and the entropy statistics of RowPartial are filled in.
hipError_t launch_lmhead_bf16(const uint16_t *h1, const uint16_t *E, const int32_t *x_t,
                              const StepParams *prm, const Shape &s, uint64_t seed, void *work,
                              float *p0, bool entropy, hipStream_t st);

// ---- k_fp32.hip (fp32 VALU path, any shape) ----
hipError_t launch_qkv_f32(const float *h0, const float *Wq, const float *Wk, const float *Wv,
                          const Shape &s, float *q, float *k, float *v, hipStream_t st);
hipError_t launch_attention_f32(const float *q, const float *k, const float *v, const float *Kp,
                                const float *Vp, const Shape &s, float *o, hipStream_t st);
// Encoder cache entries from tokens x[b * ld + i], i < n (out-of-range tokens
// embed as zero rows), into rows pos + i of K, V [B, Hkv, Pst, hd].
hipError_t launch_kv_encode_f32(const float *E, const int32_t *x, int ld, const float *Wk,
                                const float *Wv, const Shape &s, int n, int pos, int Pst, float *K,
                                float *V, hipStream_t st);
hipError_t launch_oproj_f32(const float *o, const float *Wo, const float *h0, const Shape &s,
                            float *h1, hipStream_t st);
size_t lmhead_f32_workspace_bytes(const Shape &s);
hipError_t launch_ffw_gate_up_f32(const float *u, const float *Wg, const float *Wu, int M, int d,
                                  int F, float *hid, hipStream_t st);
// z = res + hid Wd^T (res may be null: 0).
hipError_t launch_ffw_down_f32(const float *hid, const float *Wd, int M, int d, int F, int C,
                               const int32_t *frozen, const float *z_t, float *z, hipStream_t st,
                               const float *res = nullptr);
hipError_t launch_lmhead_f32(const float *h1, const float *E, const StepParams *prm,
                             const Shape &s, uint64_t seed, void *work, float *p0, bool entropy,
                             hipStream_t st);

// ---- k_combine.hip ----
// Merge the split partials of the LM head, draw the Step and finish z:
// x_out, z_out (act), lse, best (each optional except x_out/z_out).
// With `ent` (entropy-bounded step) the per-row entropy, draw and argmax go
// to ent instead of a Step select into x_out; rows of canvases marked in
// `frozen` (nullable) copy z_t to z_out instead.
// With `h0_next` (Step sampler only: no ent, no frozen) the merge also writes
// the next step's embedding h0_next = round(E[x_out] + z_out) (E row-major
// [V, d], tokens outside [0, V) as zero rows), exactly what the embedding
// pass would compute from x_out and z_out; combine_embeds_next tells whether
// it can for these arguments (bf16, the many-lane merge).
bool combine_embeds_next(bool bf16, const void *work, int splits, const Shape &s, const void *z_out);
hipError_t launch_combine(bool bf16, const void *work, int splits, const int32_t *x_t,
                          const StepParams *prm, const Shape &s, uint64_t seed, int32_t *x_out,
                          void *z_out, float *lse, int32_t *best, const EntropyRows *ent,
                          const int32_t *frozen, const void *z_t, hipStream_t st,
                          const void *E = nullptr, void *h0_next = nullptr);

// ---- k_select.hip ----
constexpr int kSelectMaxC = 1024;   // canvas positions the select kernel sorts in LDS
// Entropy-bounded acceptance, uniform re-noise and the stop test, one block
// per canvas. `det_prev` (nullable) holds the previous step's argmax
// predictions; with `stopped` (nullable) a canvas already marked there keeps
// x_t and det_prev, and a canvas that stops now is marked and records
// step + 1 in steps_out (nullable).
hipError_t launch_entropy_select(const EntropyRows &ent, const int32_t *x_t,
                                 const int32_t *det_prev, int B, int C, int V, float eps_accept,
                                 float eps_stop, uint64_t seed, int step, int32_t *x_out,
                                 int32_t *det_out, float *entropy_out, int32_t *stop_out,
                                 int32_t *stopped, int32_t *steps_out, hipStream_t st);

}  // namespace dg
