/*
 * dg.h -- C ABI of libdg, the block-canvas denoising step on gfx950 (MI355X).
 *
 * The method is the one summarised on the hyper.ai page for the
 * DiffusionGemma Technical Report ("TR summary" below), section Method:
 *   - forward path: per coordinate kappa_t delta(x_t, x_0) + (1 - kappa_t)/V,
 *     kappa_0 = 1 to kappa_1 = 0, smooth and decreasing (forward path eq.);
 *   - decoder: L_t = Decoder(x_t, z_t, H), bidirectional attention inside the
 *     canvas plus cross-attention to the KV cache H (decoder eq. and the
 *     three-stage generation pipeline);
 *   - iteration: p0 = Softmax(L_t / tau_t), z = FFW(p0 E),
 *     x_{t-dt} ~ Step(x_t, p0) (three-line update);
 *   - tau_t anneals linearly from 0.8 to 0.4 (sampler paragraph).
 * Readings where the pages stop short: Step is the Euler step of the
 * uniform-path CTMC, (1 - lambda) delta(y, x_t) + lambda p0(y) with
 * lambda = clamp(dt (-dkappa/dt) / (1 - kappa_t), 0, 1); FFW is the identity
 * unless a gated feed-forward block is attached (dg_set_ffw);
 * the decoder is one residual attention block (h0 = E[x] + z; q,k,v = h0 W^T;
 * one joint unmasked softmax over [prefix ; canvas] keys, scale 1/sqrt(hd),
 * query head h reads kv head h / (Hq/Hkv); h1 = h0 + o Wo^T) with the LM head
 * tied to E; tau_t = 0.4 + 0.4 t.
 *
 * Random numbers: Philox4x32-10 (Salmon et al., SC'11), key = (lo32(seed),
 * hi32(seed)), counter (c0, c1, c2, stream):
 *   Gumbel noise   (16 (v >> 6) + (v & 15), i, b, 0), word (v >> 4) & 3;
 *                  G = -log(-log U)
 *   Step Bernoulli (0, i, b, 1), word 0;              resample iff U < lambda_b
 *   corruption     (i >> 1, 0, b, 2), words 2(i&1) (keep iff U < kappa_b)
 *                  and 2(i&1)+1 (token floor(w V / 2^32))
 * with U(w) = (2 (w >> 9) + 1) 2^-24, i the canvas position, b the canvas.
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library
 *     never frees them. Arrays documented as "host" are read on the host
 *     before the call returns.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream). Nothing synchronises the device.
 *   - Every argument is checked on the host before any launch; on error
 *     nothing is launched or written and dg_last_error() holds a message
 *     (thread-local). No C++ exception crosses this boundary.
 *   - A dg_model is not thread-safe: calls on one model must be ordered on
 *     one stream or otherwise serialised by the caller.
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DG_OK = 0,
  DG_ERR_INVALID_ARG = 1, /* null pointer, out-of-range value, aliasing   */
  DG_ERR_UNSUPPORTED = 2, /* valid shape the kernels do not implement     */
  DG_ERR_HIP = 3,         /* a HIP runtime call or a kernel launch failed */
  DG_ERR_OOM = 4          /* device or pinned-host allocation failed      */
} dg_status;

enum { DG_DTYPE_F32 = 0, DG_DTYPE_BF16 = 1 };
enum { DG_SCHEDULE_LINEAR = 0, /* kappa = 1 - t            */
       DG_SCHEDULE_COSINE = 1  /* kappa = cos^2(pi t / 2)  */ };

/* Shapes of one model instance.
 *   B canvases of C tokens, prompt prefix of P tokens per canvas, width d,
 *   n_q_heads query heads and n_kv_heads KV heads of head_dim each
 *   (n_q_heads % n_kv_heads == 0), vocabulary V.
 *   dtype: DG_DTYPE_F32 or DG_DTYPE_BF16 -- the storage type of weights, KV
 *   cache, activations and z ("act" below); accumulation is always fp32.
 *   Limits (DG_ERR_INVALID_ARG): B, C, d, heads, head_dim >= 1, P >= 0,
 *   V >= 2, B*C*d and B*C*n_q_heads*head_dim < 2^31.
 *   Kernel coverage (DG_ERR_UNSUPPORTED otherwise): bf16 needs head_dim in
 *   {64, 128, 176}, d in {256, 512, 1024, 2048, 2816} and V % 16 == 0; fp32
 *   needs d <= 4096 and P + C <= 16384. */
typedef struct dg_config {
  int32_t B, C, P, d, n_q_heads, n_kv_heads, head_dim, V;
  int32_t dtype;
  int32_t schedule;
} dg_config;

/* Weights, device pointers in act dtype, row-major, caller-owned and
 * read-only for the model's lifetime:
 *   E  [V, d]            token embedding, also the tied LM head
 *   Wq [Hq*hd, d]        q = h0 Wq^T    (output-feature major)
 *   Wk [Hkv*hd, d], Wv [Hkv*hd, d]
 *   Wo [d, Hq*hd]        h1 = h0 + o Wo^T */
typedef struct dg_weights {
  const void *E, *Wq, *Wk, *Wv, *Wo;
} dg_weights;

/* Optional intermediate outputs of one step (all device pointers, each may be
 * NULL). Rows r = b*C + i.
 *   h0 [B,C,d] act; q [B,C,Hq,hd] act; k, v [B,Hkv,C,hd] act;
 *   o [B,C,Hq,hd] act (attention output); h1 [B,C,d] act;
 *   lse [B,C] f32 = logsumexp_v(s_v) of the scaled logits s = (h1 E^T)/tau_b;
 *   p0 [B,C,V] f32 = exp(s - lse) (extra passes; for checking only);
 *   best [B,C] int32 = Gumbel argmax for rows that resampled, -1 for kept rows;
 *   p0E [B,C,d] act = p0 E, the input of the feed-forward block (written only
 *   while a block is attached; z_out then holds FFW(p0E)). */
typedef struct dg_taps {
  void *h0, *q, *k, *v, *o, *h1;
  float *lse, *p0;
  int32_t *best;
  void *p0E;
} dg_taps;

typedef struct dg_model dg_model;

/* Create a model over caller-owned weights. Allocates the library's own
 * device workspace (activations, split partials, per-step constants,
 * generation buffers and, for bf16, a tile-major copy of E that the LM head
 * reads: E must keep its values while the model lives); per-call host arrays
 * reach the device as kernel arguments, so no host memory outlives a call.
 * Binds to the HIP device that is current at the time of the call; later
 * calls must run with that device current. Weight pointers must be 16-byte
 * aligned. Waits for the copy of E to finish. *out is set only on DG_OK. */
dg_status dg_create(const dg_config *cfg, const dg_weights *w, dg_model **out);

/* Frees the workspace; waits for the device to finish work already queued
 * on the model's buffers. NULL is accepted. */
dg_status dg_destroy(dg_model *m);

/* Bytes of device workspace dg_create would allocate for cfg. */
dg_status dg_workspace_bytes(const dg_config *cfg, size_t *bytes);

/* Forward corruption x_t ~ kappa delta(., x0) + (1 - kappa)/V per token
 * (TR summary, Method, forward path eq.).
 *   x0 [B,C] int32 in [0, V); kappa host [B], each in [0, 1];
 *   xt_out [B,C] int32, must not overlap x0. */
dg_status dg_corrupt(dg_model *m, const int32_t *x0, const float *kappa, uint64_t seed,
                     int32_t *xt_out, void *stream);

/* The same corruption without a model, for any batch shape:
 *   x0 [B,C] int32, kappa_dev DEVICE [B] f32 in [0,1] (not checked on the
 *   host), xt_out [B,C] int32 (may equal x0: the kernel reads each token
 *   before writing it). */
dg_status dg_corrupt_batch(const int32_t *x0, const float *kappa_dev, int32_t B, int32_t C,
                           int32_t V, uint64_t seed, int32_t *xt_out, void *stream);

/* One denoising step for every canvas (TR summary, Method, decoder eq. and
 * three-line update):
 *   x_t [B,C] int32 in [0,V); z_t [B,C,d] act; K_pre, V_pre [B,Hkv,P,hd] act
 *   (the prompt KV cache H); t host [B], each in (0, 1]; dt in (0, 1];
 *   seed = the Philox key of this step.
 *   Outputs: x_out [B,C] int32 (the Step draw), z_out [B,C,d] act
 *   (z = FFW(p0 E): p0 E itself unless a block is attached with dg_set_ffw),
 *   optional lse_out [B,C] f32, optional p0_out [B,C,V] f32
 *   (p0_out requires lse_out). x_out / z_out must not overlap x_t / z_t;
 *   bf16 tensors must be 16-byte aligned. The C x V logits are never written
 *   unless p0_out is given. Tokens outside [0, V) embed as a zero row. */
dg_status dg_denoise_step(dg_model *m, const int32_t *x_t, const void *z_t, const void *K_pre,
                          const void *V_pre, const float *t, float dt, uint64_t seed,
                          int32_t *x_out, void *z_out, float *lse_out, float *p0_out,
                          void *stream);

/* dg_denoise_step with every intermediate exposed through `taps` (may be NULL). */
dg_status dg_denoise_step_taps(dg_model *m, const int32_t *x_t, const void *z_t,
                               const void *K_pre, const void *V_pre, const float *t, float dt,
                               uint64_t seed, int32_t *x_out, void *z_out, const dg_taps *taps,
                               void *stream);

/* dg_denoise_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * no model object and no allocation of any kind in the call. The step's
 * whole workspace (activations, attention and LM-head split partials, the LM
 * head's tile-major copy of E, step constants) is carved from a static
 * device array of 64 MiB that each GPU the library runs on holds until the
 * process ends.
 *   cfg, w: as dg_create (checked the same way); every other argument as
 *   dg_denoise_step. The copy of E is remade on every call (V*d*2 bytes
 *   read and written on `stream`), so E may change between calls.
 *   Limits (DG_ERR_UNSUPPORTED, nothing launched): B <= 256 and a workspace
 *   of at most 64 MiB (dg_workspace_bytes bounds it from above; roughly
 *   V*d*2 bytes for the copy of E plus the activations, e.g. V*d <= 2^24
 *   at small B*C).
 *   Calls on one GPU share its array and it keeps the last call's contents
 *   (every byte a step reads is written earlier in the same call): calls
 *   that overlap in time on one GPU, on any streams, race and must be
 *   serialised by the caller. */
dg_status dg_denoise_step_static(const dg_config *cfg, const dg_weights *w, const int32_t *x_t,
                                 const void *z_t, const void *K_pre, const void *V_pre,
                                 const float *t, float dt, uint64_t seed, int32_t *x_out,
                                 void *z_out, float *lse_out, float *p0_out, void *stream);

/* Generate B canvases from noise (TR summary, Method, three-line update
 * iterated from t = 1; Experiments: about 12 and at most 48 steps).
 *   x_init = corruption of any canvas at kappa = 0 with `seed` (uniform),
 *   z = 0; for k = 0..steps-1: t_k = (float)(1 - k/steps), dt = (float)(1/steps),
 *   step seed = seed + k (mod 2^64). steps in [1, 4096].
 *   x_out [B,C] int32 final canvas; z_out [B,C,d] act final z (may be NULL). */
dg_status dg_generate_canvas(dg_model *m, const void *K_pre, const void *V_pre, int32_t steps,
                             uint64_t seed, int32_t *x_out, void *z_out, void *stream);

/* Entropy-bounded step, the recommended sampler (TR summary, Method, sampler
 * paragraph; Experiments: at most 48 steps, about 12 with adaptive stopping).
 * Same decoder, temperature and z as dg_denoise_step at time t; then, per
 * canvas (readings of the pages, which give no formula):
 *   H_i = entropy of p0_i in nats; positions taken in increasing H (ties by
 *   position) are accepted while the running sum of H stays < eps_accept, and
 *   at least the first; an accepted position takes the Gumbel-max draw of
 *   p0 (the Step path's noise); every other position is re-noised with
 *   floor(w V / 2^32), w = word 0 of Philox block (0, i, b, 3);
 *   det_out = argmax_v of the scaled logits (lowest id on ties);
 *   stop_out[b] = 1 iff det_prev is given, the mean of H over the canvas is
 *   < eps_stop and det_out equals det_prev at every position.
 *   det_prev [B,C] int32 may be NULL (first step: never stops);
 *   entropy_out [B,C] f32 may be NULL. C <= 1024 (DG_ERR_UNSUPPORTED else).
 *   x_out / z_out / det_out must not overlap x_t / z_t / det_prev. */
dg_status dg_denoise_step_entropy(dg_model *m, const int32_t *x_t, const void *z_t,
                                  const void *K_pre, const void *V_pre, const float *t,
                                  uint64_t seed, float eps_accept, float eps_stop,
                                  const int32_t *det_prev, int32_t *x_out, void *z_out,
                                  int32_t *det_out, float *entropy_out, int32_t *stop_out,
                                  void *stream);

/* Generate B canvases with the entropy-bounded step and adaptive stopping:
 * x_init and z = 0 as dg_generate_canvas; step k (t_k = 1 - k/max_steps,
 * seed + k) runs dg_denoise_step_entropy with the previous step's argmax
 * (none at k = 0); a canvas that stops keeps its tokens and z from then on
 * and steps_out[b] (device int32 [B]) receives the number of steps it took
 * (max_steps if it never stopped). Every 4 steps the call synchronises the
 * stream to end early once every canvas has stopped. x_out [B,C] int32 and
 * z_out [B,C,d] act (may be NULL) receive the final canvases. */
dg_status dg_generate_canvas_entropy(dg_model *m, const void *K_pre, const void *V_pre,
                                     int32_t max_steps, uint64_t seed, float eps_accept,
                                     float eps_stop, int32_t *x_out, void *z_out,
                                     int32_t *steps_out, void *stream);

/* Prompt prefill and canvas commit (TR summary, Method: the pipeline
 * figure's causal encoder fills the KV cache from the prompt, and each clean
 * canvas goes back through it and is appended to the cache). Reading: the
 * encoder shares the decoder's weights, and a single attention block's cache
 * entries of a token are its key and value projections with no
 * self-conditioning input, k = E[x] Wk^T and v = E[x] Wv^T (rounded to act),
 * so prefill and commit are one operation.
 * With a decoder stack attached (dg_set_stack) the encoder is the stack's
 * causal pass: h = E[x]; per layer a = rmsnorm(h) g_attn, the layer's cache
 * entries k = a Wk^T, v = a Wv^T, and (every layer but the last) attention
 * of each new token over the cache rows below it and the new tokens up to
 * itself, h += o Wo^T, h += MLP(rmsnorm(h) g_mlp); tokens go through in
 * chunks of at most C, each seeing the earlier chunks as history.
 *   tokens [B, n] int32 (a token outside [0, V) embeds as a zero row);
 *   K_cache, V_cache [B, Hkv, P, hd] act ([L, B, Hkv, P, hd] with a stack
 *   of L layers): the model's P is the cache capacity; rows [pos, pos + n)
 *   of every (layer, canvas, kv head) slice are written, nothing else.
 *   Needs n >= 0, pos >= 0 and pos + n <= P. */
dg_status dg_encode_kv(dg_model *m, const int32_t *tokens, int32_t n, int32_t pos, void *K_cache,
                       void *V_cache, void *stream);

/* Block-autoregressive generation (TR summary, Method: one canvas of C
 * tokens at a time; a finished canvas is committed to the cache and the next
 * one starts). With the prompt's entries in cache rows [0, P0), canvas
 * j = 0 .. n_canvases-1 is generated exactly as dg_generate_canvas with
 * `steps` steps and seed seed + j * steps, attending to cache rows
 * [0, P0 + j C) only; its final tokens are then encoded into rows
 * [P0 + j C, P0 + (j + 1) C) (dg_encode_kv).
 *   K_cache, V_cache [B, Hkv, P, hd] act ([L, B, Hkv, P, hd] with a stack),
 *   read and extended in place;
 *   P0 + n_canvases * C <= P; x_out [B, n_canvases, C] int32. */
dg_status dg_generate_blocks(dg_model *m, void *K_cache, void *V_cache, int32_t P0,
                             int32_t n_canvases, int32_t steps, uint64_t seed, int32_t *x_out,
                             void *stream);

/* dg_generate_blocks with the recommended sampler: canvas j is generated
 * exactly as dg_generate_canvas_entropy with at most max_steps steps and seed
 * seed + j * max_steps, against cache rows [0, P0 + j C), then committed.
 *   x_out [B, n_canvases, C] int32; steps_out [B, n_canvases] int32 (device):
 *   the steps each canvas took. Synchronises the stream every 4 steps (the
 *   early-stop poll of adaptive generation). */
dg_status dg_generate_blocks_entropy(dg_model *m, void *K_cache, void *V_cache, int32_t P0,
                                     int32_t n_canvases, int32_t max_steps, uint64_t seed,
                                     float eps_accept, float eps_stop, int32_t *x_out,
                                     int32_t *steps_out, void *stream);

/* Gated feed-forward self-conditioning block (TR summary, Method, three-line
 * update: z = FFW(p0 E) with a standard feed-forward network; the pages give
 * no structure, the reading here is the Gemma family's gated form):
 *   FFW(u) = W_down (gelu(W_gate u) * (W_up u)), gelu in its tanh form
 *   a/2 (1 + tanh(sqrt(2/pi) (a + 0.044715 a^3))), no biases, no residual;
 *   the hidden activations are rounded to act before W_down.
 * dg_set_ffw attaches the block to every later step and generation of the
 * model (hidden = 0 detaches it: z = p0 E again).
 *   W_gate, W_up [hidden, d] and W_down [d, hidden]: device pointers in act
 *   dtype, row-major, 16-byte aligned, caller-owned and unchanged while
 *   attached. The library allocates its own buffers for the block (the
 *   input and hidden activations, and for bf16 a copy of W_gate and W_up
 *   with their rows interleaved in groups of 32), freed on detach or
 *   dg_destroy. Waits for the device before and after (set-up call).
 *   bf16 needs hidden % 64 == 0 (DG_ERR_UNSUPPORTED); B*C*hidden and
 *   hidden*d must be < 2^31. */
dg_status dg_set_ffw(dg_model *m, int32_t hidden, const void *W_gate, const void *W_up,
                     const void *W_down);

/* Multi-layer decoder stack (the TR summary's decoder is a deep transformer
 * whose layers the pages do not describe; this stand-in uses the Gemma
 * family's pre-norm layout with the parts of the single block). With a stack
 * of L layers attached, every step and generation computes, from
 * h = E[x] + z:
 *   per layer l: a = rmsnorm(h) g_attn; q, k, v = a W^T; attention over
 *   [cache slice l ; canvas]; h = h + o Wo^T; a = rmsnorm(h) g_mlp;
 *   h = h + W_down (gelu(W_gate a) * (W_up a));
 *   LM head input = rmsnorm(h_L) g_final;
 * rmsnorm(x) = x / sqrt(mean(x^2) + 1e-6), everything rounded to act at each
 * tensor. K_pre / V_pre of the step and generation calls are then
 * [L, B, Hkv, P, hd] (one cache slice per layer). dg_weights' Wq..Wo are not
 * used while a stack is attached (E still is). Taps: h0 is the embedding,
 * q, k, v, o those of the last layer, h1 the LM head's input.
 *   layers: host array [n_layers] of device pointers in act dtype, 16-byte
 *   aligned, caller-owned and unchanged while attached: Wq..Wo as dg_weights,
 *   g_attn, g_mlp [d], W_gate, W_up [mlp_hidden, d], W_down [d, mlp_hidden];
 *   g_final [d]. n_layers = 0 detaches (the single block again).
 * The library allocates the stack's activations and, for bf16, a copy of
 * each layer's W_gate/W_up with rows interleaved in groups of 32; waits for
 * the device (set-up call). bf16 needs mlp_hidden % 64 == 0
 * (DG_ERR_UNSUPPORTED). dg_encode_kv and block generation then run the
 * stack's causal encoder pass (see dg_encode_kv). */
typedef struct dg_layer_weights {
  const void *Wq, *Wk, *Wv, *Wo;
  const void *g_attn, *g_mlp;
  const void *W_gate, *W_up, *W_down;
} dg_layer_weights;
dg_status dg_set_stack(dg_model *m, int32_t n_layers, int32_t mlp_hidden,
                       const dg_layer_weights *layers, const void *g_final);

/* dg_set_stack with a mixture of experts in every layer's MLP (the TR
 * summary's model is a sparse mixture of experts that activates a few of
 * many experts per token; the routing rule is a reading): router logits
 * r = a W_router^T in fp32, the top_k experts by logit (ties to the lower
 * expert), weights = softmax over the selected logits, and the MLP output
 * sum_j w_j W_down_e (gelu(W_gate_e a) * (W_up_e a)) (each expert's hidden
 * activations rounded to act, the weighted sum rounded once into h).
 *   layers[l].W_gate, W_up: [n_experts, mlp_hidden, d], W_down:
 *   [n_experts, d, mlp_hidden] (expert-major); W_router: host array
 *   [n_layers] of device pointers [n_experts, d]. 1 <= top_k <= n_experts
 *   <= 64. bf16 needs mlp_hidden % 128 == 0 and d % 128 == 0
 *   (DG_ERR_UNSUPPORTED). n_experts = 0 is dg_set_stack. */
dg_status dg_set_stack_moe(dg_model *m, int32_t n_layers, int32_t mlp_hidden, int32_t n_experts,
                           int32_t top_k, const dg_layer_weights *layers,
                           const void *const *W_router, const void *g_final);

/* z_out [B,C,d] act = FFW(u) for u [B,C,d] act through the attached block
 * (DG_ERR_INVALID_ARG if none); z_out must not overlap u. */
dg_status dg_ffw(dg_model *m, const void *u, void *z_out, void *stream);

/* Per-stage GPU time of the calls made while profiling is on, measured with a
 * HIP event pair recorded on the call's stream around each stage's launches.
 * Stages: 0 embed, 1 q/k/v projection, 2 attention (+ split merge),
 * 3 output projection, 4 LM head (logits, softmax statistics, z partials,
 * Gumbel argmax), 5 split merge + Step select, 6 corruption, 7 feed-forward
 * self-conditioning block, 8 encoder (prefill / commit), 9 decoder-stack norms
 * and MLPs (the stack's attention blocks count under 1-3).
 * dg_profile_enable(m, mask) times the stages whose bit (1 << stage) is set
 * in mask (0 turns profiling off; every event pair adds a few microseconds of
 * queue time between kernels, so time only the stages you need).
 * dg_profile_read waits for the recorded events, returns the summed
 * milliseconds and the number of timed launches per stage, and clears them. */
#define DG_NUM_STAGES 10
typedef struct dg_profile {
  double ms[DG_NUM_STAGES];
  int64_t count[DG_NUM_STAGES];
} dg_profile;
dg_status dg_profile_enable(dg_model *m, int mask);
dg_status dg_profile_read(dg_model *m, dg_profile *out);

const char *dg_status_string(dg_status s);
/* Message of the last failed call on this thread ("" if none). */
const char *dg_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
