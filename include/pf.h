/*
 * pf.h - C ABI of one pipeline stage of patch-level (PipeFusion-style) DiT
 * inference on an AMD Instinct MI355X (gfx950).
 *
 * The method (PipeFusion technical summaries, gist.science Korean page and French
 * page, "Core mechanisms"):
 *   - dual partitioning: a stage owns L contiguous transformer layers, and the token
 *     sequence is split into M non-overlapping patches that flow through the stage's
 *     layers one patch at a time (mechanism 1);
 *   - temporal redundancy: attention in step T uses stale step-(T+1) activations as
 *     context for the rows not yet recomputed, instead of waiting for fresh ones
 *     (mechanism 2);
 *   - memory: the stage keeps full-spatial K and V only for its own layers, one buffer
 *     per layer (mechanism 4);
 *   - the DiT keeps full attention over the whole image (Key contributions).
 *
 * Conventions shared by every call:
 *   - All pointers named "device" are device memory of the current HIP device and must
 *     be 16-byte aligned.  Row strides ("ld") are in elements and must keep every row
 *     16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Every call only
 *     enqueues work on that stream and returns; no call synchronises the host.
 *   - Every argument is validated before anything is enqueued: a call that returns an
 *     error has enqueued nothing and written nothing.  pf_last_error() then describes
 *     the failure.  Errors are status codes; nothing aborts or throws across the ABI.
 *   - A device fault shows up on the caller's next synchronisation; after a failed HIP
 *     call a stage returns PF_ERR_HIP from every later call.
 *   - One stage object is used from one stream at a time; there is no internal locking.
 *   - bf16 is bfloat16 (round to nearest even on every fp32 -> bf16 conversion).  bf16
 *     contractions accumulate in fp32; softmax statistics are fp32; the residual stream
 *     and the stage's input/output rows are fp32.
 */
#ifndef PF_H
#define PF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pf_status {
  PF_OK = 0,
  PF_ERR_INVALID_ARG = 1,   /* a pointer, size, stride or range is invalid            */
  PF_ERR_UNSUPPORTED = 2,   /* valid but not implemented (e.g. head_dim 96, not gfx950) */
  PF_ERR_OOM = 3,           /* device allocation failed                                */
  PF_ERR_STATE = 4,         /* call order violated (weights or condition not set)      */
  PF_ERR_HIP = 5            /* a HIP runtime call failed                               */
} pf_status;

typedef enum pf_dtype { PF_BF16 = 0, PF_FP32 = 1 } pf_dtype;
typedef enum pf_gelu { PF_GELU_TANH = 0, PF_GELU_ERF = 1 } pf_gelu;

/* Row layout of a K or V buffer.
 *   PF_LAYOUT_ROWS: element (r, c) at r * ld + c.
 *   PF_LAYOUT_K8:   rows are interleaved in groups of 8: element (r, c) at
 *                   ((r / 8) * row_elems + c) * 8 + (r % 8).  A row range [8a, 8b) is one
 *                   contiguous block; 8 consecutive rows of one column are 16 contiguous
 *                   bytes (the operand order of the attention kernel's P.V product).
 *                   `ld` is ignored and storage covers ceil(rows / 8) * 8 rows. */
typedef enum pf_layout { PF_LAYOUT_ROWS = 0, PF_LAYOUT_K8 = 1 } pf_layout;

/* Epilogues of pf_gemm (y = a . w^T + bias, a [m,k], w [n,k], y [m,n]). */
typedef enum pf_epilogue {
  PF_EPI_STORE = 0,          /* c[i,j] = y (stored in `dtype`)                          */
  PF_EPI_GELU_TANH = 1,      /* c[i,j] = gelu_tanh(y)                                    */
  PF_EPI_GELU_ERF = 2,       /* c[i,j] = gelu_erf(y)                                     */
  PF_EPI_GATED_RESIDUAL = 3  /* c[i,j] += gate[j] * y, c is fp32 (the residual stream)  */
} pf_epilogue;

#define PF_STEP_WARMUP 1u    /* stage_run_step flag: run all buffer rows as one patch */
#define PF_MAX_STAGE_BATCH 8 /* largest pf_stage_config.batch                          */

/* Block options (pf_stage_config.flags) of the MM-DiT variants the pages evaluate (SD3,
 * Flux.1; Experiments section).  The pages name the models, not their blocks; these follow
 * the published designs.  bf16 stages only.
 *   PF_STAGE_QK_NORM:     per-head RMSNorm of Q and K after the projection (eps 1e-6), scaled
 *                         by the layer's q_norm / k_norm vectors [d];
 *   PF_STAGE_DUAL_STREAM: the text-prefix rows use a second weight set (stage_load_text_weights):
 *                         their own projections, modulation and gates; attention stays joint
 *                         over every buffer row;
 *   PF_STAGE_ROPE:        rotary embedding of Q and K (after the norm): in every head, the pair
 *                         (2k, 2k+1) of buffer row r turns by angles[r][k] (stage_set_rope);
 *   PF_STAGE_PARALLEL:    the Flux.1 single-stream block: attention and MLP side by side on one
 *                         modulated LayerNorm, h1 = LN(x) (1 + scale) + shift, Q/K/V from h1,
 *                         u = GELU(h1 W1^T + b1), x += gate * ([O, u] W2^T + b2).  Weights:
 *                         w_qkv [3h, h], w1 [rh, h], w2 [h, h + rh] (columns [0, h) act on the
 *                         attention output), w_ada [3h, h] and b_ada [3h] (shift, scale, gate);
 *                         w_o / b_o are not used.  Not combined with PF_STAGE_DUAL_STREAM. */
#define PF_STAGE_QK_NORM 1u
#define PF_STAGE_DUAL_STREAM 2u
#define PF_STAGE_ROPE 4u
#define PF_STAGE_PARALLEL 8u

typedef struct pf_stage_config {
  int32_t num_layers;   /* L >= 1: contiguous layers owned by this stage                   */
  int32_t hidden;       /* h = heads * head_dim                                             */
  int32_t heads;        /* H >= 1                                                           */
  int32_t head_dim;     /* d in {64, 72, 128}                                               */
  int32_t mlp_ratio;    /* r >= 0; 0 = attention sublayer only                              */
  int32_t num_patches;  /* M >= 1; seq_img % M == 0                                         */
  int64_t seq_img;      /* image rows, >= 1                                                 */
  int64_t seq_txt;      /* text-prefix rows (>= 0), kept at buffer rows [0, seq_txt)        */
  int32_t dtype;        /* pf_dtype of weights, activations and KV buffers                  */
  int32_t gelu;         /* pf_gelu of the MLP                                               */
  float ln_eps;         /* LayerNorm epsilon (1e-6 is the DiT value)                        */
  uint32_t flags;       /* PF_STAGE_* block options (0: the plain DiT block)                 */
  int32_t batch;        /* samples sharing the weights, 0 or 1 = one; 2 = a classifier-free  */
                        /* guidance pair.  Each sample has its own condition, rows and K/V  */
                        /* buffers; the projections run once over all samples' rows.       */
} pf_stage_config;

/* One layer's parameters, all device pointers, weights in the stage dtype, row-major
 * [out, in] (nn.Linear layout), biases fp32.  W_qkv rows are Q (0..h), K (h..2h),
 * V (2h..3h); head j owns columns [j*d, (j+1)*d) of each.  W_ada rows are the six
 * modulation vectors shift1, scale1, gate1, shift2, scale2, gate2 (h rows each).
 * w1/b1/w2/b2 may be NULL when mlp_ratio == 0.  PF_STAGE_PARALLEL changes the shapes of w2
 * ([h, h + rh]) and w_ada / b_ada ([3h, h], [3h]); w_o / b_o may then be NULL, and w2 / b2
 * are required even when mlp_ratio == 0. */
typedef struct pf_layer_weights {
  const void* w_qkv;  const float* b_qkv;   /* [3h, h], [3h]   */
  const void* w_o;    const float* b_o;     /* [h, h],  [h]    */
  const void* w1;     const float* b1;      /* [rh, h], [rh]   */
  const void* w2;     const float* b2;      /* [h, rh], [h]    */
  const void* w_ada;  const float* b_ada;   /* [6h, h], [6h]   */
  const float* q_norm; const float* k_norm; /* [d], [d] fp32 (PF_STAGE_QK_NORM only; else ignored) */
} pf_layer_weights;

/* A pair of K and V row buffers (device memory). */
typedef struct pf_kv_view {
  void* k;
  void* v;
  int64_t rows;        /* logical rows                                          */
  int64_t row_elems;   /* elements per row                                      */
  int64_t k_ld;        /* K row stride in elements (K is always PF_LAYOUT_ROWS)  */
  int64_t v_ld;        /* V row stride in elements when v_layout == ROWS        */
  int32_t dtype;       /* pf_dtype                                              */
  int32_t v_layout;    /* pf_layout of V                                        */
} pf_kv_view;

typedef struct pf_stage pf_stage;

/* Create a stage on the current HIP device (must be gfx950).  Allocates, once, all
 * device memory the stage uses: the L layers' weights, the L per-layer K/V buffers of
 * seq_txt + seq_img rows per sample (one copy, updated in place: the stage keeps
 * full-spatial K/V for its own layers only, PipeFusion mechanism 4), and scratch for
 * seq_txt + seq_img rows of every sample.  bf16 stages keep V in PF_LAYOUT_K8, fp32 stages in PF_LAYOUT_ROWS.  Buffers
 * start zeroed.  Requires h = H * d, d in {64,72,128}, h % 64 == 0 for bf16,
 * seq_img % num_patches == 0.  Source: "Core mechanisms" 1 and 4 of the PipeFusion summaries
 * (a stage of contiguous layers over M patches; each device keeps the full-spatial K/V of its
 * own layers only).  Errors: INVALID_ARG, UNSUPPORTED, OOM, HIP; nothing is allocated on
 * failure.  *out receives the stage. */
pf_status stage_create(const pf_stage_config* cfg, pf_stage** out);

/* Free everything the stage owns.  The caller synchronises its stream first.  NULL is a
 * no-op.  Source: none on the pages (a resource call every user of a stage object needs). */
pf_status stage_destroy(pf_stage* st);

/* Copy layer `layer`'s parameters (device pointers, see pf_layer_weights) into memory
 * the stage owns (stream-ordered device-to-device copies).  The caller may release its
 * copies once the stream has passed this call.  Every layer must be loaded before any
 * run call (else PF_ERR_STATE).  Source: "Core mechanisms" 4 (memory efficiency) of the
 * PipeFusion summaries: a device holds only the parameters of its own contiguous layers,
 * 1/N of the model; and mechanism 1 (layer partitioning).  Errors: INVALID_ARG for a bad
 * layer index or a NULL pointer the configuration needs, HIP if a copy cannot be enqueued. */
pf_status stage_load_weights(pf_stage* st, int32_t layer, const pf_layer_weights* w, void* stream);

/* PF_STAGE_DUAL_STREAM: layer `layer`'s text-stream parameters (same form and rules as
 * stage_load_weights); every layer's must be loaded before any run call (else PF_ERR_STATE).
 * PF_ERR_INVALID_ARG on a stage created without PF_STAGE_DUAL_STREAM, a bad layer index or a
 * NULL pointer the options need (q_norm / k_norm with PF_STAGE_QK_NORM).  Source: the
 * Experiments section names SD3 and Flux.1 (MM-DiT models); their dual-stream block is a
 * reading of the published designs. */
pf_status stage_load_text_weights(pf_stage* st, int32_t layer, const pf_layer_weights* w, void* stream);

/* PF_STAGE_ROPE: copy the rotation angles, device fp32 [seq_txt + seq_img, head_dim / 2]
 * (row r: the angles of buffer row r, radians) into memory the stage owns (stream-ordered).
 * Must be called before any run call (else PF_ERR_STATE); calling it again replaces the table
 * for later runs.  PF_ERR_INVALID_ARG on a stage created without PF_STAGE_ROPE, a NULL or
 * misaligned (4-byte) pointer, or angles overlapping the stage's own table.  Source: as for
 * stage_load_text_weights (the rotary embedding of the MM-DiT models, a reading). */
pf_status stage_set_rope(pf_stage* st, const float* angles, void* stream);

/* Compute every layer's adaLN modulation from the conditioning vectors `cond` (device,
 * fp32 [batch, h], one per sample): mod_l,b = SiLU(cond_b) . W_ada,l^T + b_ada,l, kept by the
 * stage for later stage_run_patch calls of this diffusion step.  Source: none on the pages
 * (they name DiT models without their blocks); the per-step condition of a DiT block, a
 * reading.  Errors: INVALID_ARG (NULL cond), STATE (weights not loaded), HIP. */
pf_status stage_set_cond(pf_stage* st, const float* cond, void* stream);

/* One micro-step: push buffer rows [row_off, row_off + rows) through all L layers
 * (PipeFusion mechanism 1: one patch through the stage's contiguous layers).  In each
 * layer: LayerNorm + modulation, QKV projection, in-place splice of the rows' fresh K/V
 * into the layer's buffer, full attention of the rows' queries over all seq_txt +
 * seq_img buffer rows (rows not yet recomputed this step hold stale values from the
 * previous step, mechanism 2), output projection with gated residual, and (r > 0) the
 * modulated GELU MLP with gated residual.
 * x_in / x_out: device fp32 [batch, rows, h] (x_out may equal x_in; otherwise they must not
 * overlap).  With batch > 1, every sample's rows go through together: one projection over
 * batch * rows rows, each sample's own modulation and gates, its fresh K/V spliced into its
 * own buffers and its queries attending over its own buffer.  Requires 0 <= row_off,
 * rows >= 1, row_off + rows <= seq_txt + seq_img, weights loaded and stage_set_cond
 * called.  Source: "Core mechanisms" 1 and 2 of the PipeFusion summaries.  Errors:
 * INVALID_ARG (rows outside the buffer, NULL or misaligned x, partially overlapping x_in /
 * x_out), STATE (weights not loaded, stage_set_cond not called), HIP. */
pf_status stage_run_patch(pf_stage* st, int64_t row_off, int64_t rows, const float* x_in,
                          float* x_out, void* stream);

/* One diffusion step over all seq_txt + seq_img rows: stage_set_cond(cond), then
 *   with PF_STEP_WARMUP: stage_run_patch(0, seq_txt + seq_img)  (start-up: every buffer
 *                        row is computed fresh, so the pipeline has no stale context yet);
 *   otherwise:           stage_run_patch(0, seq_txt) if seq_txt > 0, then
 *                        stage_run_patch(seq_txt + m*P, P) for m = 0 .. M-1, P = seq_img/M.
 * x_in / x_out: device fp32 [batch, seq_txt + seq_img, h], x_out may equal x_in; cond: fp32
 * [batch, h].  Source: "Core mechanisms" 1 (M non-overlapping patches through the stage's
 * layers, one after another) and 2 (stale step-(T+1) context instead of waiting, so only the
 * start-up has no stale context: the warm-up step) of the PipeFusion summaries.  Errors:
 * INVALID_ARG (NULL or misaligned pointers, partially overlapping x_in / x_out, unknown
 * flags), STATE (weights or rotation table missing), HIP. */
pf_status stage_run_step(pf_stage* st, const float* x_in, float* x_out, const float* cond,
                         uint32_t flags, void* stream);

/* Bit copy of a row block into a K/V buffer pair:
 *   for i < len, c < row_elems:  dst.K(offset + i, c) = src.K(i, c), same for V,
 * each view addressed through its own layout.  No other byte of dst changes.  len == 0
 * is a no-op.  Requires equal dtype and row_elems, 0 <= offset, offset + len <= dst.rows,
 * len <= src.rows, and src/dst not overlapping.  Needs no stage.  This is the update that
 * makes a layer's buffer hold fresh rows for the current patch and the previous step's
 * values elsewhere.  Source: "Core mechanisms" 2 of the PipeFusion summaries (stale step-(T+1)
 * context, refreshed row block by row block).  Errors: INVALID_ARG (NULL view or pointer, bad
 * dtype, layout or strides, dtype or row_elems mismatch, rows out of range, misaligned or
 * overlapping src / dst), HIP. */
pf_status kvbuf_splice(const pf_kv_view* dst, const pf_kv_view* src, int64_t offset, int64_t len,
                       void* stream);

/* Describe layer `layer`'s K/V buffer of sample 0 (owned by the stage; valid until
 * stage_destroy): rows = seq_txt + seq_img, row_elems = k_ld = hidden, V in PF_LAYOUT_K8
 * (bf16) or PF_LAYOUT_ROWS (fp32).  Source: "Core mechanisms" 4 of the PipeFusion summaries:
 * the stage's one full-spatial K/V buffer per own layer (1/N of all layers' buffers), exposed
 * so a caller can inspect, checkpoint or perturb it (kvbuf_splice).  No HIP call; errors:
 * INVALID_ARG (NULL stage or out, bad layer). */
pf_status stage_get_kvbuf(pf_stage* st, int32_t layer, pf_kv_view* out);

/* The same for sample `sample` (0 <= sample < batch) of a batched stage.  Source: as
 * stage_get_kvbuf; a batch is the classifier-free guidance pair of the hybrid-parallelism
 * page (two conditioned passes sharing the weights).  Errors: INVALID_ARG. */
pf_status stage_get_kvbuf_sample(pf_stage* st, int32_t layer, int32_t sample, pf_kv_view* out);

/* The stage's configuration as created (batch 0 reads back as 1).  Source: none on the pages
 * (a query a user of a stage object needs).  Errors: INVALID_ARG (NULL argument). */
pf_status stage_get_config(const pf_stage* st, pf_stage_config* out);

/* Live timing of the stage's patch attention (instrumentation for benchmarks).
 * stage_profile_begin allocates 2 * max_launches HIP events (1 <= max_launches <= 2^20; it
 * replaces any earlier profile); from then on every attention launch of a run call (one per
 * layer, stream part and micro-step) is bracketed by a pair of events recorded on the run
 * call's stream, until the pairs run out.  stage_profile_end waits for the recorded events
 * (it synchronises the host with them), writes the number of timed launches and their summed
 * device duration in milliseconds, frees the events and stops the timing.  Source: the
 * pages' cost statement (attention grows quadratically with sequence length: "Problem
 * statement" of the PipeFusion summaries), which makes the attention launch the one to time.
 * Errors: INVALID_ARG, STATE (end without begin), OOM / HIP (event creation or reading). */
pf_status stage_profile_begin(pf_stage* st, int32_t max_launches);
pf_status stage_profile_end(pf_stage* st, int64_t* launches, double* attention_ms);

/* ---------------------------------------------------------------------------------
 * The denoising loop around one stage (one GPU holding every layer).  The pages put the
 * stage inside a diffusion loop (PipeFusion "Core mechanisms" 2: consecutive steps see
 * similar inputs, so each step reuses the previous step's K/V as stale context; only the
 * start-up has none) without defining the loop; this is the plainest DiT reading.  Per step:
 *   c_b  = W_t2 . SiLU(W_t1 . freq(t) + b_t1) + b_t2 + y_b,  freq(t) = [cos(t f_j), sin(t f_j)],
 *          f_j = 10000^(-j / (freq_dim/2));
 *   x_b  = [text rows x_txt_b (zeros if NULL); patches of z_b . W_patch^T + b_patch + pos],
 *          patches p x p, row-major over the grid, values (c p + dy) p + dx; pos a fixed
 *          2-D sine-cosine table (width quarters sin/cos of the patch row and column times
 *          10000^(-k / (h/4)));
 *   one stage_run_step(x, c) (PF_STEP_WARMUP for warm-up steps);
 *   eps_b = unpatchify(LN(x_b image rows) (1 + scale_b) + shift_b) . W_out^T + b_out), with
 *          (shift_b, scale_b) = SiLU(c_b) . W_fada^T + b_fada;
 *   a pair (batch 2: sample 0 conditional, sample 1 unconditional, sharing the latent) uses
 *          eps = eps_1 + guidance (eps_0 - eps_1) for both samples;
 *   z_b <- sqrt(abar_next) (z_b - sqrt(1 - abar_t) eps) / sqrt(abar_t) + sqrt(1 - abar_next) eps
 *          (DDIM, eta = 0), abar from a linear beta schedule, abar of "no next step" = 1.
 * Everything around the stage runs in fp32.
 * --------------------------------------------------------------------------------- */
typedef struct pf_denoiser pf_denoiser;

typedef struct pf_denoiser_config {
  int32_t in_channels;   /* C: latent channels                                       */
  int32_t patch;         /* p: patch edge                                            */
  int32_t grid_h;        /* patch rows; grid_h * grid_w must equal the stage's seq_img */
  int32_t grid_w;        /* patch columns                                            */
  int32_t freq_dim;      /* even width of the timestep frequency features            */
  int32_t train_steps;   /* T of the noise schedule; timesteps are in [0, T)         */
  float beta_start;      /* linear betas from beta_start to beta_end                 */
  float beta_end;
} pf_denoiser_config;

/* Device fp32 parameters (copied by denoiser_load_weights), [out, in] row-major. */
typedef struct pf_denoiser_weights {
  const float* w_patch; const float* b_patch;   /* [h, C p p], [h]         */
  const float* w_t1;    const float* b_t1;      /* [h, freq_dim], [h]      */
  const float* w_t2;    const float* b_t2;      /* [h, h], [h]             */
  const float* w_fada;  const float* b_fada;    /* [2h, h], [2h]: shift, scale */
  const float* w_out;   const float* b_out;     /* [C p p, h], [C p p]     */
} pf_denoiser_weights;

/* A loop around `st` (which it uses but does not own; destroy the denoiser first).  Allocates
 * its weights, the position table and per-step buffers on the current device.  Source: the diffusion
 * loop of "Core mechanisms" 2 (see above).  Errors: INVALID_ARG (grid does not match the
 * stage's image rows, bad sizes), OOM, HIP. */
pf_status denoiser_create(pf_stage* st, const pf_denoiser_config* cfg, pf_denoiser** out);

/* Free the loop's memory (not the stage's).  NULL is a no-op.  Source: none on the pages (a
 * resource call). */
pf_status denoiser_destroy(pf_denoiser* d);

/* Copy the loop's parameters (stream-ordered device-to-device copies).  Source: the diffusion
 * loop of "Core mechanisms" 2 (a reading).  Errors: INVALID_ARG (NULL pointer), HIP. */
pf_status denoiser_load_weights(pf_denoiser* d, const pf_denoiser_weights* w, void* stream);

/* One step from timestep t to t_next (-1: the last step).  z: device fp32
 * [batch, C, grid_h p, grid_w p], updated in place; y: device fp32 [batch, h]; x_txt: device
 * fp32 [batch, seq_txt, h] or NULL.  The stage's weights must be loaded.  Source: the
 * diffusion loop of "Core mechanisms" 2 (see above).  Errors: INVALID_ARG, STATE, HIP. */
pf_status denoiser_step(pf_denoiser* d, float* z, const float* y, const float* x_txt, int32_t t,
                        int32_t t_next, uint32_t flags, float guidance, void* stream);

/* n_steps steps over the host array `timesteps` (strictly decreasing); the first
 * warmup_steps (>= 1) run as warm-up steps.  Source: as
 * denoiser_step. */
pf_status denoiser_run(pf_denoiser* d, float* z, const float* y, const float* x_txt,
                       const int32_t* timesteps, int32_t n_steps, int32_t warmup_steps, float guidance,
                       void* stream);

/* Thread-local text of the last non-OK status returned on this thread (an empty string if
 * none; owned by the library, valid until the next failing call on this thread).  Source:
 * none on the pages (the error channel of this status-code ABI). */
const char* pf_last_error(void);

/* ---------------------------------------------------------------------------------
 * Component entry points: each runs one of the stage's kernels on its own.  The stage
 * calls the same kernels; these exist so each kernel can be checked and timed alone.
 * --------------------------------------------------------------------------------- */

/* y[i, :] = LayerNorm(x[i, :]) * (1 + scale) + shift for i < rows; LayerNorm without
 * affine, biased variance, fp32 statistics.  x fp32 [rows, hidden] (row stride hidden),
 * shift/scale fp32 [hidden], y [rows, hidden] in `dtype`.  Source: none on the pages beyond
 * "transformer layers" (mechanism 1); the DiT block's modulated LayerNorm is a reading.
 * Errors: INVALID_ARG, UNSUPPORTED (hidden not a multiple of 8 or above 6144), HIP. */
pf_status pf_ln_modulate(const float* x, int64_t rows, int32_t hidden, const float* shift,
                         const float* scale, float eps, void* y, int32_t dtype, void* stream);

/* y = a . w^T + bias with a [m, k] (row stride lda), w [n, k] (row-major), bias fp32 [n],
 * then the epilogue `epi` (pf_epilogue) into c (row stride ldc).  a/w/c in `dtype`, except
 * c is fp32 for PF_EPI_GATED_RESIDUAL (gate fp32 [n]).  fp32 accumulation.  For bf16:
 * n % 64 == 0 and k % 64 == 0.  `workspace` (device, may be NULL) lets a grid too small to
 * fill the GPU, or the few tiles of a last round, split k into slices summed by a second pass
 * (in a fixed order: deterministic);
 * calls sharing a workspace must not overlap in time (one stream, or ordered streams).
 * pf_gemm_workspace_size gives the bytes that allow the split the library would choose.
 * Tiles are 128 x 128, or 192 features x 128 tokens for a grid of whole tiles with n % 192 == 0
 * and at least 1.5 tiles per CU (either with a 2-stage ring, two workgroups per CU); the tile
 * does not change the result, which is the same sum in the same k order.  Source: the projections of the
 * transformer layers (mechanism 1; the block is a reading).  Errors: INVALID_ARG for a bad
 * pointer, size, stride or epilogue; UNSUPPORTED for bf16 shapes with n or k not a multiple
 * of 64; HIP if the launch fails. */
pf_status pf_gemm(const void* a, int64_t lda, const void* w, const float* bias, int64_t m,
                  int64_t n, int64_t k, int32_t epi, void* c, int64_t ldc, const float* gate,
                  int32_t dtype, void* workspace, uint64_t workspace_bytes, void* stream);

/* The stage's QKV projection with the KV splice in its epilogue (bf16 only): the product
 * y = a . w^T + bias with a [m, hidden] (row stride lda), w [3 hidden, hidden], bias fp32
 * [3 hidden], split by output feature: y[:, 0:h] (Q) to q (row stride ldq), y[:, h:2h] to
 * rows [row_offset, row_offset + m) of kv's K matrix and y[:, 2h:3h] to the same rows of its
 * V matrix.  kv must have row_elems == k_ld == hidden and V in the K8 layout; no other byte
 * of the buffer changes.  Each value is the bf16 rounding of its fp32 sum, identical to
 * pf_gemm(PF_EPI_STORE) followed by kvbuf_splice of the K and V columns.  This is the
 * in-place update of a layer's full-spatial buffer with the current patch's fresh K/V
 * done where the values are produced.  q, a and the buffer must not overlap.  The workspace is
 * as for pf_gemm with n = 3 hidden, k = hidden.  Source: "Core mechanisms" 2 of the PipeFusion
 * summaries, with the layer's QKV projection (mechanism 1).  Errors: UNSUPPORTED (not bf16, V not
 * K8, hidden % 64 != 0), INVALID_ARG (buffer row_elems or k_ld != hidden, rows outside the
 * buffer, NULL or misaligned pointers, bad strides), HIP. */
pf_status pf_gemm_qkv_splice(const void* a, int64_t lda, const void* w, const float* bias, int64_t m,
                             int64_t hidden, void* q, int64_t ldq, const pf_kv_view* kv, int64_t row_offset,
                             void* workspace, uint64_t workspace_bytes, void* stream);

/* The gated-residual projection and the modulated LayerNorm that reads its result, as a stage
 * runs them after the attention and MLP sublayers (bf16 only): x += gate * (a . w^T + bias),
 * then y = LayerNorm(x) * (1 + scale) + shift.  a [m, k] bf16 (row stride lda), w [n, k] bf16,
 * bias / gate / shift / scale fp32 [n], x fp32 [m, n] (contiguous, updated in place), y bf16
 * [m, n] (contiguous, must not overlap x).  When the workspace lets the product split k, the
 * pass that sums the slices also computes y (one launch fewer, x read once); otherwise the
 * LayerNorm runs as its own kernel.  Either way x and y hold the same bits as pf_gemm
 * (PF_EPI_GATED_RESIDUAL, same workspace) followed by pf_ln_modulate.  Requirements as for
 * both calls (n % 64 == 0, k % 64 == 0, n <= 6144).  Errors: INVALID_ARG, UNSUPPORTED, HIP.  Source: as pf_gemm and pf_ln_modulate. */
pf_status pf_gemm_residual_ln(const void* a, int64_t lda, const void* w, const float* bias, int64_t m,
                              int64_t n, int64_t k, float* x, const float* gate, const float* shift,
                              const float* scale, float eps, void* y, void* workspace,
                              uint64_t workspace_bytes, void* stream);

/* Workspace bytes pf_gemm can use for an [m, n, k] bf16 product (0: it never splits).
 * Source: as pf_gemm.
 * Errors: INVALID_ARG (bad sizes, NULL out), UNSUPPORTED (not gfx950). */
pf_status pf_gemm_workspace_size(int64_t m, int64_t n, int64_t k, uint64_t* bytes);

/* Full non-causal attention of `rows` query rows over the first seq_kv rows of kv:
 * for head j (columns [j*d, (j+1)*d)): O_j = softmax(Q_j K_j^T / sqrt(d)) V_j.
 * q [rows, heads*head_dim] (row stride ldq), o [rows, heads*head_dim] (row stride ldo),
 * both in kv->dtype.  bf16 requires kv->v_layout == PF_LAYOUT_K8, fp32 PF_LAYOUT_ROWS.
 * `workspace` (device, may be NULL) lets a query grid too small to fill the GPU split the
 * key range across workgroups; pf_attention_workspace_size gives the bytes that allow every
 * split the kernel may choose.  A smaller (or NULL) workspace limits the split; the result
 * is the same function of the inputs either way, up to fp32 summation order.  The caller
 * owns the workspace and must not use it concurrently with this call.  Source: "Key
 * contributions" of the PipeFusion summaries (the DiT keeps full attention: every query row
 * attends over every buffer row, fresh or stale).  Errors: INVALID_ARG (pointers, strides,
 * ranges, layouts), UNSUPPORTED (head_dim not 64 / 72 / 128, V not K8 for bf16), HIP. */
pf_status pf_attention(const void* q, int64_t ldq, const pf_kv_view* kv, int64_t seq_kv,
                       int64_t rows, int32_t heads, int32_t head_dim, void* o, int64_t ldo,
                       void* workspace, uint64_t workspace_bytes, void* stream);

/* pf_attention without a workspace argument and without any allocation, for callers that
 * cannot allocate (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments and result as pf_attention given a workspace of
 * pf_attention_workspace_size bytes (the same key-range split, the same bits); the split
 * partials go to the library's static device scratch of 128 MiB (134217728 bytes), which each
 * GPU the library runs on holds until the process ends.  A launch whose split needs more than
 * that (for example 6144 query rows x 3072 columns over 32768 keys, split 4 ways) returns
 * PF_ERR_UNSUPPORTED and enqueues nothing.  Every call on one GPU shares the scratch: calls that overlap in time on
 * one GPU (different streams without ordering) race.  Errors: as pf_attention. */
pf_status pf_attention_noalloc(const void* q, int64_t ldq, const pf_kv_view* kv, int64_t seq_kv, int64_t rows,
                               int32_t heads, int32_t head_dim, void* o, int64_t ldo, void* stream);

/* Workspace bytes pf_attention can use for `rows` queries of `heads` x `head_dim`.  Source:
 * as pf_attention.  Errors:
 * INVALID_ARG (bad sizes, NULL out). */
pf_status pf_attention_workspace_size(int64_t rows, int32_t heads, int32_t head_dim, uint64_t* bytes);

/* mod = SiLU(cond) . w_ada^T + b_ada: cond fp32 [hidden], w_ada [6*hidden, hidden] in
 * `dtype`, b_ada fp32 [6*hidden], mod fp32 [6*hidden].  Source: as stage_set_cond (a reading
 * of the DiT block).  Errors: INVALID_ARG, UNSUPPORTED (hidden above 16384), HIP. */
pf_status pf_adaln(const float* cond, const void* w_ada, const float* b_ada, int32_t hidden,
                   float* mod, int32_t dtype, void* stream);

/* The MM-DiT options' step between the QKV projection and attention (bf16, in place): for
 * every query row i < rows (q + i * ldq) and the K row of buffer row row_offset + i of kv, in
 * every head (columns [j*d, (j+1)*d)): with PF_STAGE_QK_NORM, x / sqrt(mean(x^2) + 1e-6) times
 * q_gamma (Q) or k_gamma (K), fp32 [head_dim]; then with PF_STAGE_ROPE, the pair (2k, 2k+1)
 * turned by angles[row_offset + i][k] (fp32 [kv->rows, head_dim / 2], radians).  fp32
 * arithmetic, one bf16 rounding per value.  `flags` holds only those two bits (0: nothing
 * happens).  V and every other buffer row stay as they are.  q must not overlap the buffer.
 * Requirements: kv->dtype bf16, row_elems == heads * head_dim <= 6144, ldq and k_ld multiples
 * of 8; q, K, the gammas and the angles 16-byte aligned.  Source: as
 * stage_load_text_weights (QK-RMSNorm and RoPE of the MM-DiT models, a reading).  Errors:
 * INVALID_ARG, UNSUPPORTED, HIP. */
pf_status pf_qk_norm_rope(void* q, int64_t ldq, const pf_kv_view* kv, int64_t row_offset, int64_t rows,
                          int32_t heads, int32_t head_dim, const float* q_gamma, const float* k_gamma,
                          const float* angles, uint32_t flags, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PF_H */
