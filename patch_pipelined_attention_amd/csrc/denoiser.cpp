// The denoising loop around one stage (C ABI declared in include/pf.h): per step, the
// timestep condition, the patch embedding of the latent, one stage step (a warm-up step
// runs every row fresh; later steps reuse the stale buffers, PipeFusion "Core mechanisms" 2),
// the final adaLN layer and the (guided) DDIM update of the latent.  Each step is a fixed
// sequence of launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <new>
#include <string>
#include <vector>

#include "pf.h"
#include "pf_internal.h"

using namespace pf;

namespace {

pf_status dfail(pf_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  pf_set_last_error(buf);
  return st;
}

pf_status dhip(hipError_t e, const char* what) {
  return dfail(PF_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

struct pf_denoiser {
  pf_stage* stage = nullptr;
  pf_stage_config scfg{};
  pf_denoiser_config cfg{};
  int64_t h = 0, batch = 1, s_kv = 0, s_img = 0, kdim = 0;   // kdim = C p p
  std::vector<double> abar;                                  // training-step schedule
  float* mem = nullptr;
  // weights (copies), then working buffers
  float *w_patch, *b_patch, *w_t1, *b_t1, *w_t2, *b_t2, *w_fada, *b_fada, *w_out, *b_out;
  float *pos, *t_hidden, *cond, *mod_f, *x, *hf, *v;
  bool loaded = false;
  bool broken = false;
};

static size_t up256(size_t n) { return (n + 63) / 64 * 64; }   // floats, 256-byte aligned

extern "C" pf_status denoiser_create(pf_stage* st, const pf_denoiser_config* cfg, pf_denoiser** out) {
  if (!out) return dfail(PF_ERR_INVALID_ARG, "denoiser_create: null out");
  *out = nullptr;
  if (!st || !cfg) return dfail(PF_ERR_INVALID_ARG, "denoiser_create: null argument");
  pf_stage_config sc;
  pf_status s = stage_get_config(st, &sc);
  if (s != PF_OK) return s;
  const int64_t h = sc.hidden, nb = sc.batch > 0 ? sc.batch : 1;
  if (cfg->in_channels < 1 || cfg->patch < 1 || cfg->grid_h < 1 || cfg->grid_w < 1)
    return dfail(PF_ERR_INVALID_ARG, "denoiser_create: bad latent geometry");
  if ((int64_t)cfg->grid_h * cfg->grid_w != sc.seq_img)
    return dfail(PF_ERR_INVALID_ARG, "denoiser_create: grid_h * grid_w != the stage's seq_img");
  if (cfg->freq_dim < 2 || cfg->freq_dim % 2 != 0 || cfg->freq_dim > 16384)
    return dfail(PF_ERR_INVALID_ARG, "denoiser_create: freq_dim must be even, in [2, 16384]");
  if (cfg->train_steps < 1 || !(cfg->beta_start > 0.f) || !(cfg->beta_end >= cfg->beta_start) || !(cfg->beta_end < 1.f))
    return dfail(PF_ERR_INVALID_ARG, "denoiser_create: bad noise schedule");
  if (h % 4 != 0 || h > 16384) return dfail(PF_ERR_UNSUPPORTED, "denoiser_create: hidden must be a multiple of 4");
  const int64_t kdim = (int64_t)cfg->in_channels * cfg->patch * cfg->patch;
  if (kdim > 4096) return dfail(PF_ERR_UNSUPPORTED, "denoiser_create: in_channels * patch^2 > 4096");

  pf_denoiser* d = new (std::nothrow) pf_denoiser();
  if (!d) return dfail(PF_ERR_OOM, "denoiser_create: host allocation failed");
  d->stage = st;
  d->scfg = sc;
  d->cfg = *cfg;
  d->h = h;
  d->batch = nb;
  d->s_kv = sc.seq_txt + sc.seq_img;
  d->s_img = sc.seq_img;
  d->kdim = kdim;
  // linear betas, abar_t = prod_{i <= t} (1 - beta_i)
  d->abar.resize(cfg->train_steps);
  double prod = 1.0;
  for (int i = 0; i < cfg->train_steps; ++i) {
    const double beta = cfg->train_steps == 1 ? cfg->beta_start
                                               : cfg->beta_start + (cfg->beta_end - cfg->beta_start) * i /
                                                                       (double)(cfg->train_steps - 1);
    prod *= 1.0 - beta;
    d->abar[i] = prod;
  }
  const size_t F = cfg->freq_dim;
  const size_t sizes[17] = {up256(h * kdim), up256(h), up256(h * F), up256(h), up256(h * h), up256(h),
                            up256(2 * h * h), up256(2 * h), up256(kdim * h), up256(kdim),
                            up256(d->s_img * h),            // pos
                            up256(h),                       // t_hidden
                            up256(nb * h),                  // cond
                            up256(nb * 2 * h),              // mod_f
                            up256(nb * d->s_kv * h),        // x
                            up256(nb * d->s_img * h),       // hf
                            up256(nb * d->s_img * kdim)};   // v
  size_t total = 0;
  for (size_t z : sizes) total += z;
  hipError_t e = hipMalloc((void**)&d->mem, total * sizeof(float));
  if (e != hipSuccess) {
    delete d;
    (void)hipGetLastError();
    return e == hipErrorOutOfMemory ? dfail(PF_ERR_OOM, "denoiser_create: device allocation failed")
                                    : dhip(e, "denoiser_create: hipMalloc");
  }
  float** ptrs[17] = {&d->w_patch, &d->b_patch, &d->w_t1, &d->b_t1, &d->w_t2, &d->b_t2, &d->w_fada, &d->b_fada,
                      &d->w_out, &d->b_out, &d->pos, &d->t_hidden, &d->cond, &d->mod_f, &d->x, &d->hf, &d->v};
  float* p = d->mem;
  for (int i = 0; i < 17; ++i) {
    *ptrs[i] = p;
    p += sizes[i];
  }
  // fixed 2-D sine-cosine position table (double on the host, stored fp32): for patch
  // s = (gy, gx), width quarters sin(gy w_k), cos(gy w_k), sin(gx w_k), cos(gx w_k),
  // w_k = 10000^(-k / (h/4))
  std::vector<float> pos((size_t)(d->s_img * h));
  const int64_t q = h / 4;
  std::vector<double> w(q);
  for (int64_t k = 0; k < q; ++k) w[k] = std::pow(10000.0, -(double)k / (double)q);
  for (int64_t s2 = 0; s2 < d->s_img; ++s2) {
    const double gy = (double)(s2 / cfg->grid_w), gx = (double)(s2 % cfg->grid_w);
    float* r = &pos[(size_t)(s2 * h)];
    for (int64_t k = 0; k < q; ++k) {
      r[k] = (float)std::sin(gy * w[k]);
      r[q + k] = (float)std::cos(gy * w[k]);
      r[2 * q + k] = (float)std::sin(gx * w[k]);
      r[3 * q + k] = (float)std::cos(gx * w[k]);
    }
  }
  if ((e = hipMemcpy(d->pos, pos.data(), pos.size() * sizeof(float), hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemset(d->x, 0, (size_t)(nb * d->s_kv * h) * sizeof(float))) != hipSuccess ||
      (e = hipDeviceSynchronize()) != hipSuccess) {
    (void)hipFree(d->mem);
    delete d;
    return dhip(e, "denoiser_create: initialising device memory");
  }
  *out = d;
  return PF_OK;
}

extern "C" pf_status denoiser_destroy(pf_denoiser* d) {
  if (!d) return PF_OK;
  if (d->mem) (void)hipFree(d->mem);
  delete d;
  return PF_OK;
}

extern "C" pf_status denoiser_load_weights(pf_denoiser* d, const pf_denoiser_weights* w, void* stream) {
  if (!d || !w) return dfail(PF_ERR_INVALID_ARG, "denoiser_load_weights: null argument");
  if (d->broken) return dfail(PF_ERR_HIP, "denoiser_load_weights: an earlier HIP call failed");
  const int64_t h = d->h, F = d->cfg.freq_dim, K = d->kdim;
  struct Cp { float* dst; const float* src; int64_t n; } cps[10] = {
      {d->w_patch, w->w_patch, h * K}, {d->b_patch, w->b_patch, h},   {d->w_t1, w->w_t1, h * F},
      {d->b_t1, w->b_t1, h},           {d->w_t2, w->w_t2, h * h},     {d->b_t2, w->b_t2, h},
      {d->w_fada, w->w_fada, 2 * h * h}, {d->b_fada, w->b_fada, 2 * h}, {d->w_out, w->w_out, K * h},
      {d->b_out, w->b_out, K}};
  for (const Cp& c : cps)
    if (!c.src) return dfail(PF_ERR_INVALID_ARG, "denoiser_load_weights: null weight pointer");
  for (const Cp& c : cps) {
    hipError_t e = hipMemcpyAsync(c.dst, c.src, (size_t)c.n * sizeof(float), hipMemcpyDeviceToDevice,
                                  (hipStream_t)stream);
    if (e != hipSuccess) {
      d->broken = true;
      return dhip(e, "denoiser_load_weights: hipMemcpyAsync");
    }
  }
  d->loaded = true;
  return PF_OK;
}

static pf_status step_impl(pf_denoiser* d, float* z, const float* y, const float* x_txt, int32_t t, int32_t t_next,
                           uint32_t flags, float guidance, hipStream_t s) {
  const int64_t h = d->h, nb = d->batch, stxt = d->scfg.seq_txt, simg = d->s_img, K = d->kdim;
  const pf_denoiser_config& c = d->cfg;
  hipError_t e;
  auto fail_hip = [&](const char* what) {
    d->broken = true;
    return dhip(e, what);
  };
  // condition: c_b = W_t2 . SiLU(W_t1 . freq(t) + b_t1) + b_t2 + y_b
  if ((e = launch_gemv_f32(nullptr, (double)t, false, d->w_t1, d->b_t1, c.freq_dim, (int)h, true, nullptr, 1,
                           d->t_hidden, s)) != hipSuccess)
    return fail_hip("denoiser: timestep MLP");
  if ((e = launch_gemv_f32(d->t_hidden, 0.0, false, d->w_t2, d->b_t2, (int)h, (int)h, false, y, (int)nb, d->cond,
                           s)) != hipSuccess)
    return fail_hip("denoiser: condition");
  // stage input rows: the text rows as given (or zeros), then the embedded patches
  if (stxt > 0) {
    const size_t bytes = (size_t)(stxt * h) * sizeof(float);
    e = x_txt ? hipMemcpy2DAsync(d->x, (size_t)(d->s_kv * h) * sizeof(float), x_txt, bytes, bytes, (size_t)nb,
                                 hipMemcpyDeviceToDevice, s)
              : hipMemset2DAsync(d->x, (size_t)(d->s_kv * h) * sizeof(float), 0, bytes, (size_t)nb, s);
    if (e != hipSuccess) return fail_hip("denoiser: text rows");
  }
  if ((e = launch_patch_embed(z, c.in_channels, c.patch, c.grid_w, simg, (int)h, d->w_patch, d->b_patch, d->pos, d->x,
                              d->s_kv * h, stxt, (int)nb, s)) != hipSuccess)
    return fail_hip("denoiser: patch embedding");
  pf_status st = stage_run_step(d->stage, d->x, d->x, d->cond, flags & PF_STEP_WARMUP, s);
  if (st != PF_OK) return st;
  // final layer: (shift, scale) = SiLU(c_b) . W_f^T + b_f; LN + modulation of the image rows
  // (fp32); projection to C p p values per patch
  for (int64_t b = 0; b < nb; ++b)
    if ((e = launch_gemv_f32(d->cond + b * h, 0.0, true, d->w_fada, d->b_fada, (int)h, (int)(2 * h), false, nullptr, 1,
                             d->mod_f + b * 2 * h, s)) != hipSuccess)
      return fail_hip("denoiser: final adaLN");
  const RowGroups rg{simg, d->s_kv * h, 2 * h};
  if ((e = launch_ln_modulate(d->x + stxt * h, nb * simg, (int)h, d->mod_f, d->mod_f + h, d->scfg.ln_eps, d->hf,
                              kDtypeFP32, s, &rg)) != hipSuccess)
    return fail_hip("denoiser: final LayerNorm");
  if ((e = launch_gemm(d->hf, h, d->w_out, d->b_out, nb * simg, K, h, kEpiStore, d->v, K, nullptr, kDtypeFP32, nullptr,
                       0, s)) != hipSuccess)
    return fail_hip("denoiser: final projection");
  const double ab_t = d->abar[t], ab_n = t_next >= 0 ? d->abar[t_next] : 1.0;
  const double a = std::sqrt(ab_n / ab_t), ecoef = std::sqrt(1.0 - ab_n) - a * std::sqrt(1.0 - ab_t);
  const bool guided = nb == 2;   // a batch of two is a guidance pair
  if ((e = launch_guided_ddim(z, d->v, c.in_channels, c.patch, c.grid_w, simg, (int)nb, guided, guidance, (float)a,
                              (float)ecoef, s)) != hipSuccess)
    return fail_hip("denoiser: DDIM update");
  return PF_OK;
}

static pf_status check_step_args(pf_denoiser* d, const float* z, const float* y, int32_t t, int32_t t_next,
                                 const char* who) {
  if (!d) return dfail(PF_ERR_INVALID_ARG, "%s: null denoiser", who);
  if (d->broken) return dfail(PF_ERR_HIP, "%s: an earlier HIP call failed", who);
  if (!d->loaded) return dfail(PF_ERR_STATE, "%s: weights not loaded", who);
  if (!z || !y) return dfail(PF_ERR_INVALID_ARG, "%s: null z or y", who);
  if (((uintptr_t)z & 15u) || ((uintptr_t)y & 3u)) return dfail(PF_ERR_INVALID_ARG, "%s: misaligned z or y", who);
  if (t < 0 || t >= d->cfg.train_steps || t_next >= t || t_next < -1)
    return dfail(PF_ERR_INVALID_ARG, "%s: need 0 <= t < train_steps and -1 <= t_next < t", who);
  return PF_OK;
}

extern "C" pf_status denoiser_step(pf_denoiser* d, float* z, const float* y, const float* x_txt, int32_t t,
                                   int32_t t_next, uint32_t flags, float guidance, void* stream) {
  pf_status s = check_step_args(d, z, y, t, t_next, "denoiser_step");
  if (s != PF_OK) return s;
  if (flags & ~PF_STEP_WARMUP) return dfail(PF_ERR_INVALID_ARG, "denoiser_step: unknown flags");
  return step_impl(d, z, y, x_txt, t, t_next, flags, guidance, (hipStream_t)stream);
}

extern "C" pf_status denoiser_run(pf_denoiser* d, float* z, const float* y, const float* x_txt,
                                  const int32_t* timesteps, int32_t n_steps, int32_t warmup_steps, float guidance,
                                  void* stream) {
  if (!timesteps || n_steps < 1) return dfail(PF_ERR_INVALID_ARG, "denoiser_run: need timesteps and n_steps >= 1");
  if (warmup_steps < 1 || warmup_steps > n_steps)
    return dfail(PF_ERR_INVALID_ARG, "denoiser_run: need 1 <= warmup_steps <= n_steps (the first step has no stale "
                                     "context)");
  for (int32_t i = 0; i < n_steps; ++i) {
    const int32_t tn = i + 1 < n_steps ? timesteps[i + 1] : -1;
    pf_status s = check_step_args(d, z, y, timesteps[i], tn, "denoiser_run");
    if (s != PF_OK) return s;
  }
  for (int32_t i = 0; i < n_steps; ++i) {
    const int32_t tn = i + 1 < n_steps ? timesteps[i + 1] : -1;
    pf_status s = step_impl(d, z, y, x_txt, timesteps[i], tn, i < warmup_steps ? PF_STEP_WARMUP : 0u, guidance,
                            (hipStream_t)stream);
    if (s != PF_OK) return s;
  }
  return PF_OK;
}
