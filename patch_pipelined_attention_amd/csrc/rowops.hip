// Row kernels of the DiT block: LayerNorm + adaLN modulation, and the adaLN GEMV.
// Both are HBM-bound: one pass over the input rows / weight rows, 16-byte accesses,
// fp32 statistics and accumulation.
#include "pf_internal.h"

namespace pf {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ---------------------------------------------------------------------------------
// y = LayerNorm(x) * (1 + scale) + shift, one wavefront per row.  The row is held in
// registers (NS float4 per lane), so x is read once; all NS loads of a lane (and, for
// hidden <= 3072, those of shift and scale) are issued before the first use: indices past
// the row are clamped to its last chunk and masked out of the sums.  mean and variance are the two-pass fp32
// statistics of the row (biased variance), no affine.
// ---------------------------------------------------------------------------------
template <typename OutT, int NS>
__global__ __launch_bounds__(256) void ln_modulate_kernel(const float* __restrict__ x, int64_t rows,
                                                          int hidden, const float* __restrict__ shift,
                                                          const float* __restrict__ scale, float eps,
                                                          OutT* __restrict__ y, RowGroups grp) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int n4 = hidden >> 2;
  // sample g's rows of x and its shift / scale (row is wavefront-uniform)
  const int64_t g = row / grp.rows;
  const float4* xr = reinterpret_cast<const float4*>(x + g * grp.x_stride + (row - g * grp.rows) * hidden);
  const float4* sh4 = reinterpret_cast<const float4*>(shift + g * grp.p_stride);
  const float4* sc4 = reinterpret_cast<const float4*>(scale + g * grp.p_stride);
  // shift and scale are loaded up front too while they fit in registers (hidden <= 3072)
  constexpr bool kPreload = NS <= 12;
  float4 v[NS], sh[NS], sc[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int idx = lane + i * 64 < n4 ? lane + i * 64 : n4 - 1;
    v[i] = xr[idx];
  }
  if constexpr (kPreload) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int idx = lane + i * 64 < n4 ? lane + i * 64 : n4 - 1;
      sh[i] = sh4[idx];
      sc[i] = sc4[idx];
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < NS; ++i)
    if (lane + i * 64 < n4) sum += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  const float inv_h = 1.0f / (float)hidden;
  const float mean = wave_sum(sum) * inv_h;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    if (lane + i * 64 < n4) {
      const float a = v[i].x - mean, b = v[i].y - mean, c = v[i].z - mean, d = v[i].w - mean;
      sq += (a * a + b * b) + (c * c + d * d);
    }
  }
  const float var = wave_sum(sq) * inv_h;
  const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int idx = lane + i * 64;
    if (idx < n4) {
      if constexpr (!kPreload) {
        sh[i] = sh4[idx];
        sc[i] = sc4[idx];
      }
      const float o0 = (v[i].x - mean) * rstd * (1.0f + sc[i].x) + sh[i].x;
      const float o1 = (v[i].y - mean) * rstd * (1.0f + sc[i].y) + sh[i].y;
      const float o2 = (v[i].z - mean) * rstd * (1.0f + sc[i].z) + sh[i].z;
      const float o3 = (v[i].w - mean) * rstd * (1.0f + sc[i].w) + sh[i].w;
      if constexpr (sizeof(OutT) == 2) {
        bf16x4 o = {(bf16)o0, (bf16)o1, (bf16)o2, (bf16)o3};
        *reinterpret_cast<bf16x4*>(y + row * hidden + idx * 4) = o;
      } else {
        *reinterpret_cast<float4*>(y + row * hidden + idx * 4) = make_float4(o0, o1, o2, o3);
      }
    }
  }
}

template <typename OutT, int NS>
static void launch_ln_ns(int ns, dim3 grid, const float* x, int64_t rows, int hidden, const float* shift,
                         const float* scale, float eps, OutT* y, const RowGroups& g, hipStream_t s) {
  if constexpr (NS > 1) {
    if (ns < NS) return launch_ln_ns<OutT, NS - 1>(ns, grid, x, rows, hidden, shift, scale, eps, y, g, s);
  }
  hipLaunchKernelGGL((ln_modulate_kernel<OutT, NS>), grid, dim3(256), 0, s, x, rows, hidden, shift, scale, eps, y,
                     g);
}

hipError_t launch_ln_modulate(const float* x, int64_t rows, int hidden, const float* shift,
                              const float* scale, float eps, void* y, int dtype, hipStream_t s,
                              const RowGroups* groups) {
  if (rows <= 0) return hipSuccess;
  constexpr int kSlots = kMaxHidden / 256;
  const int ns = (hidden / 4 + 63) / 64;             // float4 chunks per lane
  if (ns < 1 || ns > kSlots) return hipErrorInvalidValue;
  const RowGroups g = groups ? *groups : RowGroups{rows, 0, 0};
  if (g.rows <= 0) return hipErrorInvalidValue;
  dim3 grid((unsigned)((rows + 3) / 4));
  if (dtype == kDtypeBF16)
    launch_ln_ns<bf16, kSlots>(ns, grid, x, rows, hidden, shift, scale, eps, static_cast<bf16*>(y), g, s);
  else
    launch_ln_ns<float, kSlots>(ns, grid, x, rows, hidden, shift, scale, eps, static_cast<float*>(y), g, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Reduce of a k-split gated-residual projection fused with the next LayerNorm + modulation,
// one wavefront per row.  Per 4 columns: the slices summed in order, + bias, x += gate * y (the
// reduce kernel's arithmetic); the updated row stays in registers for the LayerNorm (the LN
// kernel's arithmetic and reduction order), so both results match the unfused pair bit for bit
// while x is read once and one launch disappears.
// ---------------------------------------------------------------------------------
template <int NS>
__global__ __launch_bounds__(256) void reduce_residual_ln_kernel(const float* __restrict__ part, int n_split,
                                                                 int64_t rows, int hidden,
                                                                 const float* __restrict__ bias,
                                                                 float* __restrict__ x, int64_t ldx,
                                                                 const float* __restrict__ gate, RowGroups grp,
                                                                 const float* __restrict__ shift,
                                                                 const float* __restrict__ scale, float eps,
                                                                 bf16* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int n4 = hidden >> 2;
  const int64_t g = row / grp.rows;
  float* xr = x + g * grp.x_stride + (row - g * grp.rows) * ldx;
  const float* gr = gate + g * grp.p_stride;
  // chunks in batches of kBatch, every slice unrolled to kMaxGemmSplit (indices past n_split
  // and past the row clamped, their terms skipped), so a batch's loads are all in flight
  constexpr int kBatch = 4;
  float4 v[NS];
#pragma unroll
  for (int i0 = 0; i0 < NS; i0 += kBatch) {
    float4 pv[kBatch][kMaxGemmSplit], bv[kBatch], gv[kBatch], xv[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (i0 + j >= NS) break;
      const int idx = lane + (i0 + j) * 64 < n4 ? lane + (i0 + j) * 64 : n4 - 1;
      const int64_t f = (int64_t)idx * 4;
#pragma unroll
      for (int s2 = 0; s2 < kMaxGemmSplit; ++s2) {
        const int64_t sc = s2 < n_split ? s2 : n_split - 1;
        pv[j][s2] = *reinterpret_cast<const float4*>(part + (sc * rows + row) * hidden + f);
      }
      bv[j] = *reinterpret_cast<const float4*>(bias + f);
      gv[j] = *reinterpret_cast<const float4*>(gr + f);
      xv[j] = *reinterpret_cast<const float4*>(xr + f);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = i0 + j;
      if (i >= NS) break;
      float4 acc = pv[j][0];
#pragma unroll
      for (int s2 = 1; s2 < kMaxGemmSplit; ++s2) {
        if (s2 < n_split) {
          acc.x += pv[j][s2].x;
          acc.y += pv[j][s2].y;
          acc.z += pv[j][s2].z;
          acc.w += pv[j][s2].w;
        }
      }
      acc.x += bv[j].x;
      acc.y += bv[j].y;
      acc.z += bv[j].z;
      acc.w += bv[j].w;
      float4 cv = xv[j];
      cv.x += gv[j].x * acc.x;
      cv.y += gv[j].y * acc.y;
      cv.z += gv[j].z * acc.z;
      cv.w += gv[j].w * acc.w;
      v[i] = cv;
      if (lane + i * 64 < n4) *reinterpret_cast<float4*>(xr + (int64_t)(lane + i * 64) * 4) = cv;
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < NS; ++i)
    if (lane + i * 64 < n4) sum += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  const float inv_h = 1.0f / (float)hidden;
  const float mean = wave_sum(sum) * inv_h;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    if (lane + i * 64 < n4) {
      const float a = v[i].x - mean, b = v[i].y - mean, c = v[i].z - mean, d = v[i].w - mean;
      sq += (a * a + b * b) + (c * c + d * d);
    }
  }
  const float var = wave_sum(sq) * inv_h;
  const float rstd = 1.0f / sqrtf(var + eps);
  const float4* sh4 = reinterpret_cast<const float4*>(shift + g * grp.p_stride);
  const float4* sc4 = reinterpret_cast<const float4*>(scale + g * grp.p_stride);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int idx = lane + i * 64;
    if (idx < n4) {
      const float4 sh = sh4[idx], sc = sc4[idx];
      const float o0 = (v[i].x - mean) * rstd * (1.0f + sc.x) + sh.x;
      const float o1 = (v[i].y - mean) * rstd * (1.0f + sc.y) + sh.y;
      const float o2 = (v[i].z - mean) * rstd * (1.0f + sc.z) + sh.z;
      const float o3 = (v[i].w - mean) * rstd * (1.0f + sc.w) + sh.w;
      bf16x4 o = {(bf16)o0, (bf16)o1, (bf16)o2, (bf16)o3};
      *reinterpret_cast<bf16x4*>(y + row * hidden + idx * 4) = o;
    }
  }
}

template <int NS>
static void launch_rrl_ns(int ns, dim3 grid, const float* part, int n_split, int64_t rows, int hidden,
                          const float* bias, float* x, int64_t ldx, const float* gate, const RowGroups& g,
                          const LnAfter& ln, hipStream_t s) {
  if constexpr (NS > 1) {
    if (ns < NS) return launch_rrl_ns<NS - 1>(ns, grid, part, n_split, rows, hidden, bias, x, ldx, gate, g, ln, s);
  }
  hipLaunchKernelGGL((reduce_residual_ln_kernel<NS>), grid, dim3(256), 0, s, part, n_split, rows, hidden, bias, x, ldx,
                     gate, g, ln.shift, ln.scale, ln.eps, static_cast<bf16*>(ln.y));
}

hipError_t launch_reduce_residual_ln(const float* part, int n_split, int64_t m, int n, const float* bias, float* x,
                                     int64_t ldx, const float* gate, const RowGroups& rg, const LnAfter& ln,
                                     hipStream_t s) {
  if (m <= 0) return hipSuccess;
  constexpr int kSlots = kMaxHidden / 256;
  const int ns = (n / 4 + 63) / 64;
  if (ns < 1 || ns > kSlots || n % 4 != 0 || rg.rows <= 0) return hipErrorInvalidValue;
  launch_rrl_ns<kSlots>(ns, dim3((unsigned)((m + 3) / 4)), part, n_split, m, n, bias, x, ldx, gate, rg, ln, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Q and K of one part of a micro-step, in place (bf16): per (row, head), an optional RMSNorm
// (eps 1e-6) times gamma [D], then an optional rotary embedding of the pairs (2k, 2k+1) by
// angles[buffer row][k].  Rows r < nb * n: sample g = r / n, local row i = r - g n, buffer
// row off + i; Q row r is at q + r * ldq, its K row at k + g * kv_stride + (off + i) * ldk
// (the buffer, ROWS layout).
//
// One workgroup per row.  Thread t owns the 16-byte chunks c = t, t + 256, ... (8 values; D is
// a multiple of 8, so a chunk never straddles two heads) of both the Q row and the K row, and
// issues all its loads before any arithmetic: the kernel is bound by HBM, and a row's Q and K
// (up to 24 KB) are in flight at once.  The per-head sums of squares go through LDS as one
// partial per chunk, summed by each reader in chunk order (deterministic).
// ---------------------------------------------------------------------------------
constexpr int kQkChunks = kMaxHidden / 8 / 256;   // chunks per thread and matrix

__device__ __forceinline__ float sumsq8(const bf16x8& v) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float f = (float)v[e];
    s = fmaf(f, f, s);
  }
  return s;
}

template <int D>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(bf16* __restrict__ q, int64_t ldq, bf16* __restrict__ k,
                                                           int64_t ldk, int64_t kv_stride, int64_t off, int64_t n,
                                                           int hidden, const float* __restrict__ gq,
                                                           const float* __restrict__ gk,
                                                           const float* __restrict__ angles, int do_norm,
                                                           int do_rope) {
  constexpr int kCph = D / 8;   // chunks per head
  __shared__ float part[2][kMaxHidden / 8];
  const int64_t r = blockIdx.x;
  const int64_t g = r / n, i = r - g * n;
  bf16* qr = q + r * ldq;
  bf16* kr = k + g * kv_stride + (off + i) * ldk;
  const float* ar = angles + (off + i) * (D / 2);
  const int nch = hidden / 8;
  bf16x8 vq[kQkChunks], vk[kQkChunks];
  float4 an[kQkChunks];
#pragma unroll
  for (int j = 0; j < kQkChunks; ++j) {
    const int c = threadIdx.x + j * 256;
    if (c < nch) {
      vq[j] = *reinterpret_cast<const bf16x8*>(qr + 8 * c);
      vk[j] = *reinterpret_cast<const bf16x8*>(kr + 8 * c);
      if (do_rope) an[j] = *reinterpret_cast<const float4*>(ar + (8 * c) % D / 2);
    }
  }
  float rq[kQkChunks], rk[kQkChunks];
  if (do_norm) {
#pragma unroll
    for (int j = 0; j < kQkChunks; ++j) {
      const int c = threadIdx.x + j * 256;
      if (c < nch) {
        part[0][c] = sumsq8(vq[j]);
        part[1][c] = sumsq8(vk[j]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kQkChunks; ++j) {
      const int c = threadIdx.x + j * 256;
      const int h0 = c < nch ? c / kCph * kCph : 0;
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int m = 0; m < kCph; ++m) {
        sq += part[0][h0 + m];
        sk += part[1][h0 + m];
      }
      rq[j] = 1.0f / sqrtf(sq / (float)D + 1e-6f);
      rk[j] = 1.0f / sqrtf(sk / (float)D + 1e-6f);
    }
  }
#pragma unroll
  for (int j = 0; j < kQkChunks; ++j) {
    const int c = threadIdx.x + j * 256;
    if (c >= nch) continue;
    float fq[8], fk[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      fq[e] = (float)vq[j][e];
      fk[e] = (float)vk[j][e];
    }
    if (do_norm) {
      const float4* g4q = reinterpret_cast<const float4*>(gq + (8 * c) % D);
      const float4* g4k = reinterpret_cast<const float4*>(gk + (8 * c) % D);
      const float4 q0 = g4q[0], q1 = g4q[1], k0 = g4k[0], k1 = g4k[1];
      const float wq[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
      const float wk[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        fq[e] = fq[e] * rq[j] * wq[e];
        fk[e] = fk[e] * rk[j] * wk[e];
      }
    }
    if (do_rope) {
      const float a[4] = {an[j].x, an[j].y, an[j].z, an[j].w};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        float sn, cs;
        sincosf(a[p], &sn, &cs);
        const float q0 = fq[2 * p], q1 = fq[2 * p + 1], k0 = fk[2 * p], k1 = fk[2 * p + 1];
        fq[2 * p] = q0 * cs - q1 * sn;
        fq[2 * p + 1] = q0 * sn + q1 * cs;
        fk[2 * p] = k0 * cs - k1 * sn;
        fk[2 * p + 1] = k0 * sn + k1 * cs;
      }
    }
    bf16x8 oq, ok;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      oq[e] = (bf16)fq[e];
      ok[e] = (bf16)fk[e];
    }
    *reinterpret_cast<bf16x8*>(qr + 8 * c) = oq;
    *reinterpret_cast<bf16x8*>(kr + 8 * c) = ok;
  }
}

hipError_t launch_qk_norm_rope(void* q, int64_t ldq, void* k, int64_t ldk, int64_t kv_stride, int64_t off, int64_t n,
                               int64_t nb, int heads, int head_dim, const float* gq, const float* gk,
                               const float* angles, bool norm, bool rope, hipStream_t s) {
  const int64_t rows = nb * n;
  if (rows <= 0 || (!norm && !rope)) return hipSuccess;
  const int hidden = heads * head_dim;
  if (hidden > kMaxHidden || hidden % 8 != 0 || rows > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)rows);
  bf16* qp = static_cast<bf16*>(q);
  bf16* kp = static_cast<bf16*>(k);
#define PF_QK_LAUNCH(D)                                                                                        \
  hipLaunchKernelGGL(qk_norm_rope_kernel<D>, grid, dim3(256), 0, s, qp, ldq, kp, ldk, kv_stride, off, n, hidden, \
                     gq, gk, angles, norm ? 1 : 0, rope ? 1 : 0)
  switch (head_dim) {
    case 64: PF_QK_LAUNCH(64); break;
    case 72: PF_QK_LAUNCH(72); break;
    case 128: PF_QK_LAUNCH(128); break;
    default: return hipErrorInvalidValue;
  }
#undef PF_QK_LAUNCH
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// mod[j] = sum_i SiLU(c[i]) * W[j, i] + b[j] for j < chunks * h (6 or 3 vectors of h), for a
// batch of weight sets (blockIdx.y: set m at w + m * w_stride, b + m * b_stride, output at
// mod + m * mod_stride) and conditions (blockIdx.z: sample g's cond at + g * cond_stride, its
// output at + g * mod_sample_stride), so one launch covers every layer, stream and sample.
// SiLU(c) is staged in LDS once per block; one wavefront per output row streams that row of W
// with 16-byte loads, four in flight per lane.
// ---------------------------------------------------------------------------------
template <typename WT>
__global__ __launch_bounds__(256) void adaln_kernel(const float* __restrict__ cond, int64_t cond_stride,
                                                    const WT* __restrict__ w, int64_t w_stride,
                                                    const float* __restrict__ b, int64_t b_stride, int hidden,
                                                    int n_out, float* __restrict__ mod, int64_t mod_stride,
                                                    int64_t mod_sample_stride) {
  extern __shared__ float s_act[];
  const int m = blockIdx.y, g = blockIdx.z;
  const float* cg = cond + g * cond_stride;
  for (int i = threadIdx.x; i < hidden; i += 256) {
    const float c = cg[i];
    s_act[i] = c / (1.0f + expf(-c));
  }
  __syncthreads();
  const WT* wm = w + m * w_stride;
  const float* bm = b + m * b_stride;
  float* om = mod + m * mod_stride + g * mod_sample_stride;
  const int lane = threadIdx.x & 63;
  for (int row = blockIdx.x * 4 + (threadIdx.x >> 6); row < n_out; row += gridDim.x * 4) {
    const WT* wr = wm + (int64_t)row * hidden;
    float acc = 0.f;
#pragma unroll 4
    for (int k = lane * 8; k < hidden; k += 512) {
      if constexpr (sizeof(WT) == 2) {
        const bf16x8 wv = *reinterpret_cast<const bf16x8*>(wr + k);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += (float)wv[e] * s_act[k + e];
      } else {
        const float4 w0 = *reinterpret_cast<const float4*>(wr + k);
        const float4 w1 = *reinterpret_cast<const float4*>(wr + k + 4);
        acc += w0.x * s_act[k] + w0.y * s_act[k + 1] + w0.z * s_act[k + 2] + w0.w * s_act[k + 3];
        acc += w1.x * s_act[k + 4] + w1.y * s_act[k + 5] + w1.z * s_act[k + 6] + w1.w * s_act[k + 7];
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) om[row] = acc + bm[row];
  }
}

hipError_t launch_adaln_batch(const float* cond, int64_t cond_stride, int n_samples, const void* w,
                              int64_t w_stride, const float* b, int64_t b_stride, int n_sets, int hidden,
                              float* mod, int64_t mod_stride, int64_t mod_sample_stride, int dtype, hipStream_t s,
                              int chunks) {
  if (n_sets <= 0 || n_samples <= 0) return hipSuccess;
  const int n_out = chunks * hidden;
  int blocks = (n_out + 3) / 4;
  const int cap = 8192 / (n_sets * n_samples);
  if (blocks > cap) blocks = cap > 1 ? cap : 1;
  const dim3 grid((unsigned)blocks, (unsigned)n_sets, (unsigned)n_samples);
  const size_t lds = sizeof(float) * (size_t)hidden;
  if (dtype == kDtypeBF16)
    hipLaunchKernelGGL(adaln_kernel<bf16>, grid, dim3(256), lds, s, cond, cond_stride, static_cast<const bf16*>(w),
                       w_stride, b, b_stride, hidden, n_out, mod, mod_stride, mod_sample_stride);
  else
    hipLaunchKernelGGL(adaln_kernel<float>, grid, dim3(256), lds, s, cond, cond_stride,
                       static_cast<const float*>(w), w_stride, b, b_stride, hidden, n_out, mod, mod_stride,
                       mod_sample_stride);
  return hipGetLastError();
}

hipError_t launch_adaln(const float* cond, const void* w, const float* b, int hidden, float* mod,
                        int dtype, hipStream_t s, int chunks) {
  return launch_adaln_batch(cond, 0, 1, w, 0, b, 0, 1, hidden, mod, 0, 0, dtype, s, chunks);
}

}  // namespace pf
