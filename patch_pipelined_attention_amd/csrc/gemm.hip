// Projections of the DiT block: y = a . w^T + bias with fused epilogues.
//
// bf16 path: MFMA v_mfma_f32_32x32x16_bf16, fp32 accumulation.  The kernel computes
// output tiles transposed (features x tokens): the MFMA "A" operand is a block of 32
// weight rows and the "B" operand a block of 32 activation rows, both read as 8
// consecutive k-values (16 bytes) per lane from LDS.  The 32x32 accumulator then holds,
// per lane, one token and 4 consecutive output features per 8-row group, so every
// epilogue stores 4 contiguous values per access (8 B bf16 / 16 B fp32).
//
// Tile: 128 tokens x 128 features x 64 k per iteration, 256 threads = 4 wavefronts in a
// 2x2 grid, each owning 64 features x 64 tokens = 2x2 MFMA blocks.  Global tiles are
// prefetched into registers while the current LDS tile is consumed.  LDS rows are padded
// to 72 elements (144 B = 9 x 16 B) so the 16-byte fragment reads of 16 consecutive rows
// fall in distinct bank groups.
//
// fp32 path (tiny fp32 stages only): a plain 64x64 LDS-tiled FMA kernel.
#include "pf_internal.h"

namespace pf {

__device__ __forceinline__ float gelu_tanh_f(float x) {
  // 0.5 x (1 + tanh(u)) = x * sigmoid(2u), u = sqrt(2/pi) (x + 0.044715 x^3)
  const float u = 0.7978845608028654f * (x + 0.044715f * x * x * x);
  return x / (1.0f + expf(-2.0f * u));
}

__device__ __forceinline__ float gelu_erf_f(float x) { return 0.5f * x * (1.0f + erff(x * 0.7071067811865476f)); }

template <int EPI>
__device__ __forceinline__ float epi_act(float v) {
  if constexpr (EPI == kEpiGeluTanh) return gelu_tanh_f(v);
  else if constexpr (EPI == kEpiGeluErf) return gelu_erf_f(v);
  else return v;
}

namespace {
constexpr int kBT = 128;   // tokens per tile
constexpr int kBF = 128;   // features per tile
constexpr int kBK = 64;    // k per iteration
constexpr int kLdsLd = kBK + 8;
}  // namespace

template <int EPI>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(const bf16* __restrict__ A, int64_t lda,
                                                           const bf16* __restrict__ W,
                                                           const float* __restrict__ bias, int64_t M,
                                                           int64_t N, int64_t K, void* __restrict__ C,
                                                           int64_t ldc, const float* __restrict__ gate,
                                                           int tiles_n) {
  __shared__ __attribute__((aligned(16))) bf16 sW[kBF * kLdsLd];
  __shared__ __attribute__((aligned(16))) bf16 sX[kBT * kLdsLd];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int wf = wave & 1, wt = wave >> 1;

  const int tile_n = blockIdx.x % tiles_n;
  const int64_t tile_m = blockIdx.x / tiles_n;
  const int64_t n0 = (int64_t)tile_n * kBF;
  const int64_t m0 = tile_m * kBT;

  // global -> register staging: 4 chunks of 16 B of W and of X per thread per k tile
  uint4 rw[4], rx[4];
  auto load_tile = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 3, kc = c & 7;
      const int64_t n = n0 + row, m = m0 + row;
      rw[i] = n < N ? *reinterpret_cast<const uint4*>(W + n * K + k0 + kc * 8) : make_uint4(0, 0, 0, 0);
      rx[i] = m < M ? *reinterpret_cast<const uint4*>(A + m * lda + k0 + kc * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 3, kc = c & 7;
      *reinterpret_cast<uint4*>(&sW[row * kLdsLd + kc * 8]) = rw[i];
      *reinterpret_cast<uint4*>(&sX[row * kLdsLd + kc * 8]) = rx[i];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][t][e] = 0.f;

  const int64_t nk = K / kBK;
  load_tile(0);
  store_tile();
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load_tile((kt + 1) * kBK);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&sW[(wf * 64 + i * 32 + l32) * kLdsLd + kk * 16 + hi * 8]);
#pragma unroll
      for (int t = 0; t < 2; ++t)
        b[t] = *reinterpret_cast<const bf16x8*>(&sX[(wt * 64 + t * 32 + l32) * kLdsLd + kk * 16 + hi * 8]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[t], acc[i][t], 0, 0, 0);
    }
    __syncthreads();
    if (kt + 1 < nk) {
      store_tile();
      __syncthreads();
    }
  }

  // Epilogue.  acc[i][t][4g+j] = y[token = m0 + wt*64 + t*32 + l32][feature = n0 + wf*64 + i*32 + 8g + 4hi + j]
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int64_t m = m0 + wt * 64 + t * 32 + l32;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t f = n0 + wf * 64 + i * 32 + 8 * g + 4 * hi;
        if (f >= N) continue;
        const float4 bv = *reinterpret_cast<const float4*>(bias + f);
        float v0 = acc[i][t][4 * g + 0] + bv.x;
        float v1 = acc[i][t][4 * g + 1] + bv.y;
        float v2 = acc[i][t][4 * g + 2] + bv.z;
        float v3 = acc[i][t][4 * g + 3] + bv.w;
        if constexpr (EPI == kEpiGatedResidual) {
          float* cp = static_cast<float*>(C) + m * ldc + f;
          const float4 gv = *reinterpret_cast<const float4*>(gate + f);
          float4 cv = *reinterpret_cast<float4*>(cp);
          cv.x += gv.x * v0;
          cv.y += gv.y * v1;
          cv.z += gv.z * v2;
          cv.w += gv.w * v3;
          *reinterpret_cast<float4*>(cp) = cv;
        } else {
          bf16x4 o = {(bf16)epi_act<EPI>(v0), (bf16)epi_act<EPI>(v1), (bf16)epi_act<EPI>(v2),
                      (bf16)epi_act<EPI>(v3)};
          *reinterpret_cast<bf16x4*>(static_cast<bf16*>(C) + m * ldc + f) = o;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// fp32 path: 64 tokens x 64 features per block, 256 threads with 4x4 outputs each,
// k staged 16 at a time in LDS (k-major so the inner loop reads broadcast rows).
// ---------------------------------------------------------------------------------
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int64_t lda,
                                                       const float* __restrict__ W,
                                                       const float* __restrict__ bias, int64_t M,
                                                       int64_t N, int64_t K, float* __restrict__ C,
                                                       int64_t ldc, const float* __restrict__ gate,
                                                       int tiles_n) {
  __shared__ float sA[16][64 + 4];
  __shared__ float sW[16][64 + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t n0 = (int64_t)(blockIdx.x % tiles_n) * 64;
  const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * 64;
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < K; k0 += 16) {
    for (int c = tid; c < 64 * 16; c += 256) {
      const int r = c >> 4, kk = c & 15;
      const int64_t m = m0 + r, n = n0 + r, k = k0 + kk;
      sA[kk][r] = (m < M && k < K) ? A[m * lda + k] : 0.f;
      sW[kk][r] = (n < N && k < K) ? W[n * K + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = sA[kk][ty * 4 + i];
        w[i] = sW[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], w[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + tx * 4 + j;
      if (n >= N) continue;
      const float v = acc[i][j] + bias[n];
      if constexpr (EPI == kEpiGatedResidual) C[m * ldc + n] += gate[n] * v;
      else C[m * ldc + n] = epi_act<EPI>(v);
    }
  }
}

template <int EPI>
static void launch_gemm_epi(const void* a, int64_t lda, const void* w, const float* bias, int64_t m,
                            int64_t n, int64_t k, void* c, int64_t ldc, const float* gate, int dtype,
                            hipStream_t s) {
  if (dtype == kDtypeBF16) {
    const int tiles_n = (int)((n + kBF - 1) / kBF);
    const int64_t tiles = (int64_t)tiles_n * ((m + kBT - 1) / kBT);
    hipLaunchKernelGGL(gemm_bf16_kernel<EPI>, dim3((unsigned)tiles), dim3(256), 0, s,
                       static_cast<const bf16*>(a), lda, static_cast<const bf16*>(w), bias, m, n, k, c, ldc,
                       gate, tiles_n);
  } else {
    const int tiles_n = (int)((n + 63) / 64);
    const int64_t tiles = (int64_t)tiles_n * ((m + 63) / 64);
    hipLaunchKernelGGL(gemm_f32_kernel<EPI>, dim3((unsigned)tiles), dim3(256), 0, s,
                       static_cast<const float*>(a), lda, static_cast<const float*>(w), bias, m, n, k,
                       static_cast<float*>(c), ldc, gate, tiles_n);
  }
}

hipError_t launch_gemm(const void* a, int64_t lda, const void* w, const float* bias, int64_t m, int64_t n,
                       int64_t k, int epi, void* c, int64_t ldc, const float* gate, int dtype, hipStream_t s) {
  if (m <= 0) return hipSuccess;
  switch (epi) {
    case kEpiStore: launch_gemm_epi<kEpiStore>(a, lda, w, bias, m, n, k, c, ldc, gate, dtype, s); break;
    case kEpiGeluTanh: launch_gemm_epi<kEpiGeluTanh>(a, lda, w, bias, m, n, k, c, ldc, gate, dtype, s); break;
    case kEpiGeluErf: launch_gemm_epi<kEpiGeluErf>(a, lda, w, bias, m, n, k, c, ldc, gate, dtype, s); break;
    default: launch_gemm_epi<kEpiGatedResidual>(a, lda, w, bias, m, n, k, c, ldc, gate, dtype, s); break;
  }
  return hipGetLastError();
}

}  // namespace pf
