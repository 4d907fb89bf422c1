// Projections of the DiT block: y = a . w^T + bias with fused epilogues.
//
// bf16 path: MFMA v_mfma_f32_32x32x16_bf16, fp32 accumulation.  The kernel computes
// output tiles transposed (features x tokens): the MFMA "A" operand is a block of 32
// weight rows and the "B" operand a block of 32 activation rows, both read as 8
// consecutive k-values (16 bytes) per lane from LDS.  The 32x32 accumulator then holds,
// per lane, one token and 4 consecutive output features per 8-row group, so every
// epilogue stores 4 contiguous values per access (8 B bf16 / 16 B fp32).
//
// Tiles: 128 x 128, or 192 features x 128 tokens, with a 2-stage ring, two workgroups per CU.
// The 192-feature tile (six MFMA blocks per wavefront instead of four, 80 KB of LDS) moves 17%
// fewer LDS and L2 bytes per FLOP and gives each k tile 1.5x the MFMA work to hide the next
// tile's load behind; it is taken for grids of whole tiles that still give every CU at least
// 1.5 of them (fewer leave CUs with a lone workgroup, which runs slower).  Grids too small to
// fill the GPU split k: every slice writes its fp32 partial tile and a reduce pass sums the
// slices in order (deterministic) and applies the epilogue.  A grid whose last round would run part
// full splits only the tiles of that round ("remainder split"): the full rounds run whole
// tiles, the remaining tiles run as k slices that fill one round, and a reduce pass over
// those tiles alone finishes them.  (A last-arriving-slice merge inside the
// GEMM measured slower on MI355X: the partials cross XCDs, whose L2s are not coherent, so
// they must be written through and read back from the device-coherent level, a longer
// latency chain than one more launch.)
//
// Workgroup ids map to tiles XCD by XCD (consecutive ids on one XCD), and within that in
// groups of kGroupRows tile rows walked column by column, so the workgroups an XCD runs at
// once share a few weight and activation row blocks in its L2.
//
// fp32 path (tiny fp32 stages only): a plain 64x64 LDS-tiled FMA kernel.
#include "pf_internal.h"

namespace pf {

__device__ __forceinline__ float gelu_tanh_f(float x) {
  // 0.5 x (1 + tanh(u)) = x * sigmoid(2u) = x / (1 + 2^(-2u log2 e)), u = sqrt(2/pi) (x + 0.044715 x^3).
  // Hardware exp2 and reciprocal (about 1 ulp each); for large |x| the power saturates to
  // 0 or inf and the result to x or 0.
  const float x2 = x * x;
  const float t = x * fmaf(x2, -2.0f * 1.4426950408889634f * 0.7978845608028654f * 0.044715f,
                           -2.0f * 1.4426950408889634f * 0.7978845608028654f);   // -2u log2 e
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
}

__device__ __forceinline__ float gelu_erf_f(float x) { return 0.5f * x * (1.0f + erff(x * 0.7071067811865476f)); }

template <int EPI>
__device__ __forceinline__ float epi_act(float v) {
  if constexpr (EPI == kEpiGeluTanh) return gelu_tanh_f(v);
  else if constexpr (EPI == kEpiGeluErf) return gelu_erf_f(v);
  else return v;
}

__device__ __forceinline__ int gemm_xcd_remap(int bid, int nb) {
  const int per = nb / 8, rem = nb % 8;
  const int x = bid % 8;
  return x * per + (x < rem ? x : rem) + bid / 8;
}

constexpr int kGroupRows = 4;

// Tile (row tm, column tn) of tile id `rest` in [0, tiles_m * tiles_n): groups of kGroupRows
// tile rows (fewer in the last group), each walked column by column.
__device__ __forceinline__ void gemm_tile_of(int rest, int tiles_m, int tiles_n, int64_t& tm, int& tn) {
  const int grp = rest / (kGroupRows * tiles_n);
  const int within = rest - grp * kGroupRows * tiles_n;
  const int left = tiles_m - grp * kGroupRows;
  const int gm = left < kGroupRows ? left : kGroupRows;
  tm = (int64_t)grp * kGroupRows + within % gm;
  tn = within / gm;
}

// Bias, activation and store of 4 consecutive outputs y[m][f..f+3] (f % 4 == 0).
// Gated residual: row m of sample g = m / rg.rows is row m - g * rg.rows of that sample's
// block of C, with that sample's gate.  QKV splice: the same row split over sp.grp_rows picks
// the sample's K / V buffers.
template <int EPI>
__device__ __forceinline__ void gemm_store4(float v0, float v1, float v2, float v3, int64_t m, int64_t f,
                                            const float* __restrict__ bias, void* __restrict__ C, int64_t ldc,
                                            const float* __restrict__ gate, const QkvSplice& sp,
                                            const RowGroups& rg) {
  const float4 bv = *reinterpret_cast<const float4*>(bias + f);
  v0 += bv.x;
  v1 += bv.y;
  v2 += bv.z;
  v3 += bv.w;
  if constexpr (EPI == kEpiGatedResidual) {
    const int64_t g = m / rg.rows;
    float* cp = static_cast<float*>(C) + g * rg.x_stride + (m - g * rg.rows) * ldc + f;
    const float4 gv = *reinterpret_cast<const float4*>(gate + g * rg.p_stride + f);
    float4 cv = *reinterpret_cast<float4*>(cp);
    cv.x += gv.x * v0;
    cv.y += gv.y * v1;
    cv.z += gv.z * v2;
    cv.w += gv.w * v3;
    *reinterpret_cast<float4*>(cp) = cv;
  } else if constexpr (EPI == kEpiQkvSplice) {
    const bf16x4 o = {(bf16)v0, (bf16)v1, (bf16)v2, (bf16)v3};
    const int64_t g = m / sp.grp_rows;
    const int64_t r = sp.row0 + (m - g * sp.grp_rows);      // buffer row of this sample
    if (f < sp.h) {
      *reinterpret_cast<bf16x4*>(static_cast<bf16*>(C) + m * ldc + f) = o;
    } else if (f < 2 * sp.h) {
      *reinterpret_cast<bf16x4*>(static_cast<bf16*>(sp.k) + g * sp.k_stride + r * sp.h + (f - sp.h)) = o;
    } else {
      // K8: element (r, c) at ((r / 8) * h + c) * 8 + r % 8, so columns c .. c+3 are 8 apart
      const int64_t c = f - 2 * sp.h;
      bf16* vp = static_cast<bf16*>(sp.v) + g * sp.v_stride + ((r >> 3) * sp.h + c) * 8 + (r & 7);
      vp[0] = o[0];
      vp[8] = o[1];
      vp[16] = o[2];
      vp[24] = o[3];
    }
  } else {
    const bf16x4 o = {(bf16)epi_act<EPI>(v0), (bf16)epi_act<EPI>(v1), (bf16)epi_act<EPI>(v2),
                      (bf16)epi_act<EPI>(v3)};
    *reinterpret_cast<bf16x4*>(static_cast<bf16*>(C) + m * ldc + f) = o;
  }
}

// Epilogue of a BF x BT tile held by 4 wavefronts in a 2 x 2 grid:
//   acc[i][t][4g+j] = y[token m0 + wt*BT/2 + t*32 + l32][feature n0 + wf*BF/2 + i*32 + 8g + 4hi + j].
// With SPLIT the slice stores its fp32 partial tile (part[split][m][f]) for the reduce pass.
template <int BF, int BT, int FB, int TB, int EPI, bool SPLIT>
__device__ __forceinline__ void gemm_epilogue(f32x16 (&acc)[FB][TB], int64_t m0, int64_t n0, int64_t M, int64_t N,
                                              const float* __restrict__ bias, void* __restrict__ C, int64_t ldc,
                                              const float* __restrict__ gate, const QkvSplice& sp,
                                              const RowGroups& rg, int split, float* __restrict__ part) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int wf = wave & 1, wt = wave >> 1;
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    const int64_t m = m0 + wt * (BT / 2) + t * 32 + l32;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < FB; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t f = n0 + wf * (BF / 2) + i * 32 + 8 * g + 4 * hi;
        if (f >= N) continue;
        if constexpr (SPLIT)
          *reinterpret_cast<float4*>(part + ((int64_t)split * M + m) * N + f) =
              make_float4(acc[i][t][4 * g + 0], acc[i][t][4 * g + 1], acc[i][t][4 * g + 2], acc[i][t][4 * g + 3]);
        else
          gemm_store4<EPI>(acc[i][t][4 * g + 0], acc[i][t][4 * g + 1], acc[i][t][4 * g + 2], acc[i][t][4 * g + 3], m,
                           f, bias, C, ldc, gate, sp, rg);
      }
  }
}

// Sum of the k slices of a split GEMM, then bias and the epilogue.  One thread per 4
// consecutive outputs of a row; slices are summed in order, so the result is deterministic.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const float* __restrict__ part, int n_split, int64_t M,
                                                          int64_t N, const float* __restrict__ bias,
                                                          void* __restrict__ C, int64_t ldc,
                                                          const float* __restrict__ gate, QkvSplice sp,
                                                          RowGroups rg) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nq = N / 4;
  if (id >= M * nq) return;
  const int64_t m = id / nq;
  const int64_t f = (id - m * nq) * 4;
  float4 s = *reinterpret_cast<const float4*>(part + m * N + f);
  for (int s2 = 1; s2 < n_split; ++s2) {
    const float4 v = *reinterpret_cast<const float4*>(part + ((int64_t)s2 * M + m) * N + f);
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  gemm_store4<EPI>(s.x, s.y, s.z, s.w, m, f, bias, C, ldc, gate, sp, rg);
}

// Reduce pass of a remainder split: the k slices of tiles n_whole.. (tile order of
// gemm_tile_of), one thread per 4 consecutive outputs of a tile row; slices summed in order.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_reduce_tiles_kernel(const float* __restrict__ part, int n_split,
                                                                int64_t n_whole, int64_t n_tiles, int tiles_n,
                                                                int64_t M, int64_t N, const float* __restrict__ bias,
                                                                void* __restrict__ C, int64_t ldc,
                                                                const float* __restrict__ gate, QkvSplice sp,
                                                                RowGroups rg) {
  constexpr int T = 128;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (n_tiles - n_whole) * T * (T / 4)) return;
  const int64_t tile = n_whole + id / (T * (T / 4));
  const int within = (int)(id % (T * (T / 4)));
  int64_t tm;
  int tn;
  gemm_tile_of((int)tile, (int)((M + T - 1) / T), tiles_n, tm, tn);
  const int64_t m = tm * T + within / (T / 4);
  const int64_t f = (int64_t)tn * T + (within % (T / 4)) * 4;
  if (m >= M || f >= N) return;
  float4 s = *reinterpret_cast<const float4*>(part + m * N + f);
  for (int s2 = 1; s2 < n_split; ++s2) {
    const float4 v = *reinterpret_cast<const float4*>(part + ((int64_t)s2 * M + m) * N + f);
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  gemm_store4<EPI>(s.x, s.y, s.z, s.w, m, f, bias, C, ldc, gate, sp, rg);
}

// bf16 tile kernel: BF features x BT tokens per workgroup (4 wavefronts in a 2 x 2 grid, each
// (BF/2) x (BT/2) = FB x TB blocks of 32 x 32), k staged 64 at a time (4 MFMA k-steps per
// barrier), two workgroups per CU.  Tiles [0, n_whole) run whole; with SPLIT, tiles n_whole..
// run as n_split k slices each (n_whole = 0: every tile split).  The W rows and X rows of a k tile are copied global ->
// LDS with direct 16-byte loads into a 2-stage ring (one tile ahead; the other resident
// workgroup covers the rest of the latency); LDS units are swizzled so every 8-lane operand
// read phase hits distinct bank groups, and the operands of k-step s+1 are read while the
// MFMAs of step s run.  With SPLIT, the workgroup covers one slice of the k range and writes
// an fp32 partial tile; gemm_reduce_kernel then sums the slices and applies the epilogue.
template <int BF, int BT, int EPI, bool SPLIT>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(
    const bf16* __restrict__ A, int64_t lda, const bf16* __restrict__ W, const float* __restrict__ bias, int64_t M,
    int64_t N, int64_t K, void* __restrict__ C, int64_t ldc, const float* __restrict__ gate, int tiles_n,
    int n_split, int ktiles_per_split, int64_t n_whole, float* __restrict__ part, QkvSplice sp, RowGroups rg) {
  constexpr int BK = 64;                 // k per stage: four MFMA k-steps
  constexpr int KSTEPS = BK / 16;
  constexpr int ROWS = BF + BT;          // stage rows: W rows, then X rows
  constexpr int UNITS = ROWS * 8;        // 16-byte units per stage (8 per row)
  constexpr int NINST = UNITS / 64;      // 64-lane direct loads per stage
  constexpr int NPW = NINST / 4;         // per wavefront
  constexpr int NSTAGE = 2;
  constexpr int FB = BF / 64, TB = BT / 64;
  static_assert(NINST % 4 == 0, "stage must split evenly over 4 wavefronts");
  static_assert(BF * 8 % 256 == 0, "each load fills only W rows or only X rows");
  __shared__ __attribute__((aligned(16))) uint4 lds[NSTAGE][UNITS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int wf = wave & 1, wt = wave >> 1;

  bool sliced = SPLIT;
  int split = 0, rest;
  if (SPLIT && n_whole > 0) {
    // remainder split: on every XCD (blocks are dealt to the 8 XCDs round-robin, and each XCD
    // starts its blocks in order) the first n_whole / 8 blocks run a contiguous run of whole
    // tiles, the later ones the k slices, so the slices fill the last round of every XCD
    const int x = (int)(blockIdx.x % 8), j = (int)(blockIdx.x / 8);
    const int wpx = (int)(n_whole / 8);
    sliced = j >= wpx;
    if (sliced) {
      const int64_t si = (int64_t)(j - wpx) * 8 + x;
      split = (int)(si % n_split);
      rest = (int)(n_whole + si / n_split);
    } else {
      rest = x * wpx + j;
    }
  } else {
    const int lid = gemm_xcd_remap(blockIdx.x, gridDim.x);
    split = SPLIT ? lid % n_split : 0;
    rest = SPLIT ? lid / n_split : lid;
  }
  int64_t tile_m;
  int tile_n;
  gemm_tile_of(rest, (int)((M + BT - 1) / BT), tiles_n, tile_m, tile_n);
  const int64_t n0 = (int64_t)tile_n * BF;
  const int64_t m0 = tile_m * BT;
  const int64_t nkt = K / BK;
  const int64_t kt0 = sliced ? (int64_t)split * ktiles_per_split : 0;
  const int64_t kt1 = sliced && kt0 + ktiles_per_split < nkt ? kt0 + ktiles_per_split : nkt;

  // unit of (row, chunk c in 0..7): rows r..r+7 at one chunk land in 8 distinct bank groups
  auto unit = [](int r, int c) { return r * 8 + (c ^ (r & 7)); };

  // per-lane byte offset of each of this wavefront's loads from the tile's row-0 base (rows
  // past M or N read the last valid row; their results are never stored)
  const bf16* Wt = W + n0 * K;
  const bf16* Xt = A + m0 * lda;
  uint32_t off[NPW];
  bool wrow[NPW];
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    const int u = (wave + 4 * j) * 64 + lane;
    const int r = u >> 3;
    const int c = (u & 7) ^ (r & 7);
    wrow[j] = (wave + 4 * j) * 64 < BF * 8;     // wavefront-uniform
    if (r < BF) {
      const int64_t rr = n0 + r < N ? r : N - 1 - n0;
      off[j] = (uint32_t)((rr * K + c * 8) * 2);
    } else {
      const int64_t rr = m0 + (r - BF) < M ? r - BF : M - 1 - m0;
      off[j] = (uint32_t)((rr * lda + c * 8) * 2);
    }
  }
  auto issue = [&](int64_t kt, int st) {
    const char* wb = reinterpret_cast<const char*>(Wt + kt * BK);
    const char* xb = reinterpret_cast<const char*>(Xt + kt * BK);
#pragma unroll
    for (int j = 0; j < NPW; ++j) dma_load16(wrow[j] ? wb : xb, off[j], &lds[st][(wave + 4 * j) * 64]);
  };

  f32x16 acc[FB][TB];
#pragma unroll
  for (int i = 0; i < FB; ++i)
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][t][e] = 0.f;

  auto read_frags = [&](const uint4* L, int ks, bf16x8 (&a)[FB], bf16x8 (&b)[TB]) {
#pragma unroll
    for (int i = 0; i < FB; ++i)
      a[i] = *reinterpret_cast<const bf16x8*>(&L[unit(wf * (BF / 2) + i * 32 + l32, 2 * ks + hi)]);
#pragma unroll
    for (int t = 0; t < TB; ++t)
      b[t] = *reinterpret_cast<const bf16x8*>(&L[unit(BF + wt * (BT / 2) + t * 32 + l32, 2 * ks + hi)]);
  };

  issue(kt0, 0);
  int st = 0;
  // One k tile; `more`: tile kt+1 exists (the steady-state body then has no branch, so the
  // compiler waits for exactly the operand reads each MFMA needs).
  auto ktile = [&](int64_t kt, bool more) {
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // this wavefront's loads of tile kt are done
    lds_barrier();   // ... for every wavefront; all are done reading the other stage
    const uint4* L = lds[st];
    bf16x8 a[2][FB], b[2][TB];
    read_frags(L, 0, a[0], b[0]);                      // before the loads: nothing crosses their asm
    if (more) issue(kt + 1, st ^ 1);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if (ks + 1 < KSTEPS) read_frags(L, ks + 1, a[(ks + 1) & 1], b[(ks + 1) & 1]);
#pragma unroll
      for (int i = 0; i < FB; ++i)
#pragma unroll
        for (int t = 0; t < TB; ++t)
          acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks & 1][i], b[ks & 1][t], acc[i][t], 0, 0, 0);
    }
    // schedule: operand reads of k-steps 0 and 1, then each k-step's MFMAs followed by the
    // reads of the k-step after the next, so every read has one k-step of MFMAs to land
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * (FB + TB), 0);
#pragma unroll
    for (int ks = 0; ks + 2 < KSTEPS; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, FB * TB, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, FB + TB, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * FB * TB, 0);
    st ^= 1;
  };
  int64_t kt = kt0;
  for (; kt + 1 < kt1; ++kt) ktile(kt, true);
  if (kt < kt1) ktile(kt, false);

  if (sliced)
    gemm_epilogue<BF, BT, FB, TB, EPI, true>(acc, m0, n0, M, N, bias, C, ldc, gate, sp, rg, split, part);
  else
    gemm_epilogue<BF, BT, FB, TB, EPI, false>(acc, m0, n0, M, N, bias, C, ldc, gate, sp, rg, split, part);
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
                                                       int tiles_n, RowGroups rg) {
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
      if constexpr (EPI == kEpiGatedResidual) {
        const int64_t g = m / rg.rows;
        C[g * rg.x_stride + (m - g * rg.rows) * ldc + n] += gate[g * rg.p_stride + n] * v;
      } else {
        C[m * ldc + n] = epi_act<EPI>(v);
      }
    }
  }
}

static int gemm_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) ==
                                                hipSuccess && v > 0)
      cus = v;
    else
      cus = 256;
    (void)hipGetLastError();
  }
  return cus;
}

// Work division of a bf16 GEMM with 128 x 128 tiles (two resident workgroups per CU): the
// smallest estimated time over
//   * a uniform k split s (s = 1: none): rounds of resident workgroups x one slice's time (a
//     fixed cost plus its FLOPs at one workgroup's measured rate), plus writing and re-reading
//     the fp32 partials;
//   * a remainder split s: the full rounds of whole tiles, then the last round's few tiles in
//     s slices each (at most one round of slices), plus their partials and the reduce launch.
// A split needs at least 4 k tiles per slice and fits the workspace ([s][m][n] fp32).
// Before any of that: a grid of 192 x 128 tiles (n % 192 == 0) with at least 1.5 tiles per CU
// runs whole with that tile.  Measured on the stage shapes (us, whole 192 x 128 against the
// 128 x 128 plan): 2048 x 4608 x 1536 40.7 / 46.2, 2048 x 6144 x 1536 48.0 / 54.1,
// 2048 x 9216 x 3072 113.9 / 130.2, 2048 x 12288 x 3072 152.3 / 156.4, 16384 x 1152 x 1152
// 54.8 / 63.4, 16384 x 1152 x 4608 167.2 / 183.7; with one tile per CU it loses
// (2048 x 3072 x 3072: 49.9 / 45.5; 2048 x 3072 x 12288: 165.8 / 153.1).
struct GemmPlan {
  int bf = 128;           // features per tile (tokens per tile: 128)
  int split = 1;          // k slices per split tile
  int64_t whole = 0;      // tiles run whole (the first in tile order); the rest are split
  int64_t tiles = 0;
};

static GemmPlan gemm_split_plan(int64_t m, int64_t n, int64_t k, size_t ws_bytes) {
  constexpr int64_t kTile = 128, kBk = 64;
  constexpr double kFixedS = 3e-6;       // per-tile fixed cost (prologue, epilogue)
  constexpr double kRate = 1.65e12;      // FLOP/s of one resident workgroup
  constexpr double kHbm = 5.0e12;        // B/s for partial traffic
  constexpr double kLaunchS = 2e-6;      // the extra reduce launch
  const int64_t slots = 2 * (int64_t)gemm_cus();
  if (n % 192 == 0) {
    const int64_t tiles192 = ((m + kTile - 1) / kTile) * (n / 192);
    if (2 * tiles192 >= 3 * (int64_t)gemm_cus()) {
      GemmPlan wide;
      wide.bf = 192;
      wide.tiles = wide.whole = tiles192;
      return wide;
    }
  }
  const int64_t tiles = ((m + kTile - 1) / kTile) * ((n + kTile - 1) / kTile);
  const double tile_s = 2.0 * kTile * kTile * (double)k / kRate;
  GemmPlan best;
  best.tiles = tiles;
  best.whole = tiles;
  double best_t = 1e30;
  // A grid that gives every CU a tile is not split uniformly: the rate above is that of two
  // workgroups per CU, and the CUs left with one run it faster, which the estimate misses
  // (2048 x 3072 x 12288, 384 tiles: 163 us whole against 186 us split 4 ways).
  const bool fills = tiles >= (int64_t)gemm_cus();
  for (int sp = 1; sp <= kMaxGemmSplit; ++sp) {
    if (sp > 1 && fills) break;
    if (sp > 1 && k / kBk < 4LL * sp) break;
    if (sp > 1 && (size_t)sp * m * n * sizeof(float) > ws_bytes) break;
    const double t = (double)((tiles * sp + slots - 1) / slots) * (kFixedS + tile_s / sp) +
                     (sp > 1 ? 2.0 * sp * (double)m * (double)n * sizeof(float) / kHbm + kLaunchS : 0.0);
    if (t < best_t * 0.98) {
      best_t = t;
      best.split = sp;
      best.whole = sp > 1 ? 0 : tiles;
    }
  }
  // Only a small remainder (at most one workgroup for every fourth CU) is worth it: a last round
  // that runs part full runs its lone workgroups faster than a full round's, so the measured
  // gain shrinks with the remainder (2048 x 4608 x 1536, 64 of 576 tiles left: 49.0 -> 45.6 us;
  // 2048 x 9216 x 3072, 128 of 1152: 135.9 -> 133.2; 16384 x 1152 x 4608, 128 of 1152:
  // 198.9 -> 207.7).  The full rounds must divide evenly over the 8 XCDs.
  const int64_t rem = tiles % slots;
  if (tiles > slots && rem > 0 && rem * 8 <= slots && (tiles - rem) % 8 == 0) {
    const int64_t full = tiles - rem;
    for (int sp = 2; sp <= kMaxGemmSplit; ++sp) {
      if (k / kBk < 4LL * sp || rem * sp > slots) break;
      if ((size_t)sp * m * n * sizeof(float) > ws_bytes) break;
      const double t = (double)(full / slots) * (kFixedS + tile_s) + kFixedS + tile_s / sp +
                       2.0 * sp * (double)rem * kTile * kTile * sizeof(float) / kHbm + kLaunchS;
      if (t < best_t * 0.98) {
        best_t = t;
        best.split = sp;
        best.whole = full;
      }
    }
  }
  return best;
}

size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  const GemmPlan plan = gemm_split_plan(m, n, k, (size_t)-1);
  return plan.split > 1 ? (size_t)plan.split * m * n * sizeof(float) : 0;
}

template <int EPI>
static hipError_t launch_gemm_epi(const void* a, int64_t lda, const void* w, const float* bias, int64_t m, int64_t n,
                                  int64_t k, void* c, int64_t ldc, const float* gate, int dtype, void* ws,
                                  size_t ws_bytes, hipStream_t s, const QkvSplice& sp, const RowGroups& rg,
                                  const LnAfter* ln, bool* ln_done) {
  if (dtype == kDtypeBF16) {
    // the tile kernel reads whole 64-deep k tiles and 64-feature halves of its tiles
    if (k % 64 != 0 || n % 64 != 0) return hipErrorInvalidValue;
    const bf16* A = static_cast<const bf16*>(a);
    const bf16* Wt = static_cast<const bf16*>(w);
    const GemmPlan plan = gemm_split_plan(m, n, k, ws ? ws_bytes : 0);
    const int nkt = (int)(k / 64);
    if (plan.bf == 192) {
      hipLaunchKernelGGL((gemm_bf16_kernel<192, 128, EPI, false>), dim3((unsigned)plan.tiles), dim3(256), 0, s, A, lda,
                         Wt, bias, m, n, k, c, ldc, gate, (int)(n / 192), 1, nkt, plan.tiles, nullptr, sp, rg);
      return hipGetLastError();
    }
    const int tiles_n = (int)((n + 127) / 128);
    const int64_t tiles = plan.tiles;
    const int kps = (nkt + plan.split - 1) / plan.split;
    const int used = (nkt + kps - 1) / kps;          // every slice gets at least one k tile
    if (used > 1 && (size_t)used * m * n * sizeof(float) > ws_bytes) return hipErrorInvalidValue;
    float* part = static_cast<float*>(ws);
    const dim3 grid((unsigned)(plan.whole + (tiles - plan.whole) * used));
    if (used == 1)
      hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, EPI, false>), grid, dim3(256), 0, s, A, lda, Wt, bias, m, n, k, c,
                         ldc, gate, tiles_n, 1, nkt, tiles, nullptr, sp, rg);
    else
      hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, EPI, true>), grid, dim3(256), 0, s, A, lda, Wt, bias, m, n, k, c,
                         ldc, gate, tiles_n, used, kps, plan.whole, part, sp, rg);
    if (used > 1 && plan.whole > 0) {
      const int64_t units = (tiles - plan.whole) * 128 * 32;
      hipLaunchKernelGGL(gemm_reduce_tiles_kernel<EPI>, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s, part,
                         used, plan.whole, tiles, tiles_n, m, n, bias, c, ldc, gate, sp, rg);
    } else if (used > 1) {
      if (EPI == kEpiGatedResidual && ln && n <= kMaxHidden) {
        // the reduce pass already holds whole updated rows: it applies the next LayerNorm too
        const hipError_t e =
            launch_reduce_residual_ln(part, used, m, (int)n, bias, static_cast<float*>(c), ldc, gate, rg, *ln, s);
        if (e != hipSuccess) return e;
        if (ln_done) *ln_done = true;
      } else {
        const int64_t units = m * (n / 4);
        hipLaunchKernelGGL(gemm_reduce_kernel<EPI>, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s, part,
                           used, m, n, bias, c, ldc, gate, sp, rg);
      }
    }
  } else {
    const int tiles_n = (int)((n + 63) / 64);
    const int64_t tiles = (int64_t)tiles_n * ((m + 63) / 64);
    hipLaunchKernelGGL(gemm_f32_kernel<EPI>, dim3((unsigned)tiles), dim3(256), 0, s, static_cast<const float*>(a), lda,
                       static_cast<const float*>(w), bias, m, n, k, static_cast<float*>(c), ldc, gate, tiles_n, rg);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const void* a, int64_t lda, const void* w, const float* bias, int64_t m, int64_t n, int64_t k,
                       int epi, void* c, int64_t ldc, const float* gate, int dtype, void* ws, size_t ws_bytes,
                       hipStream_t s, const QkvSplice* splice, const RowGroups* groups, const LnAfter* ln,
                       bool* ln_done) {
  if (ln_done) *ln_done = false;
  if (m <= 0) return hipSuccess;
  const QkvSplice sp = splice ? *splice : QkvSplice{nullptr, nullptr, 0, 0, m, 0, 0};
  const RowGroups rg = groups ? *groups : RowGroups{m, 0, 0};
  if (sp.grp_rows <= 0 || rg.rows <= 0) return hipErrorInvalidValue;
  switch (epi) {
    case kEpiStore:
      return launch_gemm_epi<kEpiStore>(a, lda, w, bias, m, n, k, c, ldc, gate, dtype, ws, ws_bytes, s, sp, rg,
                                        nullptr, nullptr);
    case kEpiGeluTanh:
      return launch_gemm_epi<kEpiGeluTanh>(a, lda, w, bias, m, n, k, c, ldc, gate, dtype, ws, ws_bytes, s, sp, rg,
                                           nullptr, nullptr);
    case kEpiGeluErf:
      return launch_gemm_epi<kEpiGeluErf>(a, lda, w, bias, m, n, k, c, ldc, gate, dtype, ws, ws_bytes, s, sp, rg,
                                          nullptr, nullptr);
    case kEpiQkvSplice:
      if (dtype != kDtypeBF16 || !splice) return hipErrorInvalidValue;
      return launch_gemm_epi<kEpiQkvSplice>(a, lda, w, bias, m, n, k, c, ldc, gate, dtype, ws, ws_bytes, s, sp, rg,
                                            nullptr, nullptr);
    case kEpiGatedResidual:
      return launch_gemm_epi<kEpiGatedResidual>(a, lda, w, bias, m, n, k, c, ldc, gate, dtype, ws, ws_bytes, s, sp,
                                                rg, ln, ln_done);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace pf
