// Projections of the DiT block: y = a . w^T + bias with fused epilogues.
//
// bf16 path: MFMA v_mfma_f32_32x32x16_bf16, fp32 accumulation.  The kernel computes
// output tiles transposed (features x tokens): the MFMA "A" operand is a block of 32
// weight rows and the "B" operand a block of 32 activation rows, both read as 8
// consecutive k-values (16 bytes) per lane from LDS.  The 32x32 accumulator then holds,
// per lane, one token and 4 consecutive output features per 8-row group, so every
// epilogue stores 4 contiguous values per access (8 B bf16 / 16 B fp32).
//
// Tiles: 128 x 128 with a 2-stage ring, two workgroups per CU.  A 128 x 64 variant and three
// deep-ring variants (256 x 256 and 128 x 128 with one workgroup per CU, 256 x 128 with two)
// can be forced for comparison.  Grids too small to fill the GPU split k: every slice writes its
// fp32 partial tile and a reduce pass sums the slices in order (deterministic) and applies the
// epilogue.  (A last-arriving-slice
// merge inside the GEMM measured slower on MI355X: the partials cross XCDs, whose L2s are
// not coherent, so they must be written through and read back from the device-coherent
// level, a longer latency chain than one more launch.)
//
// Workgroup ids map to tiles XCD by XCD (consecutive ids on one XCD), and within that in
// groups of kGroupRows tile rows walked column by column, so the workgroups an XCD runs at
// once share a few weight and activation row blocks in its L2.
//
// fp32 path (tiny fp32 stages only): a plain 64x64 LDS-tiled FMA kernel.
#include "pf_internal.h"

#include <cstdlib>
#include <cstring>

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

// bf16 tile kernel: BF features x BT tokens per workgroup (4 wavefronts in a 2 x 2 grid, each
// (BF/2) x (BT/2) = FB x TB blocks of 32 x 32), k staged 64 at a time (4 MFMA k-steps per
// barrier), two workgroups per CU.  The W rows and X rows of a k tile are copied global ->
// LDS with direct 16-byte loads into a 2-stage ring (one tile ahead; the other resident
// workgroup covers the rest of the latency); LDS units are swizzled so every 8-lane operand
// read phase hits distinct bank groups, and the operands of k-step s+1 are read while the
// MFMAs of step s run.  With SPLIT, the workgroup covers one slice of the k range and writes
// an fp32 partial tile; gemm_reduce_kernel then sums the slices and applies the epilogue.
template <int BF, int BT, int EPI, bool SPLIT>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(
    const bf16* __restrict__ A, int64_t lda, const bf16* __restrict__ W, const float* __restrict__ bias, int64_t M,
    int64_t N, int64_t K, void* __restrict__ C, int64_t ldc, const float* __restrict__ gate, int tiles_n,
    int n_split, int ktiles_per_split, float* __restrict__ part, QkvSplice sp, RowGroups rg) {
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

  const int lid = gemm_xcd_remap(blockIdx.x, gridDim.x);
  const int split = lid % n_split;
  const int rest = lid / n_split;
  int64_t tile_m;
  int tile_n;
  gemm_tile_of(rest, (int)((M + BT - 1) / BT), tiles_n, tile_m, tile_n);
  const int64_t n0 = (int64_t)tile_n * BF;
  const int64_t m0 = tile_m * BT;
  const int64_t nkt = K / BK;
  const int64_t kt0 = (int64_t)split * ktiles_per_split;
  const int64_t kt1 = kt0 + ktiles_per_split < nkt ? kt0 + ktiles_per_split : nkt;

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

  gemm_epilogue<BF, BT, FB, TB, EPI, SPLIT>(acc, m0, n0, M, N, bias, C, ldc, gate, sp, rg, split, part);
}

// vmcnt-only wait: at most N vector memory operations of this wavefront still outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// bf16 deep-ring kernel: BF features x BT tokens per workgroup, 4 wavefronts in a 2 x 2 grid,
// each (BF/2) x (BT/2) = FB x TB blocks of 32 x 32.  k is staged 32 at a time (two MFMA
// k-steps) in an NSTAGE ring filled NSTAGE - 1 tiles ahead by direct global -> LDS loads;
// the loads are counted with explicit vmcnt waits so they stay in flight across barriers.
// The first operands of tile kt+1 are read right after the barrier that publishes it, while
// the MFMAs of tile kt's last k-step are still running.  One workgroup per CU.
//   256 x 256, 4 stages: each wavefront 128 x 128 = 4 x 4 blocks (256 fp32 accumulators per
//     lane, kept in the accumulation registers), 0.5 KB of LDS operand reads per MFMA: the
//     highest per-k rate, for long reductions.
//   128 x 128, 8 stages: seven tiles (224 k values) in flight hide the load latency that
//     bounds a lone 2-stage workgroup, for grids with about one tile per CU.
template <int BF, int BT, int NSTAGE, int OCC, int EPI, bool SPLIT>
__global__ __launch_bounds__(256, OCC) void gemm_deep_kernel(const bf16* __restrict__ A, int64_t lda,
                                                           const bf16* __restrict__ W, const float* __restrict__ bias,
                                                           int64_t M, int64_t N, int64_t K, void* __restrict__ C,
                                                           int64_t ldc, const float* __restrict__ gate, int tiles_n,
                                                           int n_split, int ktiles_per_split,
                                                           float* __restrict__ part, QkvSplice sp, RowGroups rg) {
  constexpr int BK = 32;                 // k per stage: two MFMA k-steps
  constexpr int KSTEPS = BK / 16;
  constexpr int ROWS = BF + BT;          // stage rows: W rows, then X rows
  constexpr int UPR = BK / 8;            // 16-byte units per row (4)
  constexpr int UNITS = ROWS * UPR;      // 16-byte units per stage
  constexpr int NINST = UNITS / 64;      // 64-lane direct loads per stage
  constexpr int NPW = NINST / 4;         // per wavefront
  constexpr int FB = BF / 64, TB = BT / 64;
  constexpr int WJ = BF * UPR / 256;     // loads j < WJ of every wavefront fill W rows, the rest X rows
  static_assert(BF * UPR % 256 == 0 && BT * UPR % 256 == 0, "W and X loads split evenly over the wavefronts");
  static_assert(NSTAGE >= 3 && NSTAGE <= 9 && (NSTAGE - 2) * NPW < 64, "stage ring");
  __shared__ __attribute__((aligned(16))) uint4 lds[NSTAGE][UNITS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int wf = wave & 1, wt = wave >> 1;

  const int lid = gemm_xcd_remap(blockIdx.x, gridDim.x);
  const int split = lid % n_split;
  const int rest = lid / n_split;
  int64_t tile_m;
  int tile_n;
  gemm_tile_of(rest, (int)((M + BT - 1) / BT), tiles_n, tile_m, tile_n);
  const int64_t n0 = (int64_t)tile_n * BF;
  const int64_t m0 = tile_m * BT;
  const int64_t nkt = K / BK;
  const int64_t kt0 = (int64_t)split * ktiles_per_split;
  const int64_t kt1 = kt0 + ktiles_per_split < nkt ? kt0 + ktiles_per_split : nkt;

  // unit of (row r, chunk c in 0..3): the 8 rows of one 8-lane read phase land on distinct
  // 16-byte bank groups (rows r, r+1 differ by 64 B; pairs of rows take the 4 chunk XORs)
  auto unit = [](int r, int c) { return r * UPR + (c ^ ((r >> 1) & 3)); };

  // Loads: wavefront w issues loads i = w + 4j; the first BF * UPR / 64 fill the W rows, the
  // rest the X rows (j < WJ: W, else X, for every wavefront).  Per-lane byte offsets from the tile's
  // row-0 base; rows past N or M read the last valid row (their results are never stored).
  const bf16* Wt = W + n0 * K;
  const bf16* Xt = A + m0 * lda;
  uint32_t off[NPW];
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    const int u = (wave + 4 * j) * 64 + lane;
    const int r = u / UPR;
    const int c = (u % UPR) ^ ((r >> 1) & 3);
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
    for (int j = 0; j < NPW; ++j)
      dma_load16(j < WJ ? wb : xb, off[j], &lds[st][(wave + 4 * j) * 64]);
  };
  // this wavefront's loads of the tile before the `newer` most recently issued tiles are done
  // (newer <= NSTAGE - 2: at most that many later tiles are ever in flight)
  auto wait_tiles = [&](int newer) {
    if constexpr (NSTAGE - 2 >= 7) { if (newer >= 7) { wait_vmcnt<(NSTAGE - 2 >= 7 ? 7 : 0) * NPW>(); return; } }
    if constexpr (NSTAGE - 2 >= 6) { if (newer == 6) { wait_vmcnt<(NSTAGE - 2 >= 6 ? 6 : 0) * NPW>(); return; } }
    if constexpr (NSTAGE - 2 >= 5) { if (newer == 5) { wait_vmcnt<(NSTAGE - 2 >= 5 ? 5 : 0) * NPW>(); return; } }
    if constexpr (NSTAGE - 2 >= 4) { if (newer == 4) { wait_vmcnt<(NSTAGE - 2 >= 4 ? 4 : 0) * NPW>(); return; } }
    if constexpr (NSTAGE - 2 >= 3) { if (newer == 3) { wait_vmcnt<(NSTAGE - 2 >= 3 ? 3 : 0) * NPW>(); return; } }
    if (newer == 2) { wait_vmcnt<2 * NPW>(); return; }
    if (newer == 1) { wait_vmcnt<NPW>(); return; }
    wait_vmcnt<0>();
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

  const int64_t nt = kt1 - kt0;
  bf16x8 a[2][FB], b[2][TB];
  // prologue: tiles kt0 .. kt0+NSTAGE-2 in flight, wait for kt0
  for (int64_t u = 0; u < nt && u < NSTAGE - 1; ++u) issue(kt0 + u, (int)u);
  {
    const int64_t newer = (nt < NSTAGE - 1 ? nt : NSTAGE - 1) - 1;
    wait_tiles((int)(newer < 0 ? 0 : newer));
  }
  lds_barrier();
  if (nt > 0) read_frags(lds[0], 0, a[0], b[0]);
  int st = 0;
  // One k tile.  `steady`: tile kt + NSTAGE - 1 exists (so the loop body has no branch and
  // the compiler can wait for exactly the operand reads each MFMA needs).
  auto ktile = [&](int64_t kt, bool steady) {
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int cur = ks & 1, nxt = cur ^ 1;   // KSTEPS is even: k-step 0 of every tile uses buffer 0
      if (ks + 1 < KSTEPS) {
        read_frags(lds[st], ks + 1, a[nxt], b[nxt]);
      } else if (steady || kt + 1 < kt1) {
        // tile kt+1 landed for every wavefront; all are done with tile kt-1's stage
        if (steady) {
          wait_tiles(NSTAGE - 3);   // issued so far: tiles up to kt + NSTAGE - 2
        } else {
          const int64_t issued_after = (kt + NSTAGE - 2 < kt1 - 1 ? kt + NSTAGE - 2 : kt1 - 1) - (kt + 1);
          wait_tiles((int)issued_after);
        }
        lds_barrier();
        // operand reads first: the loads below are asm with a memory clobber, which nothing
        // crosses, so reads placed after them could only start once all loads are issued
        const int st1 = st + 1 == NSTAGE ? 0 : st + 1;
        read_frags(lds[st1], 0, a[nxt], b[nxt]);
        if (steady || kt + NSTAGE - 1 < kt1) issue(kt + NSTAGE - 1, st == 0 ? NSTAGE - 1 : st - 1);
      }
#pragma unroll
      for (int i = 0; i < FB; ++i)
#pragma unroll
        for (int t = 0; t < TB; ++t)
          acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][i], b[cur][t], acc[i][t], 0, 0, 0);
      if (ks + 1 == KSTEPS && steady) {
        // schedule: the next tile's operand reads, then this k-step's MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, FB + TB, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, FB * TB, 0);
      }
    }
    st = st + 1 == NSTAGE ? 0 : st + 1;
  };
  int64_t kt = kt0;
  for (; kt + NSTAGE - 1 < kt1; ++kt) ktile(kt, true);
  for (; kt < kt1; ++kt) ktile(kt, false);

  gemm_epilogue<BF, BT, FB, TB, EPI, SPLIT>(acc, m0, n0, M, N, bias, C, ldc, gate, sp, rg, split, part);
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

// Launch plan of a bf16 GEMM: kernel and k-split count.
enum GemmKind { kGemm128 = 0, kGemmDeep256 = 1, kGemmDeep128 = 2, kGemm128x64 = 3, kGemm256x128 = 4 };
struct GemmPlan {
  int kind;     // GemmKind: 128 x 128 2-stage (2 per CU), 256 x 256 4-stage, 128 x 128 8-stage (1 per CU),
                // 128 x 64 2-stage (2 per CU), 256 x 128 3-stage with k 32 deep (2 per CU)
  int split;    // k slices (1 = no split)
};

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

// The estimate only considers the 2-stage 128 x 128 kernel: with the grouped tile order it
// measured faster than both deep-ring kernels at every DiT projection shape on MI355X (k from
// 1152 to 12288, m from 1024 to 16384).  128 x 64 tiles beat it on narrow, short products
// timed alone (the out-projections: PixArt patch 17.6 -> 12.1 us) but lost inside the stage,
// where the weight tiles are no longer cache-resident and each is read by twice the
// workgroups (C2 step 2.354 -> 2.377 ms).  The others stay selectable through PF_GEMM_TILE.
// Smallest estimated time over tile size x k-split: rounds of resident workgroups x one
// slice's time (a fixed cost plus its FLOPs at the tile's measured rate), plus writing and
// re-reading the fp32 partials of a split.
// The environment variable PF_GEMM_TILE=128, 128x64, 256 or 128d (the 8-stage 128 x 128 kernel)
// forces the kernel (the k-split is still chosen by the estimate); any other value, or none,
// leaves both to the plan.
static int gemm_kind_override() {
  const char* v = std::getenv("PF_GEMM_TILE");
  if (!v) return -1;
  if (std::strcmp(v, "128") == 0) return kGemm128;
  if (std::strcmp(v, "256") == 0) return kGemmDeep256;
  if (std::strcmp(v, "128d") == 0) return kGemmDeep128;
  if (std::strcmp(v, "128x64") == 0) return kGemm128x64;
  if (std::strcmp(v, "256x128") == 0) return kGemm256x128;
  return -1;
}

// PF_GEMM_SPLIT=s forces s k slices where the workspace and k allow them (for measurements).
// PF_FUSE_LN=0 turns the fused reduce + LayerNorm off (read on every call).
static bool ln_fusion_enabled() {
  const char* e = getenv("PF_FUSE_LN");
  return !(e && e[0] == '0');
}

static int gemm_split_override() {
  const char* v = std::getenv("PF_GEMM_SPLIT");
  if (!v) return 0;
  const int sp = std::atoi(v);
  return sp >= 1 && sp <= kMaxGemmSplit ? sp : 0;
}

static GemmPlan gemm_plan(int64_t m, int64_t n, int64_t k, size_t ws_bytes) {
  const int cus = gemm_cus();
  const int force = gemm_kind_override();
  const int force_sp = gemm_split_override();
  GemmPlan best_plan{force >= 0 ? force : kGemm128, 1};
  double best = 1e30;
  for (int kind = 0; kind <= 4; ++kind) {
    if (force >= 0 ? kind != force : kind != kGemm128) continue;
    const int64_t bt = kind == kGemmDeep256 || kind == kGemm256x128 ? 256 : 128;   // features per tile
    const int64_t bm = kind == kGemm128x64 ? 64 : kind == kGemm256x128 ? 128 : bt;  // tokens per tile
    const int64_t bk = kind == kGemm128 || kind == kGemm128x64 ? 64 : 32;
    const int64_t tiles = ((m + bm - 1) / bm) * ((n + bt - 1) / bt);
    const int64_t slots = kind == kGemm128 || kind == kGemm128x64 || kind == kGemm256x128 ? 2 * (int64_t)cus
                                                                                          : (int64_t)cus;
    const double fixed_s = kind == kGemmDeep256 ? 30e-6 : 3e-6;
    const double rate = kind == kGemmDeep256 ? 6.7e12 : 1.65e12;      // FLOP/s of one resident workgroup
    for (int sp = 1; sp <= kMaxGemmSplit; ++sp) {
      if (sp > 1 && k / bk < 4LL * sp) break;
      if (sp > 1 && (size_t)sp * m * n * sizeof(float) > ws_bytes) break;
      if (force_sp && sp != force_sp) continue;
      const double t = (double)((tiles * sp + slots - 1) / slots) * (fixed_s + 2.0 * bt * bm * (double)k / sp / rate) +
                       (sp > 1 ? 2.0 * sp * (double)m * (double)n * sizeof(float) / 5.0e12 : 0.0);
      if (t < best * 0.98) {
        best = t;
        best_plan = {kind, sp};
      }
    }
  }
  return best_plan;
}

size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  const GemmPlan p = gemm_plan(m, n, k, (size_t)-1);
  return p.split > 1 ? (size_t)p.split * m * n * sizeof(float) : 0;
}

template <int EPI, bool SPLIT>
static constexpr auto gemm_small128 = gemm_bf16_kernel<128, 128, EPI, SPLIT>;
template <int EPI, bool SPLIT>
static constexpr auto gemm_small128x64 = gemm_bf16_kernel<128, 64, EPI, SPLIT>;
template <int EPI, bool SPLIT>
static constexpr auto gemm_deep256 = gemm_deep_kernel<256, 256, 4, 1, EPI, SPLIT>;
template <int EPI, bool SPLIT>
static constexpr auto gemm_deep128 = gemm_deep_kernel<128, 128, 8, 1, EPI, SPLIT>;
template <int EPI, bool SPLIT>
static constexpr auto gemm_wide = gemm_deep_kernel<256, 128, 3, 2, EPI, SPLIT>;

template <int EPI>
static void launch_gemm_epi(const void* a, int64_t lda, const void* w, const float* bias, int64_t m, int64_t n,
                            int64_t k, void* c, int64_t ldc, const float* gate, int dtype, void* ws,
                            size_t ws_bytes, hipStream_t s, const QkvSplice& sp, const RowGroups& rg,
                            const LnAfter* ln, bool* ln_done) {
  if (dtype == kDtypeBF16) {
    const bf16* A = static_cast<const bf16*>(a);
    const bf16* Wt = static_cast<const bf16*>(w);
    const GemmPlan p = gemm_plan(m, n, k, ws ? ws_bytes : 0);
    const int bt = p.kind == kGemmDeep256 || p.kind == kGemm256x128 ? 256 : 128;
    const int bm = p.kind == kGemm128x64 ? 64 : p.kind == kGemm256x128 ? 128 : bt;
    const int nkt = (int)(k / (p.kind == kGemm128 || p.kind == kGemm128x64 ? 64 : 32));
    const int tiles_n = (int)((n + bt - 1) / bt);
    const int64_t tiles = (int64_t)tiles_n * ((m + bm - 1) / bm);
    const int kps = (nkt + p.split - 1) / p.split;
    const int used = (nkt + kps - 1) / kps;          // every slice gets at least one k tile
    float* part = static_cast<float*>(ws);
    const dim3 grid((unsigned)(tiles * used));
#define PF_GEMM_LAUNCH(KERNEL)                                                                                       \
  do {                                                                                                               \
    if (used == 1)                                                                                                   \
      hipLaunchKernelGGL((KERNEL<EPI, false>), grid, dim3(256), 0, s, A, lda, Wt, bias, m, n, k, c, ldc, gate, tiles_n, \
                         1, nkt, nullptr, sp, rg);                                                                   \
    else                                                                                                             \
      hipLaunchKernelGGL((KERNEL<EPI, true>), grid, dim3(256), 0, s, A, lda, Wt, bias, m, n, k, c, ldc, gate, tiles_n, \
                         used, kps, part, sp, rg);                                                                   \
  } while (0)
    if (p.kind == kGemmDeep256) PF_GEMM_LAUNCH(gemm_deep256);
    else if (p.kind == kGemmDeep128) PF_GEMM_LAUNCH(gemm_deep128);
    else if (p.kind == kGemm128x64) PF_GEMM_LAUNCH(gemm_small128x64);
    else if (p.kind == kGemm256x128) PF_GEMM_LAUNCH(gemm_wide);
    else PF_GEMM_LAUNCH(gemm_small128);
#undef PF_GEMM_LAUNCH
    if (used > 1) {
      if (EPI == kEpiGatedResidual && ln && ln_fusion_enabled() && n <= kMaxHidden) {
        // the reduce pass already holds whole updated rows: it applies the next LayerNorm too
        (void)launch_reduce_residual_ln(part, used, m, (int)n, bias, static_cast<float*>(c), ldc, gate, rg, *ln, s);
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
      launch_gemm_epi<kEpiStore>(a, lda, w, bias, m, n, k, c, ldc, gate, dtype, ws, ws_bytes, s, sp, rg, nullptr,
                                 nullptr);
      break;
    case kEpiGeluTanh:
      launch_gemm_epi<kEpiGeluTanh>(a, lda, w, bias, m, n, k, c, ldc, gate, dtype, ws, ws_bytes, s, sp, rg, nullptr,
                                    nullptr);
      break;
    case kEpiGeluErf:
      launch_gemm_epi<kEpiGeluErf>(a, lda, w, bias, m, n, k, c, ldc, gate, dtype, ws, ws_bytes, s, sp, rg, nullptr,
                                   nullptr);
      break;
    case kEpiQkvSplice:
      if (dtype != kDtypeBF16 || !splice) return hipErrorInvalidValue;
      launch_gemm_epi<kEpiQkvSplice>(a, lda, w, bias, m, n, k, c, ldc, gate, dtype, ws, ws_bytes, s, sp, rg, nullptr,
                                     nullptr);
      break;
    default:
      launch_gemm_epi<kEpiGatedResidual>(a, lda, w, bias, m, n, k, c, ldc, gate, dtype, ws, ws_bytes, s, sp, rg, ln,
                                         ln_done);
      break;
  }
  return hipGetLastError();
}

}  // namespace pf
