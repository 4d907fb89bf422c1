// Patch attention: the queries of one patch attend over every row of a layer's
// full-spatial K/V buffer (PipeFusion keeps full attention; the buffer mixes fresh and
// stale rows).  Flash-style single pass with online softmax; no score matrix is stored.
//
// bf16 kernel (head_dim D in {64, 72, 128}), gfx950 MFMA v_mfma_f32_32x32x16_bf16:
//   * workgroup = 4 wavefronts; each wavefront owns QB blocks of 32 queries of one head,
//     so every K/V operand read from LDS feeds QB MFMAs.  Key tiles of 32 rows are copied
//     global -> LDS by the gfx950 direct 16-byte loads (no register staging) into a
//     5-stage ring; one barrier per tile.  K keeps its rows in a permuted, swizzled unit
//     order (conflict-free operand reads), V the K8 layout of the buffer (see pf.h).
//   * scores are computed transposed, S^T = K . Q^T, so each lane owns one query and 16
//     keys per block: the row max is a lane-local max chain plus one exchange with the
//     lane 32 away, and the row sum stays lane-local until the end.
//   * the K rows feeding the score MFMA are permuted (bits 2 and 3 of the row index
//     swapped) so that each lane's 8 consecutive score registers are 8 consecutive keys:
//     they pack directly into the bf16 "B" operand of O^T += V^T . P^T without any
//     cross-lane shuffle, and the matching V^T operand is one 16-byte K8 read per lane.
//   * softmax in base 2: p = exp2(s * log2(e)/sqrt(D) - m), fp32 statistics, P rounded to
//     bf16 for the P.V product and the row sum taken over the same rounded values (for
//     D = 72 by the P.V MFMA itself, through a ones row in the padding of O^T).  The reference max m is raised (and O, l rescaled) only
//     when a tile's max exceeds it by more than 8, so p <= 2^8 and the rescale is rare.
//   * D = 72 pads the score contraction to 80 and the output rows to 96 with zero
//     operands; nothing outside the real 72 columns is read or written.
//   * when there are too few (query tile, head) pairs to fill the GPU, the key range is
//     split across workgroups; each writes its unnormalised partial O with (m, l) and a
//     combine kernel merges them.
//   * the block index is remapped so each XCD (blocks are dealt round-robin to the 8
//     XCDs) works on a contiguous run of query tiles that share K/V in its L2.
//
// fp32 kernel (tiny fp32 stages only): one thread per query, key tiles in LDS.
#include "pf_internal.h"

namespace pf {

namespace {
constexpr int kTileKeys = 32;   // keys per LDS tile
}  // namespace

__device__ __forceinline__ int swap_bits23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  const int per = nb / 8, rem = nb % 8;
  const int x = bid % 8;
  return x * per + (x < rem ? x : rem) + bid / 8;
}

// Per head_dim tuning: query blocks of 32 per wavefront (QB) and the wavefronts per SIMD the
// register budget is sized for (MINW; 2 caps a wavefront at 256 registers).
#ifndef PF_ATTN_QB64
#define PF_ATTN_QB64 2
#endif
#ifndef PF_ATTN_QB72
#define PF_ATTN_QB72 2
#endif
#ifndef PF_ATTN_QB128
#define PF_ATTN_QB128 1
#endif
#ifndef PF_ATTN_MINW64
#define PF_ATTN_MINW64 2
#endif
#ifndef PF_ATTN_MINW72
#define PF_ATTN_MINW72 2
#endif
#ifndef PF_ATTN_MINW128
#define PF_ATTN_MINW128 2
#endif
template <int D> struct AttnCfg;
template <> struct AttnCfg<64> { static constexpr int QB = PF_ATTN_QB64, MINW = PF_ATTN_MINW64; };
template <> struct AttnCfg<72> { static constexpr int QB = PF_ATTN_QB72, MINW = PF_ATTN_MINW72; };
template <> struct AttnCfg<128> { static constexpr int QB = PF_ATTN_QB128, MINW = PF_ATTN_MINW128; };

template <int D, int QB>
__global__ __launch_bounds__(256, AttnCfg<D>::MINW) void attn_bf16_kernel(const bf16* __restrict__ Q, int64_t ldq,
                                                           const bf16* __restrict__ Kb, int64_t ldk,
                                                           const bf16* __restrict__ Vb, int64_t hidden,
                                                           int64_t S, int64_t rows, int n_qtiles, int n_split,
                                                           int tiles_per_split, bf16* __restrict__ O,
                                                           int64_t ldo, float* __restrict__ part_o,
                                                           float* __restrict__ part_ml, float scale_log2) {
  constexpr int BQ = 4 * 32 * QB;                     // queries per workgroup
  constexpr int KS = (D + 15) / 16;                   // k-steps of the score MFMA
  constexpr int DB = (D + 31) / 32;                   // 32-row blocks of O^T
  constexpr int TK = kTileKeys;
  constexpr int W = D / 8;                            // 16-byte units per K row
  constexpr int KU = TK * W;                          // units of the K part of a tile (= V part)
  constexpr int KUP = (KU + 63) / 64 * 64;            // ... rounded to whole 64-lane loads
  constexpr int NI = KUP / 64;                        // 64-lane direct loads per part
  constexpr int NINST = 2 * NI;                       // per tile (K loads, then V loads)
  constexpr int NJ = (NINST + 3) / 4;                 // most loads one wavefront issues per tile
  constexpr int NMIN = NINST / 4;                     // fewest
  constexpr int NSTAGE = 5;                           // tile t being read, t+1 .. t+3 loading

  // Tile stage in LDS, in 16-byte units.  K part: position p (0..31) holds key row
  // swap_bits23(p), W units per position, unit order swizzled so the 8 lanes of one LDS
  // read phase (positions p..p+7, same chunk) hit distinct bank groups.  V part (from unit
  // KUP): the K8 order of the buffer, [TK/8 groups][D][8 keys].
  __shared__ __attribute__((aligned(16))) uint4 lds[NSTAGE][2 * KUP];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = lid % n_qtiles;
  const int rest = lid / n_qtiles;
  const int split = rest % n_split;
  const int head = rest / n_split;
  const int64_t col0 = (int64_t)head * D;
  const int64_t ntiles = (S + TK - 1) / TK;
  const int64_t t_begin = (int64_t)split * tiles_per_split;
  const int64_t t_end = t_begin + tiles_per_split < ntiles ? t_begin + tiles_per_split : ntiles;

  int64_t q_row[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) q_row[qb] = (int64_t)qt * BQ + (wave * QB + qb) * 32 + l32;

  // Q^T fragments (the "B" operand of the score MFMA): 8 consecutive d of this lane's query.
  bf16x8 qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = ks * 16 + hi * 8;
      if (q_row[qb] < rows && d0 < D) {
        qf[qb][ks] = *reinterpret_cast<const bf16x8*>(Q + q_row[qb] * ldq + col0 + d0);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[qb][ks][e] = (bf16)0.f;
      }
    }

  f32x16 o[QB][DB];
  float m_ref[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[qb][db][e] = 0.f;
  }

  const int64_t ngroups = (S + 7) >> 3;   // K8 groups present in the V buffer
  auto k_unit = [](int p, int c) -> int {
    if constexpr (W % 2 == 1) return p * W + c;
    else if constexpr (W == 8) return p * 8 + (c ^ (p & 7));
    else return p * 16 + (c ^ (p & 15));
  };

  // Direct global -> LDS loads of key tile t into stage st: wavefront w issues the 64-lane
  // loads i = w, w+4, ...; lane l of load i fills unit 64i + l of its part.  Each lane's
  // byte offset from the tile's (uniform) base is fixed, so a full tile costs one address
  // add per load.  In a tile that runs past the end of the buffer, rows and groups read a
  // clamped (valid) address; their scores are masked and their V entries zeroed before use.
  uint32_t ld_off[NJ];
  int ld_row[NJ];
  bool ld_on[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int i = wave + 4 * j;
    const bool kpart = i < NI;
    const int u = (kpart ? i : i - NI) * 64 + lane;
    ld_on[j] = i < NINST && u < KU;
    if (kpart) {
      int p, c;
      if constexpr (W % 2 == 1) {
        p = u / W;
        c = u - p * W;
      } else if constexpr (W == 8) {
        p = u >> 3;
        c = (u & 7) ^ (p & 7);
      } else {
        p = u >> 4;
        c = (u & 15) ^ (p & 15);
      }
      const int row = swap_bits23(p);
      ld_row[j] = row;
      ld_off[j] = (uint32_t)(row * ldk * 2 + c * 16);
    } else {
      const int g = u / D, d = u - g * D;
      ld_row[j] = g;
      ld_off[j] = (uint32_t)((g * hidden + d) * 16);
    }
  }
  auto issue_tile = [&](int64_t t, int st) {
    const char* kbase = reinterpret_cast<const char*>(Kb + (t * TK) * ldk + col0);
    const char* vbase = reinterpret_cast<const char*>(Vb + (t * (TK / 8) * hidden + col0) * 8);
    const bool full = (t + 1) * TK <= S;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int i = wave + 4 * j;
      if (i >= NINST) continue;                   // wavefront-uniform
      if (!ld_on[j]) continue;                    // tail lanes of a part's last load
      const bool kpart = i < NI;
      const char* src = (kpart ? kbase : vbase) + ld_off[j];
      if (!full) {
        if (kpart) {
          const int64_t over = t * TK + ld_row[j] - (S - 1);
          if (over > 0) src -= over * ldk * 2;
        } else {
          const int64_t over = t * (TK / 8) + ld_row[j] - (ngroups - 1);
          if (over > 0) src -= over * hidden * 16;
        }
      }
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)&lds[st][(kpart ? i : KUP / 64 + i - NI) * 64],
                                       16, 0, 0);
    }
  };
  // Stage ring: tile t lives in stage (t - t_begin + 1) mod NSTAGE.
  auto next_stage = [](int st) { return st + 1 == NSTAGE ? 0 : st + 1; };
  auto wait_loads = [&](int newer_tiles) {   // at most `newer_tiles` tiles of loads still in flight
    if (newer_tiles >= 2) __builtin_amdgcn_s_waitcnt(((2 * NMIN) & 15) | (((2 * NMIN) >> 4) << 14) | (7 << 4) | (15 << 8));
    else if (newer_tiles == 1) __builtin_amdgcn_s_waitcnt((NMIN & 15) | ((NMIN >> 4) << 14) | (7 << 4) | (15 << 8));
    else __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
  };

  for (int64_t t = t_begin; t < t_end && t < t_begin + 3; ++t) issue_tile(t, (int)(t - t_begin + 1));

  // score tile t: S^T = K_t . Q^T (lane: query l32 of each block, 16 keys)
  auto scores = [&](int st, f32x16 (&sc)[QB]) {
    const uint4* base = lds[st];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[qb][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = ks * 16 + hi * 8;
      bf16x8 a;
      if (d0 < D) {
        a = *reinterpret_cast<const bf16x8*>(&base[k_unit(l32, 2 * ks + hi)]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = (bf16)0.f;
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][ks], sc[qb], 0, 0, 0);
    }
  };
  // keys of a lane's acc index 4g+j: t*32 + swap_bits23(8g + 4hi + j) = t*32 + 16(g>>1) + 8hi + 4(g&1) + j;
  // only the buffer's last tile has keys past S
  auto mask_scores = [&](int64_t t, f32x16 (&sc)[QB]) {
    const int lim = (int)(S - t * TK);      // valid keys in this tile (< 32 here)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (16 * (g >> 1) + 8 * hi + 4 * (g & 1) + j >= lim) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) sc[qb][4 * g + j] = -INFINITY;
        }
      }
  };
  auto tile_max = [&](const f32x16 (&sc)[QB], float (&mt)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float m0 = fmaxf(sc[qb][0], fmaxf(sc[qb][1], sc[qb][2]));
      float m1 = fmaxf(sc[qb][3], fmaxf(sc[qb][4], sc[qb][5]));
      float m2 = fmaxf(sc[qb][6], fmaxf(sc[qb][7], sc[qb][8]));
      float m3 = fmaxf(sc[qb][9], fmaxf(sc[qb][10], sc[qb][11]));
      float m4 = fmaxf(sc[qb][12], fmaxf(sc[qb][13], sc[qb][14]));
      float mx = fmaxf(fmaxf(m0, fmaxf(m1, m2)), fmaxf(m3, fmaxf(m4, sc[qb][15])));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      mt[qb] = mx * scale_log2;
    }
  };
  // D = 72: the padded O^T row 72 (lane l32 == 8 of the last block) multiplies ones, so the
  // P.V MFMA itself accumulates the row sum of the same bf16 weights; other head_dims keep
  // the row sum with v_dot2 in the softmax.
  constexpr bool kSumRow = D % 32 != 0;
  constexpr int kSumIdx = 4 * ((D % 32) / 8) + 0;          // acc index of row D in the last block (hi = 0)
  // O^T += V_t^T . P^T for two halves of 16 keys; `zero_tail` zeroes V rows past S
  auto pv = [&](int64_t t, int st, const bf16x8 (&pb)[QB][2], bool zero_tail) {
    const uint4* base = lds[st] + KUP;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int grp = 2 * h2 + hi;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = db * 32 + l32;
        bf16x8 a;
        if (d < D) {
          a = *reinterpret_cast<const bf16x8*>(&base[grp * D + d]);
          if (zero_tail) {
            const int lim = (int)(S - t * TK) - grp * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (e >= lim) a[e] = (bf16)0.f;
          }
        } else {
          const bf16 fill = (kSumRow && d == D) ? (bf16)1.0f : (bf16)0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) a[e] = fill;
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qb][h2], o[qb][db], 0, 0, 0);
      }
    }
  };
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
  // p = 2^(s*c - m) rounded to bf16 in pairs (the P.V operand); without the MFMA sum row the
  // row sum accumulates the same rounded values with v_dot2 against (1, 1)
  auto softmax = [&](const f32x16 (&sc)[QB], bf16x8 (&pc)[QB][2]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      uint32_t pk[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const f32x2 pp = {__builtin_amdgcn_exp2f(fmaf(sc[qb][2 * e], scale_log2, -m_ref[qb])),
                          __builtin_amdgcn_exp2f(fmaf(sc[qb][2 * e + 1], scale_log2, -m_ref[qb]))};
        const bf16x2 pb2 = __builtin_convertvector(pp, bf16x2);
        if constexpr (!kSumRow) l_run[qb] = __builtin_amdgcn_fdot2_f32_bf16(pb2, ones, l_run[qb], false);
        pk[e] = __builtin_bit_cast(uint32_t, pb2);
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const u32x4 w = {pk[4 * h2], pk[4 * h2 + 1], pk[4 * h2 + 2], pk[4 * h2 + 3]};
        pc[qb][h2] = __builtin_bit_cast(bf16x8, w);
      }
    }
  };

  // ---- main loop: tile t is in LDS; tiles up to t+4 are loading ----
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) m_ref[qb] = -INFINITY;
  int st = 1, st_issue = 4;   // stages of tiles t and t+3
  // `partial` is a literal at both call sites: only the buffer's last tile can run past S,
  // so the main loop carries no masking code.
  auto tile = [&](int64_t t, bool partial) {
    const int64_t ahead = t_end - 1 - t;              // tiles issued after t (at most 2)
    wait_loads((int)(ahead < 2 ? ahead : 2));
    __syncthreads();   // tile t landed for every wavefront; all are done with tile t-1
    if (t + 3 < t_end) issue_tile(t + 3, st_issue);

    f32x16 sc[QB];
    scores(st, sc);
    if (partial) mask_scores(t, sc);
    float mt[QB];
    tile_max(sc, mt);
    bool raise = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) raise |= mt[qb] > m_ref[qb] + 8.0f;
    if (__any(raise)) {
      // a tile max exceeds the reference by more than 2^8: move the reference, rescale O, l
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float m_new = fmaxf(m_ref[qb], mt[qb]);
        const float alpha = __builtin_amdgcn_exp2f(m_ref[qb] - m_new);
        m_ref[qb] = m_new;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[qb][db][e] *= alpha;
      }
    }
    bf16x8 pb[QB][2];
    softmax(sc, pb);
    pv(t, st, pb, partial);
    st = next_stage(st);
    st_issue = next_stage(st_issue);
  };
  const int64_t t_full = t_end * TK > S ? t_end - 1 : t_end;   // tiles before t_full are full
  for (int64_t t = t_begin; t < t_full; ++t) tile(t, false);
  if (t_full < t_end) tile(t_full, true);

  if constexpr (kSumRow) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float sum_row = o[qb][DB - 1][kSumIdx];   // valid in lanes hi == 0
      l_run[qb] = hi == 0 ? sum_row : 0.f;
    }
  }

  // ---- finish: lane holds O[query][d = db*32 + 8g + 4hi + j] ----
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32, 64);
    if (q_row[qb] >= rows) continue;
    if (n_split == 1) {
      const float inv = 1.0f / l_tot;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = db * 32 + 8 * g + 4 * hi;
          if (d < D) {
            bf16x4 ov = {(bf16)(o[qb][db][4 * g + 0] * inv), (bf16)(o[qb][db][4 * g + 1] * inv),
                         (bf16)(o[qb][db][4 * g + 2] * inv), (bf16)(o[qb][db][4 * g + 3] * inv)};
            *reinterpret_cast<bf16x4*>(O + q_row[qb] * ldo + col0 + d) = ov;
          }
        }
    } else {
      float* po = part_o + ((int64_t)split * rows + q_row[qb]) * hidden + col0;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = db * 32 + 8 * g + 4 * hi;
          if (d < D)
            *reinterpret_cast<float4*>(po + d) =
                make_float4(o[qb][db][4 * g + 0], o[qb][db][4 * g + 1], o[qb][db][4 * g + 2], o[qb][db][4 * g + 3]);
        }
      if (hi == 0) {
        const int64_t H = hidden / D;
        part_ml[(((int64_t)split * 2 + 0) * H + head) * rows + q_row[qb]] = m_ref[qb];
        part_ml[(((int64_t)split * 2 + 1) * H + head) * rows + q_row[qb]] = l_tot;
      }
    }
  }
}

// Merge the per-split partial results: O = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
// One thread per (row, head, 8 columns).
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml, int n_split,
                                                           int64_t rows, int H, bf16* __restrict__ O,
                                                           int64_t ldo) {
  constexpr int NC = D / 8;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= rows * H * NC) return;
  const int chunk = (int)(id % NC);
  const int64_t rest = id / NC;
  const int head = (int)(rest % H);
  const int64_t row = rest / H;
  const int64_t hidden = (int64_t)H * D;
  float M = -INFINITY;
  for (int sp = 0; sp < n_split; ++sp) M = fmaxf(M, part_ml[(((int64_t)sp * 2) * H + head) * rows + row]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  for (int sp = 0; sp < n_split; ++sp) {
    const float m = part_ml[(((int64_t)sp * 2) * H + head) * rows + row];
    const float l = part_ml[(((int64_t)sp * 2 + 1) * H + head) * rows + row];
    const float w = __builtin_amdgcn_exp2f(m - M);
    wsum += w * l;
    const float* po = part_o + ((int64_t)sp * rows + row) * hidden + (int64_t)head * D + chunk * 8;
    const float4 a = *reinterpret_cast<const float4*>(po);
    const float4 b = *reinterpret_cast<const float4*>(po + 4);
    acc[0] += w * a.x; acc[1] += w * a.y; acc[2] += w * a.z; acc[3] += w * a.w;
    acc[4] += w * b.x; acc[5] += w * b.y; acc[6] += w * b.z; acc[7] += w * b.w;
  }
  const float inv = 1.0f / wsum;
  bf16x8 out;
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = (bf16)(acc[e] * inv);
  *reinterpret_cast<bf16x8*>(O + row * ldo + (int64_t)head * D + chunk * 8) = out;
}

// ---------------------------------------------------------------------------------
// fp32: block = 64 queries of one head (one thread each), key tiles of 32 rows in LDS.
// Per tile: 32 scores in registers, tile max, one rescale of the running sums.
// ---------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(const float* __restrict__ Q, int64_t ldq,
                                                      const float* __restrict__ Kb, int64_t ldk,
                                                      const float* __restrict__ Vb, int64_t ldv,
                                                      int64_t S, int64_t rows, int n_qtiles,
                                                      float* __restrict__ O, int64_t ldo, float scale) {
  __shared__ float sK[32][D];
  __shared__ float sV[32][D];
  const int head = blockIdx.x / n_qtiles;
  const int qt = blockIdx.x - head * n_qtiles;
  const int64_t q_row = (int64_t)qt * 64 + threadIdx.x;
  const int64_t col0 = (int64_t)head * D;
  float q[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = q_row < rows ? Q[q_row * ldq + col0 + d] : 0.f;
    o[d] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  for (int64_t k0 = 0; k0 < S; k0 += 32) {
    for (int c = threadIdx.x; c < 32 * D; c += 64) {
      const int r = c / D, d = c - r * D;
      const int64_t key = k0 + r;
      sK[r][d] = key < S ? Kb[key * ldk + col0 + d] : 0.f;
      sV[r][d] = key < S ? Vb[key * ldv + col0 + d] : 0.f;
    }
    __syncthreads();
    const int nk = (int)((S - k0) < 32 ? (S - k0) : 32);
    float sc[32];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = fmaf(q[d], sK[r][d], acc);
      sc[r] = r < nk ? acc * scale : -INFINITY;
      mx = fmaxf(mx, sc[r]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = expf(m_run - m_new);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      const float p = expf(sc[r] - m_new);
      rs += p;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(p, sV[r][d], o[d]);
    }
    l_run = l_run * alpha + rs;
    __syncthreads();
  }
  if (q_row < rows) {
    const float inv = 1.0f / l_run;
#pragma unroll
    for (int d = 0; d < D; ++d) O[q_row * ldo + col0 + d] = o[d] * inv;
  }
}

// Workgroups of this kernel that fit on the device at once (CUs x blocks per CU).
template <int D>
static int attn_slots() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_bf16_kernel<D, AttnCfg<D>::QB>, 256, 0) !=
            hipSuccess || per_cu <= 0)
      per_cu = 1;
    (void)hipGetLastError();
    cached[dev] = cus * per_cu;
  }
  return cached[dev];
}

// Number of key-range splits: the smallest that minimises the estimated time
// ceil(wg * s / slots) / s, limited so every split keeps at least 8 key tiles and the
// partial results fit in the workspace.
static int choose_split(int64_t wg, int slots, int64_t ntiles, int64_t rows, int64_t hidden, int heads,
                        size_t ws_bytes) {
  int best = 1;
  double best_cost = (double)((wg + slots - 1) / slots);
  for (int sp = 2; sp <= kMaxAttnSplit; ++sp) {
    if (ntiles < 8LL * sp) break;
    if (attention_workspace_bytes(rows, hidden, heads, sp) > ws_bytes) break;
    const double cost = (double)((wg * sp + slots - 1) / slots) / sp * 1.03;   // 3% for the merge pass
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = sp;
    }
  }
  return best;
}

template <int D>
static hipError_t launch_attn_d(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v, int64_t ldv,
                                int64_t hidden, int64_t seq_kv, int64_t rows, int heads, void* o, int64_t ldo,
                                int dtype, void* ws, size_t ws_bytes, hipStream_t s) {
  if (dtype == kDtypeBF16) {
    constexpr int QB = AttnCfg<D>::QB;
    constexpr int BQ = 4 * 32 * QB;
    const int n_qtiles = (int)((rows + BQ - 1) / BQ);
    const int64_t ntiles = (seq_kv + kTileKeys - 1) / kTileKeys;
    const int64_t wg = (int64_t)n_qtiles * heads;
    const int n_split = ws ? choose_split(wg, attn_slots<D>(), ntiles, rows, hidden, heads, ws_bytes) : 1;
    const int tps = (int)((ntiles + n_split - 1) / n_split);
    const int n_used = (int)((ntiles + tps - 1) / tps);      // every split gets at least one tile
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    float* part_o = static_cast<float*>(ws);
    float* part_ml = part_o ? part_o + (size_t)n_used * rows * hidden : nullptr;
    hipLaunchKernelGGL((attn_bf16_kernel<D, QB>), dim3((unsigned)(wg * n_used)), dim3(256), 0, s,
                       static_cast<const bf16*>(q), ldq, static_cast<const bf16*>(k), ldk,
                       static_cast<const bf16*>(v), hidden, seq_kv, rows, n_qtiles, n_used, tps,
                       static_cast<bf16*>(o), ldo, part_o, part_ml, scale_log2);
    if (n_used > 1) {
      const int64_t units = rows * heads * (D / 8);
      hipLaunchKernelGGL(attn_combine_kernel<D>, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s, part_o,
                         part_ml, n_used, rows, heads, static_cast<bf16*>(o), ldo);
    }
  } else {
    const int n_qtiles = (int)((rows + 63) / 64);
    hipLaunchKernelGGL(attn_f32_kernel<D>, dim3((unsigned)(n_qtiles * heads)), dim3(64), 0, s,
                       static_cast<const float*>(q), ldq, static_cast<const float*>(k), ldk,
                       static_cast<const float*>(v), ldv, seq_kv, rows, n_qtiles, static_cast<float*>(o), ldo,
                       1.0f / sqrtf((float)D));
  }
  return hipGetLastError();
}

size_t attention_workspace_bytes(int64_t rows, int64_t hidden, int heads, int n_split) {
  if (n_split <= 1) return 0;
  return sizeof(float) * ((size_t)n_split * rows * hidden + 2 * (size_t)n_split * rows * heads);
}

hipError_t launch_attention(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v, int64_t ldv,
                            int v_layout, int64_t hidden, int64_t seq_kv, int64_t rows, int heads, int head_dim,
                            void* o, int64_t ldo, int dtype, void* ws, size_t ws_bytes, hipStream_t s) {
  (void)v_layout;
  if (rows <= 0) return hipSuccess;
  switch (head_dim) {
    case 64: return launch_attn_d<64>(q, ldq, k, ldk, v, ldv, hidden, seq_kv, rows, heads, o, ldo, dtype, ws, ws_bytes, s);
    case 72: return launch_attn_d<72>(q, ldq, k, ldk, v, ldv, hidden, seq_kv, rows, heads, o, ldo, dtype, ws, ws_bytes, s);
    default: return launch_attn_d<128>(q, ldq, k, ldk, v, ldv, hidden, seq_kv, rows, heads, o, ldo, dtype, ws, ws_bytes, s);
  }
}

}  // namespace pf
