// Patch attention: the queries of one patch attend over every row of a layer's
// full-spatial K/V buffer (PipeFusion keeps full attention; the buffer mixes fresh and
// stale rows).  Flash-style single pass with online softmax; no score matrix is stored.
//
// bf16 kernel (head_dim D in {64, 72, 128}), gfx950 MFMA v_mfma_f32_32x32x16_bf16:
//   * workgroup = 8 wavefronts in two groups of four; wavefronts w and w + 4 share a SIMD.
//     Each wavefront owns QB blocks of 32 queries of one head, so every K/V operand read
//     from LDS feeds QB MFMAs.  The groups run one phase apart between workgroup barriers
//     ("ping-pong"): while one wavefront of a SIMD issues its MFMAs (P.V of the previous
//     key tile and the scores of the current one) the other runs its softmax on the VALU,
//     so the matrix cores and the vector ALUs of every SIMD work at the same time.
//   * key tiles of 32 rows are copied global -> LDS by the gfx950 direct 16-byte loads (no
//     register staging) into a 5-stage ring, three tiles ahead; the loads are counted with
//     explicit vmcnt waits, so they stay in flight across barriers.  K keeps its rows in a
//     permuted, swizzled unit order (conflict-free operand reads), V the K8 layout of the
//     buffer (see pf.h).  The V operands of a tile are read into registers at the end of
//     its softmax phase, so the next MFMA phase starts without waiting on LDS.
//   * scores are computed transposed, S^T = K . Q^T, so each lane owns one query and 16
//     keys per block: the row max is a lane-local max chain plus one exchange with the
//     lane 32 away, and the row sum stays lane-local until the end.
//   * the K rows feeding the score MFMA are permuted (bits 2 and 3 of the row index
//     swapped) so that each lane's 8 consecutive score registers are 8 consecutive keys:
//     they pack directly into the bf16 "B" operand of O^T += V^T . P^T without any
//     cross-lane shuffle, and the matching V^T operand is one 16-byte K8 read per lane.
//   * softmax in base 2: p = exp2(s * log2(e)/sqrt(D) - m), fp32 statistics, P rounded to
//     bf16 for the P.V product and the row sum taken over the same rounded values (for
//     D = 72 by the P.V MFMA itself, through a ones row in the padding of O^T).  The
//     reference max m is raised (and O, l rescaled) only when a tile's max exceeds it by
//     more than 8, so p <= 2^8 and the rescale is rare.
//   * D = 72 pads the score contraction to 80 and the output rows to 96 with zero
//     operands; nothing outside the real 72 columns is read or written.
//   * when there are too few (query tile, head) pairs to fill the GPU, the key range is
//     split across workgroups; each writes its slice's normalised result in bf16 with the
//     slice's (m, l), and a combine kernel merges them (a convex combination).
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

// Query blocks of 32 per wavefront (QB) per head_dim; two wavefronts per SIMD cap each at
// 256 registers (head_dim 128 with QB = 2 would spill).
template <int D> struct AttnCfg;
template <> struct AttnCfg<64> { static constexpr int QB = 2; };
template <> struct AttnCfg<72> { static constexpr int QB = 2; };
template <> struct AttnCfg<128> { static constexpr int QB = 1; };
constexpr int kAttnWaves = 8;
constexpr int kAttnStages = 5;

template <int D, int QB>
__global__ __launch_bounds__(512, 1) void attn_bf16_kernel(const bf16* __restrict__ Q, int64_t ldq,
                                                         const bf16* __restrict__ Kb, int64_t ldk,
                                                         const bf16* __restrict__ Vb, int64_t hidden,
                                                         int64_t S, int64_t rows, int n_qtiles, int n_split,
                                                         int tiles_per_split, bf16* __restrict__ O,
                                                         int64_t ldo, bf16* __restrict__ part_o,
                                                         float* __restrict__ part_ml, float scale_log2,
                                                         int64_t grp_rows, int qtiles_per_grp, int64_t kv_stride) {
  constexpr int BQ = kAttnWaves * 32 * QB;
  constexpr int KS = (D + 15) / 16;
  constexpr int DB = (D + 31) / 32;
  constexpr int TK = kTileKeys;
  constexpr int W = D / 8;
  constexpr int KU = TK * W;
  constexpr int KUP = (KU + 63) / 64 * 64;
  constexpr int NI = KUP / 64;
  constexpr int NINST = 2 * NI;
  constexpr int NJ = (NINST + 3) / 4;
  constexpr int NMIN = NINST / 4;
  constexpr int NSTAGE = kAttnStages;
  static_assert(NSTAGE >= 3 && NSTAGE <= 8, "stage ring");
  __shared__ __attribute__((aligned(16))) uint4 lds[NSTAGE][2 * KUP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wavefront-uniform (scalar)
  const int grp = wave >> 2, wl = wave & 3;
  const int l32 = lane & 31, hi = lane >> 5;

  // Samples of a batch: query rows [g * grp_rows, (g+1) * grp_rows) of Q / O and the partials
  // belong to sample g, whose K / V buffers start g * kv_stride elements on; each sample has
  // qtiles_per_grp query tiles (n_qtiles in all).
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int qt_all = lid % n_qtiles;
  const int rest = lid / n_qtiles;
  const int split = rest % n_split;
  const int head = rest / n_split;
  const int grp_id = qt_all / qtiles_per_grp;
  const int qt = qt_all - grp_id * qtiles_per_grp;
  Kb += grp_id * kv_stride;
  Vb += grp_id * kv_stride;
  const int64_t row_base = (int64_t)grp_id * grp_rows;
  const int64_t col0 = (int64_t)head * D;
  const int64_t ntiles = (S + TK - 1) / TK;
  const int64_t t_begin = (int64_t)split * tiles_per_split;
  const int64_t t_end = t_begin + tiles_per_split < ntiles ? t_begin + tiles_per_split : ntiles;

  int64_t q_row[QB];   // row of Q / O / the partials
  bool q_ok[QB];       // inside this sample's rows
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int64_t local = (int64_t)qt * BQ + (wave * QB + qb) * 32 + l32;
    q_ok[qb] = local < grp_rows;
    q_row[qb] = row_base + local;
  }

  bf16x8 qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = ks * 16 + hi * 8;
      if (q_ok[qb] && d0 < D) {
        qf[qb][ks] = *reinterpret_cast<const bf16x8*>(Q + q_row[qb] * ldq + col0 + d0);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[qb][ks][e] = (bf16)0.f;
      }
    }
  // Q has landed before the first direct load is issued: from here on every outstanding
  // global load is a tile load, counted by the explicit waits below.
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));

  f32x16 o[QB][DB];
  float m_ref[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    l_run[qb] = 0.f;
    m_ref[qb] = -INFINITY;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[qb][db][e] = 0.f;
  }

  const int64_t ngroups = (S + 7) >> 3;
  auto k_unit = [](int p, int c) -> int {
    if constexpr (W % 2 == 1) return p * W + c;
    else if constexpr (W == 8) return p * 8 + (c ^ (p & 7));
    else return p * 16 + (c ^ (p & 15));
  };

  // Lane l of load i (i = wl + 4j, this wavefront's j-th) fills unit 64(i mod NI) + l of the
  // K part (i < NI) or the V part.  Lanes past the part's KU real units fill padding units
  // that nothing reads, from the part's unit 0 (a valid address), so no lane is masked off.
  uint32_t ld_off[NJ];
  int ld_row[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int i = wl + 4 * j;
    const bool kpart = i < NI;
    int u = (kpart ? i : i - NI) * 64 + lane;
    if (u >= KU) u = 0;
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
  // Tile t into stage st (group 0 only).  Only the buffer's last tile can run past S: its rows
  // (K8 groups) past the end read the last valid row (group) instead; their scores are masked
  // and their V entries zeroed before use.
  auto issue_tile = [&](int64_t t, int st) {
    const char* kbase = reinterpret_cast<const char*>(Kb + (t * TK) * ldk + col0);
    const char* vbase = reinterpret_cast<const char*>(Vb + (t * (TK / 8) * hidden + col0) * 8);
    if ((t + 1) * TK <= S) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int i = wl + 4 * j;
        if (i >= NINST) continue;                   // wavefront-uniform
        const bool kpart = i < NI;
        dma_load16(kpart ? kbase : vbase, ld_off[j], &lds[st][(kpart ? i : KUP / 64 + i - NI) * 64]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int i = wl + 4 * j;
        if (i >= NINST) continue;
        const bool kpart = i < NI;
        uint32_t off = ld_off[j];
        if (kpart) {
          const int64_t over = t * TK + ld_row[j] - (S - 1);
          if (over > 0) off -= (uint32_t)(over * ldk * 2);
        } else {
          const int64_t over = t * (TK / 8) + ld_row[j] - (ngroups - 1);
          if (over > 0) off -= (uint32_t)(over * hidden * 16);
        }
        dma_load16(kpart ? kbase : vbase, off, &lds[st][(kpart ? i : KUP / 64 + i - NI) * 64]);
      }
    }
  };
  auto wait_loads = [&](int newer_tiles) {
    if (newer_tiles >= 3) __builtin_amdgcn_s_waitcnt(((3 * NMIN) & 15) | (((3 * NMIN) >> 4) << 14) | (7 << 4) | (15 << 8));
    else if (newer_tiles == 2) __builtin_amdgcn_s_waitcnt(((2 * NMIN) & 15) | (((2 * NMIN) >> 4) << 14) | (7 << 4) | (15 << 8));
    else if (newer_tiles == 1) __builtin_amdgcn_s_waitcnt((NMIN & 15) | ((NMIN >> 4) << 14) | (7 << 4) | (15 << 8));
    else __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
  };
  auto barrier = [] {
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // K_t operands of S^T = K_t . Q^T (lane: key row l32, 8 consecutive d).  Rows of the
  // padded k-step past D read a valid LDS unit and are zeroed by a select (no branch).
  auto read_k = [&](int st, bf16x8 (&kf)[KS]) {
    const uint4* base = lds[st];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = ks * 16 + hi * 8;
      if constexpr (KS * 16 > D) {
        if (ks == KS - 1) {
          const int c = d0 < D ? 2 * ks + hi : 2 * ks;
          const u32x4 w = *reinterpret_cast<const u32x4*>(&base[k_unit(l32, c)]);
          const u32x4 z = {0u, 0u, 0u, 0u};
          kf[ks] = __builtin_bit_cast(bf16x8, d0 < D ? w : z);
          continue;
        }
      }
      kf[ks] = *reinterpret_cast<const bf16x8*>(&base[k_unit(l32, 2 * ks + hi)]);
    }
  };
  auto scores = [&](const bf16x8 (&kf)[KS], f32x16 (&sc)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[qb][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[qb][ks], sc[qb], 0, 0, 0);
  };
  auto mask_scores = [&](int64_t t, f32x16 (&sc)[QB]) {
    const int lim = (int)(S - t * TK);
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
  constexpr bool kSumRow = D % 32 != 0;
  constexpr int kSumIdx = 4 * ((D % 32) / 8) + 0;
  // V_t^T operands of O^T += V_t^T . P^T (lane: row d = db*32 + l32, 8 keys of group 2*h2 + hi);
  // rows past D are zero, or ones in row D for the MFMA row sum; `zero_tail` zeroes keys past S
  auto read_v = [&](int64_t t, int st, bf16x8 (&vf)[2][DB], bool zero_tail) {
    const uint4* base = lds[st] + KUP;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int grp8 = 2 * h2 + hi;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = db * 32 + l32;
        if (db * 32 + 32 <= D) {
          vf[h2][db] = *reinterpret_cast<const bf16x8*>(&base[grp8 * D + d]);
        } else {
          // rows past D: zero, or ones in row D (MFMA row sum); selected without a branch
          const u32x4 w = *reinterpret_cast<const u32x4*>(&base[grp8 * D + (d < D ? d : D - 1)]);
          const uint32_t f = (kSumRow && d == D) ? 0x3f803f80u : 0u;   // bf16 pair (1, 1) or (0, 0)
          const u32x4 fv = {f, f, f, f};
          vf[h2][db] = __builtin_bit_cast(bf16x8, d < D ? w : fv);
        }
        if (zero_tail) {
          const int lim = (int)(S - t * TK) - grp8 * 8;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e >= lim && db * 32 + l32 < D) vf[h2][db][e] = (bf16)0.f;
        }
      }
    }
  };
  auto pv = [&](const bf16x8 (&vf)[2][DB], const bf16x8 (&pb)[QB][2]) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[h2][db], pb[qb][h2], o[qb][db], 0, 0, 0);
  };
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
  // tile max (3-input maximum tree; the two 32-lane halves hold the same queries' other keys),
  // lazy rescale, p = 2^(s*c - m) packed to bf16
  auto softmax = [&](f32x16 (&sc)[QB], bf16x8 (&pc)[QB][2]) {
    float mt[QB];
    bool raise = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      auto mx3 = [](float a, float b, float c) {
        return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
      };
      const float m0 = mx3(sc[qb][0], sc[qb][1], sc[qb][2]);
      const float m1 = mx3(sc[qb][3], sc[qb][4], sc[qb][5]);
      const float m2 = mx3(sc[qb][6], sc[qb][7], sc[qb][8]);
      const float m3 = mx3(sc[qb][9], sc[qb][10], sc[qb][11]);
      const float m4 = mx3(sc[qb][12], sc[qb][13], sc[qb][14]);
      const float m5 = mx3(m0, m1, sc[qb][15]);
      const float mh = mx3(m2, m3, mx3(m4, m5, m5));
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mh), __float_as_uint(mh), false, false);
      const float mx = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      mt[qb] = mx * scale_log2;
      raise |= mt[qb] > m_ref[qb] + 8.0f;
    }
    if (__any(raise)) {
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

  // Slots between barriers: group 0 runs the MFMA phase of tile t in slot 2(t - t_begin) and
  // its softmax in the next slot; group 1 runs the same one slot later.  MFMA phase of t:
  // P.V of tile t-1 (V operands already in registers) and the scores of tile t.  Softmax
  // phase of t: P_t, then the V_t operands are read for the next MFMA phase.  Tile t sits in
  // stage (t - t_begin) mod NSTAGE and is last read by group 1 in slot 2(t - t_begin) + 2,
  // so group 0 issues tile t + NSTAGE - 2 at the start of its slot 2(t - t_begin), into
  // the stage tile t - 2 used.
  const int64_t nt = t_end - t_begin;
  if (grp == 0) {
    for (int64_t u = 0; u < nt && u < NSTAGE - 2; ++u) issue_tile(t_begin + u, (int)u);
    const int64_t newer = (nt < NSTAGE - 2 ? nt : NSTAGE - 2) - 1;
    wait_loads((int)newer);
  }
  barrier();
  if (grp == 1) barrier();

  // P.V of "tile t_begin - 1" multiplies zero weights, so every MFMA phase has the same shape
  bf16x8 pb[QB][2];
  bf16x8 vf[2][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int e = 0; e < 8; ++e) pb[qb][0][e] = pb[qb][1][e] = (bf16)0.f;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 8; ++e) vf[0][db][e] = vf[1][db][e] = (bf16)0.f;
  int st = 0;                         // stage of tile t
  int st_issue = NSTAGE - 2;          // stage of tile t + NSTAGE - 2
  auto iter = [&](int64_t t, bool partial) {
    bf16x8 kf[KS];
    read_k(st, kf);
    f32x16 sc[QB];
    pv(vf, pb);
    if (grp == 0 && t + NSTAGE - 2 < t_end) issue_tile(t + NSTAGE - 2, st_issue);
    scores(kf, sc);
    barrier();
    if (partial) mask_scores(t, sc);
    softmax(sc, pb);
    read_v(t, st, vf, partial);
    if (grp == 0) {
      const int64_t last_issued = t + NSTAGE - 2 < t_end - 1 ? t + NSTAGE - 2 : t_end - 1;
      const int64_t newer = last_issued - (t + 1);
      wait_loads((int)(newer < 0 ? 0 : newer));
    }
    barrier();
    st = st + 1 == NSTAGE ? 0 : st + 1;
    st_issue = st_issue + 1 == NSTAGE ? 0 : st_issue + 1;
  };
  const int64_t t_full = t_end * TK > S ? t_end - 1 : t_end;
  for (int64_t t = t_begin; t < t_full; ++t) iter(t, false);
  if (t_full < t_end) iter(t_full, true);
  if (nt > 0) pv(vf, pb);
  if (grp == 0) barrier();

  if constexpr (kSumRow) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float sum_row = o[qb][DB - 1][kSumIdx];
      l_run[qb] = hi == 0 ? sum_row : 0.f;
    }
  }

#pragma unroll
  // Whole key range: O = acc / l in bf16.  One slice of a split range: the slice's own
  // normalised result acc_s / l_s, also in bf16, plus (m_s, l_s) for the merge.
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32, 64);
    if (!q_ok[qb]) continue;
    const float inv = 1.0f / l_tot;
    bf16* dst = n_split == 1 ? O + q_row[qb] * ldo + col0 : part_o + ((int64_t)split * rows + q_row[qb]) * hidden + col0;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + 8 * g + 4 * hi;
        if (d < D) {
          bf16x4 ov = {(bf16)(o[qb][db][4 * g + 0] * inv), (bf16)(o[qb][db][4 * g + 1] * inv),
                       (bf16)(o[qb][db][4 * g + 2] * inv), (bf16)(o[qb][db][4 * g + 3] * inv)};
          *reinterpret_cast<bf16x4*>(dst + d) = ov;
        }
      }
    if (n_split > 1) {
      if (hi == 0) {
        const int64_t H = hidden / D;
        reinterpret_cast<float2*>(part_ml)[((int64_t)split * H + head) * rows + q_row[qb]] =
            make_float2(m_ref[qb], l_tot);
      }
    }
  }
}

// Merge the per-split partial results.  Slice s holds x_s = acc_s / l_s (bf16) with its
// reference max m_s and weight sum l_s, so O = sum_s w_s x_s / sum_s w_s with
// w_s = 2^(m_s - M) l_s (M = max_s m_s): a convex combination of the slices' results.
// One thread per (row, head, 8 columns).  The loop over slices is unrolled to the largest
// split count (indices past n_split clamped, their terms skipped), so every load of a thread
// is issued before the first is used.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(const bf16* __restrict__ part_o,
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
  float m[kMaxAttnSplit], l[kMaxAttnSplit];
  bf16x8 x[kMaxAttnSplit];
#pragma unroll
  for (int sp = 0; sp < kMaxAttnSplit; ++sp) {
    const int64_t sc = sp < n_split ? sp : n_split - 1;   // slices past n_split re-read the last (unused)
    const float2 ml = reinterpret_cast<const float2*>(part_ml)[(sc * H + head) * rows + row];
    m[sp] = ml.x;
    l[sp] = ml.y;
    x[sp] = *reinterpret_cast<const bf16x8*>(part_o + (sc * rows + row) * hidden + (int64_t)head * D + chunk * 8);
  }
  float M = m[0];
#pragma unroll
  for (int sp = 1; sp < kMaxAttnSplit; ++sp)
    if (sp < n_split) M = fmaxf(M, m[sp]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
#pragma unroll
  for (int sp = 0; sp < kMaxAttnSplit; ++sp) {
    if (sp < n_split) {
      const float w = __builtin_amdgcn_exp2f(m[sp] - M) * l[sp];
      wsum += w;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, (float)x[sp][e], acc[e]);
    }
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
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_bf16_kernel<D, AttnCfg<D>::QB>, 64 * kAttnWaves,
                                                     0) != hipSuccess || per_cu <= 0)
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

// `rows` query rows per sample, `batch` samples: sample b's query rows are rows b*rows ..
// of Q and O, its K / V buffers start b * kv_stride elements after sample 0's.
template <int D>
static hipError_t launch_attn_d(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v, int64_t ldv,
                                int64_t hidden, int64_t seq_kv, int64_t rows, int heads, void* o, int64_t ldo,
                                int dtype, void* ws, size_t ws_bytes, hipStream_t s, int64_t batch,
                                int64_t kv_stride) {
  if (dtype == kDtypeBF16) {
    constexpr int QB = AttnCfg<D>::QB;
    constexpr int BQ = kAttnWaves * 32 * QB;
    const int64_t all_rows = batch * rows;
    const int per_grp = (int)((rows + BQ - 1) / BQ);
    const int n_qtiles = (int)(batch * per_grp);
    const int64_t ntiles = (seq_kv + kTileKeys - 1) / kTileKeys;
    const int64_t wg = (int64_t)n_qtiles * heads;
    const int n_split = ws ? choose_split(wg, attn_slots<D>(), ntiles, all_rows, hidden, heads, ws_bytes) : 1;
    const int tps = (int)((ntiles + n_split - 1) / n_split);
    const int n_used = (int)((ntiles + tps - 1) / tps);      // every split gets at least one tile
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    // workspace: bf16 slice results [n_used][all_rows][hidden], then fp32 (m, l) pairs [n_used][heads][all_rows]
    bf16* part_o = static_cast<bf16*>(ws);
    float* part_ml = part_o ? reinterpret_cast<float*>(part_o + (size_t)n_used * all_rows * hidden) : nullptr;
    hipLaunchKernelGGL((attn_bf16_kernel<D, QB>), dim3((unsigned)(wg * n_used)), dim3(64 * kAttnWaves), 0, s,
                       static_cast<const bf16*>(q), ldq, static_cast<const bf16*>(k), ldk,
                       static_cast<const bf16*>(v), hidden, seq_kv, all_rows, n_qtiles, n_used, tps,
                       static_cast<bf16*>(o), ldo, part_o, part_ml, scale_log2, rows, per_grp, kv_stride);
    if (n_used > 1) {
      const int64_t units = all_rows * heads * (D / 8);
      hipLaunchKernelGGL(attn_combine_kernel<D>, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s, part_o,
                         part_ml, n_used, all_rows, heads, static_cast<bf16*>(o), ldo);
    }
  } else {
    const int n_qtiles = (int)((rows + 63) / 64);
    for (int64_t b = 0; b < batch; ++b)
      hipLaunchKernelGGL(attn_f32_kernel<D>, dim3((unsigned)(n_qtiles * heads)), dim3(64), 0, s,
                         static_cast<const float*>(q) + b * rows * ldq, ldq, static_cast<const float*>(k) + b * kv_stride,
                         ldk, static_cast<const float*>(v) + b * kv_stride, ldv, seq_kv, rows, n_qtiles,
                         static_cast<float*>(o) + b * rows * ldo, ldo, 1.0f / sqrtf((float)D));
  }
  return hipGetLastError();
}

size_t attention_workspace_bytes(int64_t rows, int64_t hidden, int heads, int n_split) {
  if (n_split <= 1) return 0;
  return sizeof(bf16) * (size_t)n_split * rows * hidden + sizeof(float) * 2 * (size_t)n_split * rows * heads;
}

hipError_t launch_attention(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v, int64_t ldv,
                            int v_layout, int64_t hidden, int64_t seq_kv, int64_t rows, int heads, int head_dim,
                            void* o, int64_t ldo, int dtype, void* ws, size_t ws_bytes, hipStream_t s,
                            int64_t batch, int64_t kv_stride) {
  (void)v_layout;
  if (rows <= 0 || batch <= 0) return hipSuccess;
  switch (head_dim) {
    case 64:
      return launch_attn_d<64>(q, ldq, k, ldk, v, ldv, hidden, seq_kv, rows, heads, o, ldo, dtype, ws, ws_bytes, s,
                               batch, kv_stride);
    case 72:
      return launch_attn_d<72>(q, ldq, k, ldk, v, ldv, hidden, seq_kv, rows, heads, o, ldo, dtype, ws, ws_bytes, s,
                               batch, kv_stride);
    default:
      return launch_attn_d<128>(q, ldq, k, ldk, v, ldv, hidden, seq_kv, rows, heads, o, ldo, dtype, ws, ws_bytes, s,
                                batch, kv_stride);
  }
}

}  // namespace pf
