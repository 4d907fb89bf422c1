// Patch attention: the queries of one patch attend over every row of a layer's
// full-spatial K/V buffer (PipeFusion keeps full attention; the buffer mixes fresh and
// stale rows).  Flash-style single pass with online softmax; no score matrix is stored.
//
// bf16 kernel (head_dim D in {64, 72, 128}), gfx950 MFMA v_mfma_f32_32x32x16_bf16:
//   * workgroup = 8 wavefronts in two groups of four; wavefronts w and w + 4 share a SIMD.
//     Each wavefront owns QB blocks of 32 queries of one head, so every K/V operand read
//     from LDS feeds QB MFMAs.  The groups run one phase apart ("ping-pong"): while one
//     wavefront of a SIMD issues its MFMAs (P.V of the previous key tile and the scores of
//     the current one) the other runs its softmax on the VALU, so the matrix cores and the
//     vector ALUs of every SIMD work at the same time.  The phases are held apart by a
//     workgroup barrier after every phase, or (stream-K and D = 72) by one barrier per key
//     tile that falls after the MFMA phase in group 1 and after the softmax in group 0.
//   * key tiles of 32 rows are copied global -> LDS by the gfx950 direct 16-byte loads (no
//     register staging) into a 5-stage ring, three tiles ahead; the loads are counted with
//     explicit vmcnt waits, so they stay in flight across barriers.  K keeps its rows in a
//     permuted, swizzled unit order (conflict-free operand reads), V the K8 layout of the
//     buffer (see pf.h).  The V operands of a tile are read into registers one phase before
//     the P.V MFMAs that use them (in the MFMA phase at D = 64 and in the single-piece D = 72
//     kernel, in the softmax phase otherwise), so no MFMA phase starts by waiting on LDS.
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
//     reference m is an integer, raised (and O, l rescaled) only when a tile holds a score
//     more than 64 above it, so p < 2^64, far from fp32 overflow, and the rescale is rare;
//     the common path takes no row max (a lane-local sum or max test instead).  Because m is
//     an integer, every rescale multiplies by an exact power of two, and the rounded weights
//     are those of bf16(2^(s log2(e)/sqrt(D))) scaled by 2^-m: the same values whatever the
//     order of the key tiles, the split of the key range or the running max at the time a
//     tile is seen.
//   * D = 72 pads the score contraction to 80 and the output rows to 96 with zero
//     operands; nothing outside the real 72 columns is read or written.
//   * when there are too few (query tile, head) pairs to fill the GPU, the key range is
//     cut into pieces run by different workgroups: either a fixed split of every head's key
//     range, or (one patch of a large stage: a few query tiles, many heads) a grouped stream-K
//     schedule, where one group of workgroups per query-tile set takes an equal stretch of the
//     (head, key tile) line, so every CU gets the same number of key tiles in one round.  A
//     piece short of a whole key range writes its normalised result in fp32 with its (m, l),
//     and a combine kernel merges them (a convex combination with power-of-two weights times
//     l, so the merge adds only fp32 rounding to the unsplit result).
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

// SK: the grouped stream-K schedule (a workgroup may run several pieces); otherwise every
// workgroup runs exactly one piece and the kernel has no piece loop.
template <int D, int QB, bool SK>
__global__ __launch_bounds__(512, 1) void attn_bf16_kernel(const bf16* __restrict__ Q, int64_t ldq,
                                                         const bf16* __restrict__ Kb, int64_t ldk,
                                                         const bf16* __restrict__ Vb, int64_t hidden,
                                                         int64_t S, int64_t rows, int n_qtiles, int n_split,
                                                         int tiles_per_split, int64_t group_tiles,
                                                         bf16* __restrict__ O,
                                                         int64_t ldo, float* __restrict__ part_o,
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

  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);   // wavefront-uniform (scalar)
  const int grp = wave >> 2, wl = wave & 3;

  // Samples of a batch: query rows [g * grp_rows, (g+1) * grp_rows) of Q / O and the partials
  // belong to sample g, whose K / V buffers start g * kv_stride elements on; each sample has
  // qtiles_per_grp query tiles (n_qtiles in all).
  // Work of the launch: for every query tile, the key tiles of every head in the order
  // (head, key tile), a line of H * ntiles tiles.  Workgroup (query tile qt_all, index gi) takes
  // one stretch of that line:
  //   * fixed split (group_tiles == 0): gi = split + n_split * head, key tiles
  //     [split * tiles_per_split, +tiles_per_split) of that head;
  //   * grouped stream-K (group_tiles > 0): gi is a group of n_qtiles workgroups, one per
  //     query tile, that all take line positions [gi * group_tiles, +group_tiles): the same
  //     key tiles at the same time (shared in L2), and a stretch may run over several heads.
  // Each head met by a stretch is one piece.  A piece covering all of a head's key tiles writes
  // O directly; any other piece writes its normalised fp32 result and (m, l) into partial slot
  // split * H + head (fixed split) or head + gi (stream-K), merged by attn_combine_kernel.  The
  // fp32 results of the fixed split lie as [split][row][hidden] (a row's heads side by side, as
  // the merge reads them), those of stream-K as [slot][row][D].
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int qt_all = lid % n_qtiles;
  const int gi = lid / n_qtiles;
  const int grp_id = qt_all / qtiles_per_grp;
  const int qt = qt_all - grp_id * qtiles_per_grp;
  Kb += grp_id * kv_stride;
  Vb += grp_id * kv_stride;
  const int64_t row_base = (int64_t)grp_id * grp_rows;
  const int64_t ntiles = (S + TK - 1) / TK;
  const int64_t H = hidden / D;
  int64_t pos, pos_end;
  if (group_tiles > 0) {
    pos = (int64_t)gi * group_tiles;
    pos_end = pos + group_tiles < H * ntiles ? pos + group_tiles : H * ntiles;
  } else {
    const int split = gi % n_split, head0 = gi / n_split;
    pos = head0 * ntiles + (int64_t)split * tiles_per_split;
    pos_end = pos + tiles_per_split < (head0 + 1) * ntiles ? pos + tiles_per_split : (head0 + 1) * ntiles;
  }

  auto barrier_all = [] {
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  for (bool first = true; pos < pos_end; first = false) {
    const int64_t head = pos / ntiles;
    const int64_t t_begin = pos - head * ntiles;
    const int64_t t_end = t_begin + (pos_end - pos) < ntiles ? t_begin + (pos_end - pos) : ntiles;
    pos += t_end - t_begin;
    const bool whole = t_begin == 0 && t_end == ntiles;
    const int64_t slot = group_tiles > 0 ? head + gi : (int64_t)(gi % n_split) * H + head;
    const int64_t col0 = head * D;
    // a later piece reuses the LDS ring: every wavefront is past its last read of the previous one
    if (!first) barrier_all();
    // With several pieces at head_dim 72, lane-dependent values are derived anew in every piece
    // from a copy of the thread id the compiler cannot see through, so none of them is hoisted
    // out of the piece loop and kept live across the key loop: hoisted, they push that kernel
    // past 256 registers (spills).  At 64 and 128 the hoisted form fits and measured faster.
    int tid = (int)threadIdx.x;
    if constexpr (SK && D == 72) asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int l32 = lane & 31, hi = lane >> 5;
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
    // LDS unit of K row p, 16-byte chunk c.  An operand read of 16 consecutive rows at one chunk
    // must hit 16 distinct 16-byte bank groups (a b128 read is served 16 lanes at a time): odd
    // W strides rows apart by itself, W = 16 XORs the chunk with p mod 16, and W = 8 (two rows
    // per 16 units) with p / 2 mod 8 (p mod 8 left rows p and p + 8 on the same banks: measured
    // SQ_LDS_BANK_CONFLICT 2 cycles per LDS instruction, 3% of the time at 16384 x 16384 keys).
    auto k_unit = [](int p, int c) -> int {
      if constexpr (W % 2 == 1) return p * W + c;
      else if constexpr (W == 8) return p * 8 + (c ^ ((p >> 1) & 7));
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
          c = (u & 7) ^ ((p >> 1) & 7);
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
    auto issue_tile_full = [&](int64_t t, int st) {
      const char* kbase = reinterpret_cast<const char*>(Kb + (t * TK) * ldk + col0);
      const char* vbase = reinterpret_cast<const char*>(Vb + (t * (TK / 8) * hidden + col0) * 8);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int i = wl + 4 * j;
        if (i >= NINST) continue;                   // wavefront-uniform
        const bool kpart = i < NI;
        dma_load16(kpart ? kbase : vbase, ld_off[j], &lds[st][(kpart ? i : KUP / 64 + i - NI) * 64]);
      }
    };
    // NSTAGE - 3 newer tiles in flight (the steady state)
    auto wait_loads_const = [&] {
      constexpr int n = (NSTAGE - 3) * NMIN;
      __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
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

    // K_t operands of S^T = K_t . Q^T (lane: key row l32, 8 consecutive d).  In the padded
    // k-step (D = 72: d 64..79) only the lanes of real columns read LDS, into a register that
    // lives across the key loop; the other lanes never write it and keep its zeros (an
    // exec-masked read of half the lanes; reading a valid unit in every lane and selecting
    // zero measured 2.5% slower at 16384 x 262144 keys, 16 heads).
    bf16x8 kpad;
#pragma unroll
    for (int e = 0; e < 8; ++e) kpad[e] = (bf16)0.f;
    auto read_k = [&](int st, bf16x8 (&kf)[KS]) {
      const uint4* base = lds[st];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int d0 = ks * 16 + hi * 8;
        if constexpr (KS * 16 > D) {
          if (ks == KS - 1) {
            if (d0 < D) kpad = *reinterpret_cast<const bf16x8*>(&base[k_unit(l32, 2 * ks + hi)]);
            kf[ks] = kpad;
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
            // rows past D: only lanes of real rows read LDS (reading a valid unit in every lane and
            // selecting measured 3% slower at D = 72); the others keep the zeros, or the ones of row
            // D (MFMA row sum), they were given before the key loop
            if (d < D) vf[h2][db] = *reinterpret_cast<const bf16x8*>(&base[grp8 * D + d]);
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
    // p = 2^(s c - m) packed to bf16 for every score of the tile; the reference m of a query is an
    // integer, raised only when the tile holds a score more than kRaise above it (so p < 2^kRaise
    // and sums stay far from fp32 overflow).  Common path without a row max: for D = 64 / 128 the
    // lane's partial sum of the tile's rounded weights (needed for l anyway) exceeds 2^kRaise
    // whenever a weight does (the first tile, where m = -inf, gives inf); for D = 72 (the row sum
    // comes from the P.V MFMA) a lane-local maximum of the raw scores is compared with the
    // threshold.  Only then (rare after the first tile) does the wave take the row max across
    // both halves of the query's keys, raise m to its ceiling and rescale O and l by the exact
    // power of two 2^(m_old - m_new), and recompute the tile's weights.
    constexpr float kRaise = 64.0f;
    auto exp_pack = [&](f32x16 (&sc)[QB], bf16x8 (&pc)[QB][2], float (&lt)[QB]) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        uint32_t pk[8];
        lt[qb] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const f32x2 pp = {__builtin_amdgcn_exp2f(fmaf(sc[qb][2 * e], scale_log2, -m_ref[qb])),
                            __builtin_amdgcn_exp2f(fmaf(sc[qb][2 * e + 1], scale_log2, -m_ref[qb]))};
          const bf16x2 pb2 = __builtin_convertvector(pp, bf16x2);
          if constexpr (!kSumRow) lt[qb] = __builtin_amdgcn_fdot2_f32_bf16(pb2, ones, lt[qb], false);
          pk[e] = __builtin_bit_cast(uint32_t, pb2);
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const u32x4 w = {pk[4 * h2], pk[4 * h2 + 1], pk[4 * h2 + 2], pk[4 * h2 + 3]};
          pc[qb][h2] = __builtin_bit_cast(bf16x8, w);
        }
      }
    };
    auto mx3 = [](float a, float b, float c) {
      return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
    };
    auto lane_max = [&](const f32x16& v) {
      const float m0 = mx3(v[0], v[1], v[2]);
      const float m1 = mx3(v[3], v[4], v[5]);
      const float m2 = mx3(v[6], v[7], v[8]);
      const float m3 = mx3(v[9], v[10], v[11]);
      const float m4 = mx3(v[12], v[13], v[14]);
      const float m5 = mx3(m0, m1, v[15]);
      return mx3(m2, m3, mx3(m4, m5, m5));
    };
    auto softmax = [&](f32x16 (&sc)[QB], bf16x8 (&pc)[QB][2]) {
      float lt[QB];
      bool raise = false;
      if constexpr (kSumRow) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) raise |= lane_max(sc[qb]) * scale_log2 > m_ref[qb] + kRaise;
      }
      if (!kSumRow || !__any(raise)) {
        exp_pack(sc, pc, lt);
        if constexpr (!kSumRow) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) raise |= !(lt[qb] <= 0x1p64f);   // also true for inf / nan
        }
      }
      if (__any(raise)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float mh = lane_max(sc[qb]);
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mh), __float_as_uint(mh), false, false);
          const float mt = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale_log2;
          // integer reference: alpha is an exact power of two (0 on the first tile)
          const float m_new = fmaxf(m_ref[qb], __builtin_ceilf(mt));
          const float alpha = __builtin_amdgcn_exp2f(m_ref[qb] - m_new);
          m_ref[qb] = m_new;
          l_run[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[qb][db][e] *= alpha;
        }
        exp_pack(sc, pc, lt);
      }
      if constexpr (!kSumRow) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) l_run[qb] += lt[qb];
      }
    };

    // MFMA phase of tile t: P.V of tile t-1 (V operands already in registers) and the scores
    // of tile t.  Softmax phase of t: P_t (and, where the V operands are not read in the MFMA
    // phase, the V_t operands for the next one).  Tile t sits in stage (t - t_begin) mod NSTAGE.
    //   * Two barriers per tile: group 0 runs the MFMA phase of t in slot 2(t - t_begin) and its
    //     softmax in the next slot; group 1 runs the same one slot later (one extra barrier at
    //     the start, matched by group 0 at the end).  Tile t is last read by group 1 in slot
    //     2(t - t_begin) + 2, so group 0 issues tile t + NSTAGE - 2 at the start of its slot
    //     2(t - t_begin), into the stage tile t - 2 used.
    //   * One barrier per tile (kOneBarrier): between barriers t-1 and t group 0 runs the MFMA
    //     phase of t, then its softmax; group 1 the softmax of t-1, then the MFMA phase of t.
    //     Tile t is last read by group 1 before barrier t+1 (its V operands, where they are read
    //     in the softmax phase).  Group 0 issues tile t + NSTAGE - 2 between barriers t-1 and t,
    //     into the stage of tile t - 2, so tile t's stage is written again only after barrier
    //     t+1.  Tile t+1 has landed (group 0 waits for it before barrier t) and barrier t
    //     publishes it before either group reads it.  Measured against two barriers:
    //     -2% for the stream-K launches of 2048 x 16384 keys (24 heads, d = 64) and 2048 x
    //     16896 (d = 128), -1.5% for the split launch of 1024 x 4096 (d = 72), the same at
    //     16384 x 262144 (d = 72); 2% slower for whole-head launches at d = 64 and no faster at
    //     d = 128, hence not for those.
    const int64_t nt = t_end - t_begin;
    constexpr bool kOneBarrier = SK || D == 72;
    if (grp == 0) {
      for (int64_t u = 0; u < nt && u < NSTAGE - 2; ++u) issue_tile(t_begin + u, (int)u);
      const int64_t newer = (nt < NSTAGE - 2 ? nt : NSTAGE - 2) - 1;
      wait_loads((int)newer);
    }
    barrier();
    if (!kOneBarrier && grp == 1) barrier();

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
    if constexpr (DB * 32 > D) {
      // rows past D of the padded V^T block keep their values: zero, or ones in row D (MFMA row sum)
      const int d = (DB - 1) * 32 + l32;
      const uint32_t f = (kSumRow && d == D) ? 0x3f803f80u : 0u;
      const u32x4 w = {f, f, f, f};
      vf[0][DB - 1] = vf[1][DB - 1] = __builtin_bit_cast(bf16x8, w);
    }
    int st = 0;                         // stage of tile t
    int st_issue = NSTAGE - 2;          // stage of tile t + NSTAGE - 2
    auto iter = [&](int64_t t, bool partial) {
      bf16x8 kf[KS];
      read_k(st, kf);
      f32x16 sc[QB];
      pv(vf, pb);
      if (grp == 0 && t + NSTAGE - 2 < t_end) issue_tile(t + NSTAGE - 2, st_issue);
      scores(kf, sc);
      if (!kOneBarrier || grp == 1) barrier();
      if (partial) mask_scores(t, sc);
      softmax(sc, pb);
      read_v(t, st, vf, partial);
      if (grp == 0) {
        const int64_t last_issued = t + NSTAGE - 2 < t_end - 1 ? t + NSTAGE - 2 : t_end - 1;
        const int64_t newer = last_issued - (t + 1);
        wait_loads((int)(newer < 0 ? 0 : newer));
      }
      if (!kOneBarrier || grp == 0) barrier();
      st = st + 1 == NSTAGE ? 0 : st + 1;
      st_issue = st_issue + 1 == NSTAGE ? 0 : st_issue + 1;
    };
    // steady state: the tile NSTAGE - 2 ahead exists and is full, so every wait is the same.  For
    // D = 72 and 128 the wavefront in its MFMA phase runs at a raised priority, so the SIMD's
    // arbiter issues its MFMAs as soon as the matrix core frees up and fills the gaps with the
    // other wavefront's softmax (measured: +5% at 262144 keys, d = 72; at d = 64, where the
    // softmax phase is the longer one, it costs 3%).  In the D = 128 stream-K kernel group 0's
    // MFMA phase runs one level above group 1's: with one barrier per key tile group 1 can enter
    // its MFMA phase while group 0 is still in its own, and equal priorities then share the
    // matrix core between them, which stretches group 0's MFMA phase and pushes its softmax
    // towards the barrier (measured: -1.8% for the 2048 x 16896-key, 24-head stream-K launch; at
    // D = 72 it cost 0.8%)
    constexpr bool kPingPongPrio = D != 64;
    constexpr bool kGroupPrio = D == 128 && kOneBarrier;
    // Where the V operands of tile t are read.  At D = 64 and 72 the wavefront in its MFMA phase
    // reads them right after its P.V MFMAs have consumed the previous tile's: a wavefront then
    // issues its LDS reads next to its MFMAs, not next to its softmax VALU work (measured: -5%
    // time at 16384 x 262144 keys, 16 heads, d = 72; -5% at 16384 x 16384 keys, 24 heads, d = 64;
    // neutral for d = 64 stream-K; in the d = 72 stream-K kernel the extra live registers spill).
    // At D = 128 they go out before the softmax, so their latency hides behind its exponentials
    // (-7% at 2048 x 16896 keys, 24 heads).
    constexpr bool kVInMfmaPhase = (D == 72 && !SK) || D == 64;
    constexpr bool kEarlyV = D == 128;
    auto iter_steady = [&](int64_t t) {
      bf16x8 kf[KS];
      if constexpr (kGroupPrio) {
        if (grp == 0) __builtin_amdgcn_s_setprio(2);
        else __builtin_amdgcn_s_setprio(1);
      } else if constexpr (kPingPongPrio) {
        __builtin_amdgcn_s_setprio(1);
      }
      read_k(st, kf);
      f32x16 sc[QB];
      pv(vf, pb);
      if constexpr (kVInMfmaPhase) read_v(t, st, vf, false);
      if (grp == 0) issue_tile_full(t + NSTAGE - 2, st_issue);
      scores(kf, sc);
      if (!kOneBarrier || grp == 1) barrier();
      if constexpr (kPingPongPrio) __builtin_amdgcn_s_setprio(0);
      if constexpr (kEarlyV) read_v(t, st, vf, false);
      softmax(sc, pb);
      if constexpr (!kEarlyV && !kVInMfmaPhase) read_v(t, st, vf, false);
      if (grp == 0) wait_loads_const();
      if (!kOneBarrier || grp == 0) barrier();
      st = st + 1 == NSTAGE ? 0 : st + 1;
      st_issue = st_issue + 1 == NSTAGE ? 0 : st_issue + 1;
    };
    const int64_t t_full = t_end * TK > S ? t_end - 1 : t_end;
    // the last full tile t can run steady if t + NSTAGE - 2 is a full tile below t_end
    const int64_t t_steady_end = t_full - (NSTAGE - 2) > t_begin ? t_full - (NSTAGE - 2) : t_begin;
    int64_t t = t_begin;
    for (; t < t_steady_end; ++t) iter_steady(t);
    for (; t < t_full; ++t) iter(t, false);
    if (t_full < t_end) iter(t_full, true);
    if (nt > 0) pv(vf, pb);
    if (!kOneBarrier && grp == 0) barrier();

    if constexpr (kSumRow) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float sum_row = o[qb][DB - 1][kSumIdx];
        l_run[qb] = hi == 0 ? sum_row : 0.f;
      }
    }

#pragma unroll
    // Whole key range: O = acc / l in bf16.  One slice of a split range: the slice's own
    // normalised result acc_s / l_s in fp32, plus (m_s, l_s) for the merge.
    for (int qb = 0; qb < QB; ++qb) {
      const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32, 64);
      if (!q_ok[qb]) continue;
      const float inv = 1.0f / l_tot;
      if (whole) {
        bf16* dst = O + q_row[qb] * ldo + col0;
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
      } else {
        float* dst = part_o + (group_tiles > 0 ? (slot * rows + q_row[qb]) * D
                                               : ((int64_t)(gi % n_split) * rows + q_row[qb]) * hidden + col0);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int d = db * 32 + 8 * g + 4 * hi;
            if (d < D)
              *reinterpret_cast<float4*>(dst + d) = make_float4(o[qb][db][4 * g + 0] * inv, o[qb][db][4 * g + 1] * inv,
                                                                o[qb][db][4 * g + 2] * inv, o[qb][db][4 * g + 3] * inv);
          }
      }
      if (!whole && hi == 0)
        reinterpret_cast<float2*>(part_ml)[slot * rows + q_row[qb]] = make_float2(m_ref[qb], l_tot);
    }
    if constexpr (!SK) break;   // one piece
  }   // pieces
}

// Merge the partial results of the pieces of each (query row, head).  Piece k holds
// x_k = acc_k / l_k (fp32) with its integer reference m_k and weight sum l_k, so
// O = sum_k w_k x_k / sum_k w_k with w_k = 2^(m_k - M) l_k (M = max_k m_k, 2^(m_k - M) exact):
// a convex combination of the pieces' results.  The pieces of head h sit in slots
// h + k * H, k < n_split (fixed split: results [k][row][hidden]), or h + g for the groups g
// whose stretches of the (head, key tile) line meet head h (stream-K: results [slot][row][D];
// a head inside one stretch was written whole).
// One thread per (row, head, 8 columns).  The loop over pieces is unrolled to the largest
// piece count (indices past the count clamped, their terms skipped), so every load of a
// thread is issued before the first is used.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml, int n_split,
                                                           int64_t group_tiles, int64_t ntiles, int64_t rows,
                                                           int H, bf16* __restrict__ O, int64_t ldo) {
  constexpr int NC = D / 8;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= rows * H * NC) return;
  const int chunk = (int)(id % NC);
  const int64_t rest = id / NC;
  const int head = (int)(rest % H);
  const int64_t row = rest / H;
  int count;
  int64_t base, stride;
  if (group_tiles > 0) {
    const int64_t g0 = (int64_t)head * ntiles / group_tiles;
    const int64_t g1 = ((int64_t)head * ntiles + ntiles - 1) / group_tiles;
    if (g0 == g1) return;
    count = (int)(g1 - g0 + 1);
    base = head + g0;
    stride = 1;
  } else {
    count = n_split;
    base = head;
    stride = H;
  }
  float m[kMaxAttnSplit], l[kMaxAttnSplit];
  float4 xa[kMaxAttnSplit], xb[kMaxAttnSplit];
#pragma unroll
  for (int sp = 0; sp < kMaxAttnSplit; ++sp) {
    const int64_t sc = base + (sp < count ? sp : count - 1) * stride;   // past the count: re-read the last (unused)
    const float2 ml = reinterpret_cast<const float2*>(part_ml)[sc * rows + row];
    m[sp] = ml.x;
    l[sp] = ml.y;
    const int64_t k = sp < count ? sp : count - 1;
    const float4* src = reinterpret_cast<const float4*>(
        part_o + (group_tiles > 0 ? (sc * rows + row) * D : (k * rows + row) * (int64_t)H * D + (int64_t)head * D) +
        chunk * 8);
    xa[sp] = src[0];
    xb[sp] = src[1];
  }
  float M = m[0];
#pragma unroll
  for (int sp = 1; sp < kMaxAttnSplit; ++sp)
    if (sp < count) M = fmaxf(M, m[sp]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
#pragma unroll
  for (int sp = 0; sp < kMaxAttnSplit; ++sp) {
    if (sp < count) {
      const float w = __builtin_amdgcn_exp2f(m[sp] - M) * l[sp];
      wsum += w;
      acc[0] = fmaf(w, xa[sp].x, acc[0]);
      acc[1] = fmaf(w, xa[sp].y, acc[1]);
      acc[2] = fmaf(w, xa[sp].z, acc[2]);
      acc[3] = fmaf(w, xa[sp].w, acc[3]);
      acc[4] = fmaf(w, xb[sp].x, acc[4]);
      acc[5] = fmaf(w, xb[sp].y, acc[5]);
      acc[6] = fmaf(w, xb[sp].z, acc[6]);
      acc[7] = fmaf(w, xb[sp].w, acc[7]);
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
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_bf16_kernel<D, AttnCfg<D>::QB, false>, 64 * kAttnWaves,
                                                     0) != hipSuccess || per_cu <= 0)
      per_cu = 1;
    (void)hipGetLastError();
    cached[dev] = cus * per_cu;
  }
  return cached[dev];
}

// How one bf16 launch divides its work (see attn_bf16_kernel): the fixed split of every
// (query tile, head) pair's key range into n_split equal parts, or the grouped stream-K
// schedule with group_tiles key tiles per group.  The choice minimises an estimate of the
// busiest workgroup slot's time in key tiles: the tiles it runs plus kPieceTiles for each
// piece (Q load, ring fill, result write), plus 3% for the merge pass when there are
// partials, among the schedules whose partials fit in ws_bytes.
struct AttnPlan {
  int n_split = 1;            // fixed split: parts of each key range (1: no partials)
  int tps = 0;                // fixed split: key tiles per part
  int64_t group_tiles = 0;    // > 0: grouped stream-K, key tiles per group
  int64_t grid = 0;           // workgroups
  int64_t slots = 0;          // partial slots (0: none)
};
constexpr double kPieceTiles = 16.0;

static size_t partial_bytes(int64_t slots, int64_t rows, int head_dim) {
  return (size_t)slots * rows * ((size_t)head_dim * sizeof(float) + 2 * sizeof(float));
}

static AttnPlan plan_attention(int64_t n_qtiles, int heads, int64_t ntiles, int64_t all_rows, int head_dim,
                               int slots, size_t ws_bytes) {
  AttnPlan best;
  const int64_t wg = n_qtiles * heads;
  best.tps = (int)ntiles;
  best.grid = wg;
  double best_cost = (double)((wg + slots - 1) / slots) * ((double)ntiles + kPieceTiles);
  // fixed split: every part keeps at least 8 key tiles
  for (int sp = 2; sp <= kMaxAttnSplit; ++sp) {
    if (ntiles < 8LL * sp) break;
    const int tps = (int)((ntiles + sp - 1) / sp);
    const int used = (int)((ntiles + tps - 1) / tps);
    if (partial_bytes((int64_t)used * heads, all_rows, head_dim) > ws_bytes) break;
    const double cost = (double)((wg * used + slots - 1) / slots) * (tps + kPieceTiles) * 1.03;
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best.n_split = used;
      best.tps = tps;
      best.grid = wg * used;
      best.slots = (int64_t)used * heads;
    }
  }
  // grouped stream-K: one group of n_qtiles workgroups per slot group, one round
  const int64_t groups = slots / n_qtiles;
  if (groups >= 2) {
    const int64_t line = (int64_t)heads * ntiles;
    const int64_t gt = (line + groups - 1) / groups;
    const int64_t used = (line + gt - 1) / gt;
    const int64_t pieces = (gt + ntiles - 1) / ntiles + 1;        // heads one stretch can meet
    const int64_t per_head = (ntiles + gt - 1) / gt + 1;          // stretches one head can meet
    const int64_t nslots = heads + used - 1;
    if (gt >= 8 && per_head <= kMaxAttnSplit && partial_bytes(nslots, all_rows, head_dim) <= ws_bytes) {
      const double cost = ((double)gt + kPieceTiles * (double)pieces) * 1.03;
      if (cost < best_cost - 1e-9) {
        best_cost = cost;
        best.n_split = 1;
        best.tps = 0;
        best.group_tiles = gt;
        best.grid = used * n_qtiles;
        best.slots = nslots;
      }
    }
  }
  return best;
}

// `rows` query rows per sample, `batch` samples: sample b's query rows are rows b*rows ..
// of Q and O, its K / V buffers start b * kv_stride elements after sample 0's.
template <int D>
static AttnPlan plan_attn_d(int64_t rows, int64_t seq_kv, int heads, int64_t batch, size_t ws_bytes) {
  constexpr int BQ = kAttnWaves * 32 * AttnCfg<D>::QB;
  const int64_t n_qtiles = batch * ((rows + BQ - 1) / BQ);
  const int64_t ntiles = (seq_kv + kTileKeys - 1) / kTileKeys;
  return plan_attention(n_qtiles, heads, ntiles, batch * rows, D, attn_slots<D>(), ws_bytes);
}

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
    const AttnPlan plan = plan_attn_d<D>(rows, seq_kv, heads, batch, ws ? ws_bytes : 0);
    if (plan.slots && partial_bytes(plan.slots, all_rows, D) > ws_bytes) return hipErrorInvalidValue;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    // workspace: fp32 piece results (slots x all_rows x D floats), then fp32 (m, l) pairs [slots][all_rows]
    float* part_o = plan.slots ? static_cast<float*>(ws) : nullptr;
    float* part_ml = part_o ? part_o + (size_t)plan.slots * all_rows * D : nullptr;
    auto kernel = plan.group_tiles > 0 ? attn_bf16_kernel<D, QB, true> : attn_bf16_kernel<D, QB, false>;
    hipLaunchKernelGGL(kernel, dim3((unsigned)plan.grid), dim3(64 * kAttnWaves), 0, s,
                       static_cast<const bf16*>(q), ldq, static_cast<const bf16*>(k), ldk,
                       static_cast<const bf16*>(v), hidden, seq_kv, all_rows, n_qtiles, plan.n_split, plan.tps,
                       plan.group_tiles, static_cast<bf16*>(o), ldo, part_o, part_ml, scale_log2, rows, per_grp,
                       kv_stride);
    if (plan.slots) {
      const int64_t units = all_rows * heads * (D / 8);
      hipLaunchKernelGGL(attn_combine_kernel<D>, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s, part_o,
                         part_ml, plan.n_split, plan.group_tiles, ntiles, all_rows, heads,
                         static_cast<bf16*>(o), ldo);
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

template <int D>
static size_t split_bytes_d(int64_t rows, int64_t seq_kv, int heads, int64_t batch) {
  const AttnPlan plan = plan_attn_d<D>(rows, seq_kv, heads, batch, attention_workspace_bytes(batch * rows, (int64_t)heads * D, heads, kMaxAttnSplit));
  return partial_bytes(plan.slots, batch * rows, D);
}

size_t attention_split_workspace_bytes(int64_t rows, int64_t seq_kv, int64_t hidden, int heads, int head_dim,
                                       int dtype, int64_t batch) {
  if (dtype != kDtypeBF16 || rows <= 0 || batch <= 0) return 0;
  switch (head_dim) {
    case 64: return split_bytes_d<64>(rows, seq_kv, heads, batch);
    case 72: return split_bytes_d<72>(rows, seq_kv, heads, batch);
    case 128: return split_bytes_d<128>(rows, seq_kv, heads, batch);
    default: return 0;
  }
}

size_t attention_workspace_bytes(int64_t rows, int64_t hidden, int heads, int n_split) {
  if (n_split <= 1) return 0;
  return sizeof(float) * (size_t)n_split * rows * hidden + sizeof(float) * 2 * (size_t)n_split * rows * heads;
}

hipError_t launch_attention(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v, int64_t ldv,
                            int v_layout, int64_t hidden, int64_t seq_kv, int64_t rows, int heads, int head_dim,
                            void* o, int64_t ldo, int dtype, void* ws, size_t ws_bytes, hipStream_t s,
                            int64_t batch, int64_t kv_stride) {
  if (rows <= 0 || batch <= 0) return hipSuccess;
  // the bf16 kernel reads V in the K8 layout (8 keys of a column per 16 bytes) and whole
  // heads of hidden columns; the fp32 kernel reads V row by row
  if (v_layout != (dtype == kDtypeBF16 ? kLayoutK8 : kLayoutRows) || hidden != (int64_t)heads * head_dim ||
      seq_kv < 1)
    return hipErrorInvalidValue;
  switch (head_dim) {
    case 64:
      return launch_attn_d<64>(q, ldq, k, ldk, v, ldv, hidden, seq_kv, rows, heads, o, ldo, dtype, ws, ws_bytes, s,
                               batch, kv_stride);
    case 72:
      return launch_attn_d<72>(q, ldq, k, ldk, v, ldv, hidden, seq_kv, rows, heads, o, ldo, dtype, ws, ws_bytes, s,
                               batch, kv_stride);
    case 128:
      return launch_attn_d<128>(q, ldq, k, ldk, v, ldv, hidden, seq_kv, rows, heads, o, ldo, dtype, ws, ws_bytes, s,
                                batch, kv_stride);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace pf
