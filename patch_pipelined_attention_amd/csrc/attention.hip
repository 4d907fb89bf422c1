// Patch attention: the queries of one patch attend over every row of a layer's
// full-spatial K/V buffer (PipeFusion keeps full attention; the buffer mixes fresh and
// stale rows).  Flash-style single pass with online softmax; no score matrix is stored.
//
// bf16 kernel (head_dim D in {64, 72, 128}), gfx950 MFMA v_mfma_f32_32x32x16_bf16:
//   * workgroup = 128 queries of one head, 4 wavefronts x 32 queries; key tiles of 64
//     rows staged in LDS (K row-major, V in the K8 layout of the buffer, see pf.h).
//   * scores are computed transposed, S^T = K . Q^T, so each lane owns one query and 16
//     keys per 32x32 block: the row max is a lane-local max3 chain plus one exchange with
//     the lane 32 away, and the row sum stays lane-local until the end.
//   * the K rows feeding the score MFMA are permuted (bits 2 and 3 of the row index
//     swapped) so that each lane's 8 consecutive score registers are 8 consecutive keys:
//     they pack directly into the bf16 "B" operand of O^T += V^T . P^T without any
//     cross-lane shuffle, and the matching V^T operand is one 16-byte K8 read per lane.
//   * softmax in base 2: p = exp2(s * log2(e)/sqrt(D) - m), fp32 statistics, P rounded to
//     bf16 for the P.V product.
//   * D = 72 pads the score contraction to 80 and the output rows to 96 with zero
//     operands; nothing outside the real 72 columns is read or written.
//   * the block index is remapped so each XCD (blocks are dealt round-robin to the 8
//     XCDs) works on a contiguous run of query tiles of the same head, which share K/V
//     in that XCD's L2.
//
// fp32 kernel (tiny fp32 stages only): one thread per query, key tiles in LDS.
#include "pf_internal.h"

namespace pf {

namespace {
constexpr int kBQ = 128;   // queries per workgroup
constexpr int kBKey = 64;  // keys per tile
}  // namespace

__device__ __forceinline__ int swap_bits23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  const int per = nb / 8, rem = nb % 8;
  const int x = bid % 8;
  return x * per + (x < rem ? x : rem) + bid / 8;
}

template <int D>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(const bf16* __restrict__ Q, int64_t ldq,
                                                           const bf16* __restrict__ Kb, int64_t ldk,
                                                           const bf16* __restrict__ Vb, int64_t hidden,
                                                           int64_t S, int64_t rows, int n_qtiles,
                                                           bf16* __restrict__ O, int64_t ldo,
                                                           float scale_log2) {
  constexpr int KS = (D + 15) / 16;                 // k-steps of the score MFMA
  constexpr int DB = (D + 31) / 32;                 // 32-row blocks of O^T
  constexpr int KLD = ((D / 8) % 2 == 0) ? D + 8 : D;  // odd number of 16-byte units per LDS row
  constexpr int KCH = kBKey * D / 8;                // 16-byte chunks per K (and per V) tile
  constexpr int KPT = (KCH + 255) / 256;            // chunks per thread

  __shared__ __attribute__((aligned(16))) bf16 sK[kBKey * KLD];
  __shared__ __attribute__((aligned(16))) bf16 sV[kBKey * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int head = lid / n_qtiles;
  const int qt = lid - head * n_qtiles;
  const int64_t q_row = (int64_t)qt * kBQ + wave * 32 + l32;
  const int64_t col0 = (int64_t)head * D;

  // Q^T fragments (the "B" operand of the score MFMA): 8 consecutive d of this lane's query.
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int d0 = ks * 16 + hi * 8;
    if (q_row < rows && d0 < D) {
      qf[ks] = *reinterpret_cast<const bf16x8*>(Q + q_row * ldq + col0 + d0);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ks][e] = (bf16)0.f;
    }
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int64_t ngroups = (S + 7) >> 3;   // K8 groups present in the V buffer
  uint4 rk[KPT], rv[KPT];
  auto load_tile = [&](int64_t t) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + 256 * i;
      if (c < KCH) {
        const int row = c / (D / 8), c8 = c - row * (D / 8);
        const int64_t key = t * kBKey + row;
        rk[i] = key < S ? *reinterpret_cast<const uint4*>(Kb + key * ldk + col0 + c8 * 8) : make_uint4(0, 0, 0, 0);
        const int g = c / D, d = c - g * D;
        const int64_t gg = t * 8 + g;
        if (gg < ngroups) {
          uint4 v = *reinterpret_cast<const uint4*>(Vb + ((gg * hidden) + col0 + d) * 8);
          const int64_t valid = S - gg * 8;   // keys of this group inside the buffer
          if (valid < 8) {                    // zero the rows past the end of the buffer
            uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (e >= valid) w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
            v = make_uint4(w[0], w[1], w[2], w[3]);
          }
          rv[i] = v;
        } else {
          rv[i] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + 256 * i;
      if (c < KCH) {
        const int row = c / (D / 8), c8 = c - row * (D / 8);
        *reinterpret_cast<uint4*>(&sK[row * KLD + c8 * 8]) = rk[i];
        *reinterpret_cast<uint4*>(&sV[c * 8]) = rv[i];   // K8 tile: [group][d][8] is contiguous
      }
    }
  };

  const int64_t ntiles = (S + kBKey - 1) / kBKey;
  load_tile(0);
  store_tile();
  __syncthreads();

  for (int64_t t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) load_tile(t + 1);

    // ---- S^T = K . Q^T for 2 blocks of 32 keys ----
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
      const int krow = kb * 32 + swap_bits23(l32);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int d0 = ks * 16 + hi * 8;
        bf16x8 a;
        if (d0 < D) {
          a = *reinterpret_cast<const bf16x8*>(&sK[krow * KLD + d0]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) a[e] = (bf16)0.f;
        }
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
      }
    }
    // lane owns query l32 and, for acc index 4g+j of block kb, key
    // t*64 + kb*32 + swap_bits23(8g + 4hi + j) = t*64 + kb*32 + 16(g>>1) + 8hi + 4(g&1) + j.
    if ((t + 1) * kBKey > S) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int64_t key = t * kBKey + kb * 32 + 16 * (g >> 1) + 8 * hi + 4 * (g & 1) + j;
            if (key >= S) s[kb][4 * g + j] = -INFINITY;
          }
    }

    // ---- online softmax (base 2) ----
    float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, fmaxf(s[0][e], s[1][e]));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][e], scale_log2, -m_new));
        s[kb][e] = p;
        rs += p;
      }
    l_run = fmaf(l_run, alpha, rs);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[db][e] *= alpha;

    // ---- O^T += V^T . P^T : 2 key blocks x 2 halves of 16 keys ----
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int j = 0; j < 4; ++j) pb[4 * e + j] = (bf16)s[kb][4 * (2 * h2 + e) + j];
        const int grp = 4 * kb + 2 * h2 + hi;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int d = db * 32 + l32;
          bf16x8 a;
          if (d < D) {
            a = *reinterpret_cast<const bf16x8*>(&sV[(grp * D + d) * 8]);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] = (bf16)0.f;
          }
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o[db], 0, 0, 0);
        }
      }

    __syncthreads();
    if (t + 1 < ntiles) {
      store_tile();
      __syncthreads();
    }
  }

  // ---- normalise and store: lane holds O[query l32][d = db*32 + 8g + 4hi + j] ----
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  if (q_row < rows) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + 8 * g + 4 * hi;
        if (d < D) {
          bf16x4 ov = {(bf16)(o[db][4 * g + 0] * inv), (bf16)(o[db][4 * g + 1] * inv),
                       (bf16)(o[db][4 * g + 2] * inv), (bf16)(o[db][4 * g + 3] * inv)};
          *reinterpret_cast<bf16x4*>(O + q_row * ldo + col0 + d) = ov;
        }
      }
  }
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

template <int D>
static void launch_attn_d(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v, int64_t ldv,
                          int64_t hidden, int64_t seq_kv, int64_t rows, int heads, void* o, int64_t ldo,
                          int dtype, hipStream_t s) {
  if (dtype == kDtypeBF16) {
    const int n_qtiles = (int)((rows + kBQ - 1) / kBQ);
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    hipLaunchKernelGGL(attn_bf16_kernel<D>, dim3((unsigned)(n_qtiles * heads)), dim3(256), 0, s,
                       static_cast<const bf16*>(q), ldq, static_cast<const bf16*>(k), ldk,
                       static_cast<const bf16*>(v), hidden, seq_kv, rows, n_qtiles, static_cast<bf16*>(o), ldo,
                       scale_log2);
  } else {
    const int n_qtiles = (int)((rows + 63) / 64);
    hipLaunchKernelGGL(attn_f32_kernel<D>, dim3((unsigned)(n_qtiles * heads)), dim3(64), 0, s,
                       static_cast<const float*>(q), ldq, static_cast<const float*>(k), ldk,
                       static_cast<const float*>(v), ldv, seq_kv, rows, n_qtiles, static_cast<float*>(o), ldo,
                       1.0f / sqrtf((float)D));
  }
}

hipError_t launch_attention(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v, int64_t ldv,
                            int v_layout, int64_t hidden, int64_t seq_kv, int64_t rows, int heads, int head_dim,
                            void* o, int64_t ldo, int dtype, hipStream_t s) {
  (void)v_layout;
  if (rows <= 0) return hipSuccess;
  switch (head_dim) {
    case 64: launch_attn_d<64>(q, ldq, k, ldk, v, ldv, hidden, seq_kv, rows, heads, o, ldo, dtype, s); break;
    case 72: launch_attn_d<72>(q, ldq, k, ldk, v, ldv, hidden, seq_kv, rows, heads, o, ldo, dtype, s); break;
    default: launch_attn_d<128>(q, ldq, k, ldk, v, ldv, hidden, seq_kv, rows, heads, o, ldo, dtype, s); break;
  }
  return hipGetLastError();
}

}  // namespace pf
