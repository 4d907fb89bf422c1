// Internal declarations shared by the HIP kernels and the stage runtime of libpf.
// Device code targets gfx950 (CDNA4) only: 64-lane wavefronts, bf16 MFMA with fp32
// accumulation, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pf {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Message returned by pf_last_error() on this thread (set by every failing call).
void pf_set_last_error(const char* msg);

constexpr int kDtypeBF16 = 0;
constexpr int kDtypeFP32 = 1;
constexpr int kLayoutRows = 0;
constexpr int kLayoutK8 = 1;

// Epilogue codes (same values as pf_epilogue in pf.h).
constexpr int kEpiStore = 0;
constexpr int kEpiGeluTanh = 1;
constexpr int kEpiGeluErf = 2;
constexpr int kEpiGatedResidual = 3;
constexpr int kEpiQkvSplice = 4;   // stage only: Q to C, K and V into the layer's KV buffer

// Workgroup barrier for kernels that keep direct global -> LDS loads in flight across
// barriers.  __syncthreads() (and any release fence covering LDS) makes each wavefront
// drain every outstanding global load, those LDS-bound ones included, before the
// barrier.  Here the caller waits for exactly the loads that must have landed with an
// explicit vmcnt count, and every LDS read issued before the barrier has been consumed
// (and so completed) by then; the empty asm statements keep the compiler from moving
// memory accesses across the barrier, the scheduling barriers keep any instruction from
// crossing it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// 16-byte direct global -> LDS load (gfx950 global_load_lds_dwordx4, scalar-base form):
// lane l reads sbase + voff[l] and writes lds_base + 16 l.  sbase and lds_base must be
// wavefront-uniform (the first lane's values are used).  Written as asm so that the compiler does not see an LDS store it
// cannot tell apart from every LDS read: it would otherwise make each later LDS read
// wait for all loads in flight (vmcnt 0), which serialises a prefetch ring.  The caller
// owns the wait: s_waitcnt vmcnt for this wavefront's loads, then a workgroup barrier,
// before any wavefront reads the stage.  The instruction has no destination register.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_load16(const void* sbase, uint32_t voff, const void* lds_base) {
  // readfirstlane returns int: both halves go through uint32_t so the low word is
  // zero-extended when the pointer is put back together
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  const uint64_t b = (uint64_t)(uintptr_t)sbase;
  const uint32_t b_hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t b_lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint64_t bs = ((uint64_t)b_hi << 32) | (uint64_t)b_lo;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(bs), "s"(m0)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Largest hidden size the row kernels (LayerNorm) keep in registers.
constexpr int kMaxHidden = 6144;

struct KVDesc {            // one K or V matrix
  const void* base;
  int64_t ld;              // row stride in elements (ROWS layout)
  int layout;              // kLayoutRows / kLayoutK8
};

// Rows of a batched launch (samples that share the weights): row j belongs to sample
// g = j / rows, local row i = j - g * rows.  Sample g's rows of a strided operand (x, or C of
// the gated residual) start `x_stride` elements after sample g-1's, and its per-feature
// parameter vectors (shift, scale, gate) `p_stride` elements after sample g-1's.  One sample
// is {total rows, 0, 0}.
struct RowGroups {
  int64_t rows;
  int64_t x_stride;
  int64_t p_stride;
};

// Destination of the fused QKV epilogue (kEpiQkvSplice, bf16 only): output features [0, h)
// (Q) go to c; features [h, 2h) of row j (sample g, local row i, see RowGroups with
// grp_rows) are row `row0 + i` of sample g's K buffer (ROWS layout, row stride h) and
// [2h, 3h) the same row of its V buffer (K8 layout, h columns).  Sample g's buffers start
// k_stride / v_stride elements after sample g-1's.
struct QkvSplice {
  void* k;
  void* v;
  int64_t row0;
  int64_t h;
  int64_t grp_rows;
  int64_t k_stride;
  int64_t v_stride;
};

// ---- launchers (each enqueues one kernel on `s` and returns hipGetLastError()) ----

// y (contiguous [rows, hidden]) from x; `groups` (NULL: one sample) gives each sample's x rows
// and shift / scale vectors.
hipError_t launch_ln_modulate(const float* x, int64_t rows, int hidden, const float* shift,
                              const float* scale, float eps, void* y, int dtype, hipStream_t s,
                              const RowGroups* groups = nullptr);

// mod [chunks * hidden] = SiLU(cond) . w^T + b (chunks: 6 for the DiT block, 3 for the parallel one)
hipError_t launch_adaln(const float* cond, const void* w, const float* b, int hidden, float* mod,
                        int dtype, hipStream_t s, int chunks = 6);

// The same for n_sets weight sets x n_samples conditions in one launch: set m's matrix at
// w + m * w_stride elements, its bias at b + m * b_stride, its output for sample g at
// mod + m * mod_stride + g * mod_sample_stride; sample g's cond at cond + g * cond_stride.
hipError_t launch_adaln_batch(const float* cond, int64_t cond_stride, int n_samples, const void* w,
                              int64_t w_stride, const float* b, int64_t b_stride, int n_sets, int hidden,
                              float* mod, int64_t mod_stride, int64_t mod_sample_stride, int dtype, hipStream_t s,
                              int chunks = 6);

// The LayerNorm + modulation that follows a gated-residual projection (the next sublayer's):
// y [m, n] bf16 (row stride n) = LN(x)(1 + scale) + shift of the updated residual rows, with
// each sample's shift / scale at + g * groups->p_stride.
struct LnAfter {
  const float* shift;
  const float* scale;
  float eps;
  void* y;
};

// `ws` (may be NULL) is scratch for the k-split of grids too small to fill the GPU.
// `groups` (NULL: one sample) applies to the gated residual: each sample's rows of c and its
// gate vector.  `ln` (gated residual, bf16 only): when the product is k-split, its reduce pass
// also computes the LayerNorm + modulation of the updated rows and sets *ln_done (otherwise
// *ln_done is false and the caller runs launch_ln_modulate itself).
hipError_t launch_gemm(const void* a, int64_t lda, const void* w, const float* bias, int64_t m,
                       int64_t n, int64_t k, int epi, void* c, int64_t ldc, const float* gate,
                       int dtype, void* ws, size_t ws_bytes, hipStream_t s,
                       const QkvSplice* splice = nullptr, const RowGroups* groups = nullptr,
                       const LnAfter* ln = nullptr, bool* ln_done = nullptr);

// Reduce of a k-split gated-residual product fused with the following LayerNorm + modulation:
// per row m, y = sum_s part[s][m][:] + bias, x_m += gate_g * y (stored), then ln.y[m] =
// LN(x_m)(1 + scale_g) + shift_g in bf16.  Same arithmetic, in the same order, as the plain
// reduce followed by launch_ln_modulate, so the results are bit-identical.
hipError_t launch_reduce_residual_ln(const float* part, int n_split, int64_t m, int n, const float* bias, float* x,
                                     int64_t ldx, const float* gate, const RowGroups& rg, const LnAfter& ln,
                                     hipStream_t s);

// Scratch bytes the bf16 GEMM would use for its k-split at this shape (0: no split).
size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k);

constexpr int kMaxGemmSplit = 8;

// `ws` (may be NULL) is scratch for the key-range split of small query grids; the split
// count is chosen so its partial results fit in ws_bytes (NULL: no split).  `batch` samples of
// `rows` query rows each in one launch: sample b's rows are rows b*rows .. of q and o, its K / V
// buffers start b * kv_stride elements after k / v.
hipError_t launch_attention(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v,
                            int64_t ldv, int v_layout, int64_t hidden, int64_t seq_kv, int64_t rows,
                            int heads, int head_dim, void* o, int64_t ldo, int dtype, void* ws,
                            size_t ws_bytes, hipStream_t s, int64_t batch = 1, int64_t kv_stride = 0);

// Scratch bytes the attention needs for `n_split` key-range splits of `rows` queries (all
// samples' rows of a batched launch).
size_t attention_workspace_bytes(int64_t rows, int64_t hidden, int heads, int n_split);

// Upper bound of the split count launch_attention uses.
constexpr int kMaxAttnSplit = 8;

// Workspace bytes of the key-range split launch_attention chooses for this launch when the
// workspace does not limit it (0: no split; always 0 for fp32).
size_t attention_split_workspace_bytes(int64_t rows, int64_t seq_kv, int64_t hidden, int heads, int head_dim,
                                       int dtype, int64_t batch = 1);

// The library's static device scratch (allocation-free entry points): its address on the
// current device (looked up once per device) and its size.
constexpr size_t kStaticScratchBytes = (size_t)128 << 20;
hipError_t static_scratch(void** ptr);

// Q rows (q, row stride ldq) and K buffer rows [off, off + n) (row stride ldk; sample g's
// buffer kv_stride elements after sample 0's) of nb samples, bf16 in place: per-head RMSNorm
// times gq / gk (norm), then rotary pairs by angles[buffer row] (rope).
hipError_t launch_qk_norm_rope(void* q, int64_t ldq, void* k, int64_t ldk, int64_t kv_stride, int64_t off, int64_t n,
                               int64_t nb, int heads, int head_dim, const float* gq, const float* gk,
                               const float* angles, bool norm, bool rope, hipStream_t s);

// ---- the denoising loop around a stage (fp32) ----
// out[b][j] = act(sum_i in[i] W[j, i] + bias[j]) + add[b][j]; in == NULL uses the frequency
// features of timestep t; add == NULL needs batch == 1.
hipError_t launch_gemv_f32(const float* in, double t, bool silu_in, const float* W, const float* bias, int k,
                           int n_out, bool silu_out, const float* add, int batch, float* out, hipStream_t s);
// x[b][row0 + s] = patch_{b,s} . Wp^T + bp + pos[s] for every patch s of every sample b.
hipError_t launch_patch_embed(const float* z, int C, int p, int grid_w, int64_t n_patches, int hidden, const float* Wp,
                              const float* bp, const float* pos, float* x, int64_t x_batch_stride, int64_t row0,
                              int batch, hipStream_t s);
// z = a z + e eps per latent element, eps unpatchified from v [batch][n_patches][C p p]
// (guided: a pair's eps_1 + g (eps_0 - eps_1) for both samples).
hipError_t launch_guided_ddim(float* z, const float* v, int C, int p, int grid_w, int64_t n_patches, int batch,
                              bool guided, float g, float a, float e, hipStream_t s);

// Bit copy of `len` rows x `row_elems` elements of K and of V (two matrices per call).
hipError_t launch_splice(const KVDesc dst[2], const KVDesc src[2], int64_t row_elems, int64_t offset,
                         int64_t len, int esize, hipStream_t s);

}  // namespace pf
