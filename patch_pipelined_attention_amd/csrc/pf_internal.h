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

constexpr int kDtypeBF16 = 0;
constexpr int kDtypeFP32 = 1;
constexpr int kLayoutRows = 0;
constexpr int kLayoutK8 = 1;

// Epilogue codes (same values as pf_epilogue in pf.h).
constexpr int kEpiStore = 0;
constexpr int kEpiGeluTanh = 1;
constexpr int kEpiGeluErf = 2;
constexpr int kEpiGatedResidual = 3;

// Largest hidden size the row kernels (LayerNorm) keep in registers.
constexpr int kMaxHidden = 6144;

struct KVDesc {            // one K or V matrix
  const void* base;
  int64_t ld;              // row stride in elements (ROWS layout)
  int layout;              // kLayoutRows / kLayoutK8
};

// ---- launchers (each enqueues one kernel on `s` and returns hipGetLastError()) ----

hipError_t launch_ln_modulate(const float* x, int64_t rows, int hidden, const float* shift,
                              const float* scale, float eps, void* y, int dtype, hipStream_t s);

hipError_t launch_adaln(const float* cond, const void* w, const float* b, int hidden, float* mod,
                        int dtype, hipStream_t s);

// `ws` (may be NULL) is scratch for the k-split of grids too small to fill the GPU.
hipError_t launch_gemm(const void* a, int64_t lda, const void* w, const float* bias, int64_t m,
                       int64_t n, int64_t k, int epi, void* c, int64_t ldc, const float* gate,
                       int dtype, void* ws, size_t ws_bytes, hipStream_t s);

// Scratch bytes the bf16 GEMM would use for its k-split at this shape (0: no split).
size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k);

constexpr int kMaxGemmSplit = 8;

// `ws` (may be NULL) is scratch for the key-range split of small query grids; the split
// count is chosen so its partial results fit in ws_bytes (NULL: no split).
hipError_t launch_attention(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v,
                            int64_t ldv, int v_layout, int64_t hidden, int64_t seq_kv, int64_t rows,
                            int heads, int head_dim, void* o, int64_t ldo, int dtype, void* ws,
                            size_t ws_bytes, hipStream_t s);

// Scratch bytes the attention needs for `n_split` key-range splits of `rows` queries.
size_t attention_workspace_bytes(int64_t rows, int64_t hidden, int heads, int n_split);

// Upper bound of the split count launch_attention uses.
constexpr int kMaxAttnSplit = 8;

// Bit copy of `len` rows x `row_elems` elements of K and of V (two matrices per call).
hipError_t launch_splice(const KVDesc dst[2], const KVDesc src[2], int64_t row_elems, int64_t offset,
                         int64_t len, int esize, hipStream_t s);

}  // namespace pf
