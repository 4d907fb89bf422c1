// Stage runtime and C ABI of libpf (declarations and contracts in include/pf.h).
//
// One pf_stage is one GPU's share of a PipeFusion pipeline (technical summaries on
// gist.science, "Core mechanisms" 1, 2 and 4): the weights of L contiguous layers, one
// full-spatial K/V buffer per layer (a single copy, updated in place), and scratch for a
// micro-step of up to seq_txt + seq_img rows.  Every call validates its arguments before
// enqueuing anything, then enqueues kernels on the caller's stream and returns.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "pf.h"
#include "pf_internal.h"

using namespace pf;

// ------------------------------------------------------------------------------------
// errors
// ------------------------------------------------------------------------------------
static thread_local std::string g_last_error;

static pf_status fail(pf_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

static pf_status hip_fail(hipError_t e, const char* what) {
  return fail(PF_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

extern "C" const char* pf_last_error(void) { return g_last_error.c_str(); }

void pf::pf_set_last_error(const char* msg) { g_last_error = msg; }

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
static bool ranges_overlap(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + bn && b0 < a0 + an;
}
static size_t dtype_size(int dt) { return dt == PF_BF16 ? 2 : 4; }
static bool dtype_ok(int dt) { return dt == PF_BF16 || dt == PF_FP32; }

// The kernels are built for gfx950 only.  Also drops any error a HIP call outside this
// library left behind, so that the launch checks below report only this call's errors.
static pf_status check_device() {
  static thread_local int checked_dev = -1;
  (void)hipGetLastError();
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev == checked_dev) return PF_OK;
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(PF_ERR_UNSUPPORTED, "device %d is %s; libpf is built for gfx950 only", dev, prop.gcnArchName);
  checked_dev = dev;
  return PF_OK;
}

// ------------------------------------------------------------------------------------
// component validation helpers (pure host checks: no HIP call)
// ------------------------------------------------------------------------------------
static pf_status validate_ln(const float* x, int64_t rows, int32_t hidden, const float* shift,
                             const float* scale, void* y, int32_t dtype) {
  if (!dtype_ok(dtype)) return fail(PF_ERR_INVALID_ARG, "ln_modulate: bad dtype %d", dtype);
  if (rows < 0) return fail(PF_ERR_INVALID_ARG, "ln_modulate: rows < 0");
  if (hidden <= 0 || hidden % 8 != 0 || hidden > kMaxHidden)
    return fail(PF_ERR_UNSUPPORTED, "ln_modulate: hidden %d must be a positive multiple of 8 <= %d", hidden,
                kMaxHidden);
  if (!x || !shift || !scale || !y) return fail(PF_ERR_INVALID_ARG, "ln_modulate: null pointer");
  if (!aligned16(x) || !aligned16(shift) || !aligned16(scale) || !aligned16(y))
    return fail(PF_ERR_INVALID_ARG, "ln_modulate: pointers must be 16-byte aligned");
  return PF_OK;
}

static pf_status validate_gemm(const void* a, int64_t lda, const void* w, const float* bias, int64_t m,
                               int64_t n, int64_t k, int32_t epi, void* c, int64_t ldc, const float* gate,
                               int32_t dtype) {
  if (!dtype_ok(dtype)) return fail(PF_ERR_INVALID_ARG, "gemm: bad dtype %d", dtype);
  if (epi < PF_EPI_STORE || epi > PF_EPI_GATED_RESIDUAL) return fail(PF_ERR_INVALID_ARG, "gemm: bad epilogue %d", epi);
  if (m < 0 || n <= 0 || k <= 0) return fail(PF_ERR_INVALID_ARG, "gemm: bad sizes m=%lld n=%lld k=%lld",
                                             (long long)m, (long long)n, (long long)k);
  if (!a || !w || !bias || !c || (epi == PF_EPI_GATED_RESIDUAL && !gate))
    return fail(PF_ERR_INVALID_ARG, "gemm: null pointer");
  if (lda < k || ldc < n) return fail(PF_ERR_INVALID_ARG, "gemm: lda < k or ldc < n");
  if (!aligned16(a) || !aligned16(w) || !aligned16(bias) || !aligned16(c) || (gate && !aligned16(gate)))
    return fail(PF_ERR_INVALID_ARG, "gemm: pointers must be 16-byte aligned");
  if (dtype == PF_BF16) {
    if (n % 64 != 0 || k % 64 != 0)
      return fail(PF_ERR_UNSUPPORTED, "gemm: bf16 needs n %% 64 == 0 and k %% 64 == 0 (n=%lld k=%lld)",
                  (long long)n, (long long)k);
    if (lda % 8 != 0 || ldc % 4 != 0) return fail(PF_ERR_INVALID_ARG, "gemm: bf16 needs lda %% 8 == 0, ldc %% 4 == 0");
  }
  return PF_OK;
}

static pf_status validate_kv_view(const pf_kv_view* v, const char* who) {
  if (!v) return fail(PF_ERR_INVALID_ARG, "%s: null view", who);
  if (!dtype_ok(v->dtype)) return fail(PF_ERR_INVALID_ARG, "%s: bad view dtype", who);
  if (v->v_layout != PF_LAYOUT_ROWS && v->v_layout != PF_LAYOUT_K8)
    return fail(PF_ERR_INVALID_ARG, "%s: bad v_layout", who);
  if (v->rows < 0 || v->row_elems <= 0) return fail(PF_ERR_INVALID_ARG, "%s: bad view rows/row_elems", who);
  if (!v->k || !v->v) return fail(PF_ERR_INVALID_ARG, "%s: null K or V pointer", who);
  if (v->k_ld < v->row_elems) return fail(PF_ERR_INVALID_ARG, "%s: k_ld < row_elems", who);
  if (v->v_layout == PF_LAYOUT_ROWS && v->v_ld < v->row_elems)
    return fail(PF_ERR_INVALID_ARG, "%s: v_ld < row_elems", who);
  return PF_OK;
}

// byte extent [lo, hi) of the K or V matrix of a view (rows covered by the view)
static void view_extent(const pf_kv_view* v, bool is_v, int64_t r0, int64_t n, uintptr_t* lo, uintptr_t* hi) {
  const size_t es = dtype_size(v->dtype);
  if (n <= 0) { *lo = *hi = 0; return; }
  if (is_v && v->v_layout == PF_LAYOUT_K8) {
    const int64_t g0 = r0 / 8, g1 = (r0 + n - 1) / 8 + 1;
    *lo = (uintptr_t)v->v + (uintptr_t)(g0 * v->row_elems * 8 * es);
    *hi = (uintptr_t)v->v + (uintptr_t)(g1 * v->row_elems * 8 * es);
  } else {
    const int64_t ld = is_v ? v->v_ld : v->k_ld;
    const char* base = (const char*)(is_v ? v->v : v->k);
    *lo = (uintptr_t)base + (uintptr_t)(r0 * ld * es);
    *hi = (uintptr_t)base + (uintptr_t)(((r0 + n - 1) * ld + v->row_elems) * es);
  }
}

static pf_status validate_splice(const pf_kv_view* dst, const pf_kv_view* src, int64_t offset, int64_t len) {
  pf_status st = validate_kv_view(dst, "kvbuf_splice(dst)");
  if (st != PF_OK) return st;
  st = validate_kv_view(src, "kvbuf_splice(src)");
  if (st != PF_OK) return st;
  if (dst->dtype != src->dtype) return fail(PF_ERR_INVALID_ARG, "kvbuf_splice: dtype mismatch");
  if (dst->row_elems != src->row_elems) return fail(PF_ERR_INVALID_ARG, "kvbuf_splice: row_elems mismatch");
  if (offset < 0 || len < 0) return fail(PF_ERR_INVALID_ARG, "kvbuf_splice: negative offset or len");
  if (offset + len > dst->rows) return fail(PF_ERR_INVALID_ARG, "kvbuf_splice: offset + len > dst.rows");
  if (len > src->rows) return fail(PF_ERR_INVALID_ARG, "kvbuf_splice: len > src.rows");
  const size_t es = dtype_size(dst->dtype);
  if (!aligned16(dst->k) || !aligned16(dst->v) || (es == 4 && (((uintptr_t)src->k | (uintptr_t)src->v) & 3)) ||
      (es == 2 && (((uintptr_t)src->k | (uintptr_t)src->v) & 1)))
    return fail(PF_ERR_INVALID_ARG, "kvbuf_splice: misaligned pointer");
  if (len == 0) return PF_OK;
  for (int a = 0; a < 2; ++a)
    for (int b = 0; b < 2; ++b) {
      uintptr_t dlo, dhi, slo, shi;
      view_extent(dst, a == 1, offset, len, &dlo, &dhi);
      view_extent(src, b == 1, 0, len, &slo, &shi);
      if (dlo < shi && slo < dhi) return fail(PF_ERR_INVALID_ARG, "kvbuf_splice: src and dst overlap");
    }
  return PF_OK;
}

static pf_status validate_attention(const void* q, int64_t ldq, const pf_kv_view* kv, int64_t seq_kv,
                                    int64_t rows, int32_t heads, int32_t head_dim, void* o, int64_t ldo) {
  pf_status st = validate_kv_view(kv, "attention");
  if (st != PF_OK) return st;
  if (head_dim != 64 && head_dim != 72 && head_dim != 128)
    return fail(PF_ERR_UNSUPPORTED, "attention: head_dim %d not in {64, 72, 128}", head_dim);
  if (heads <= 0) return fail(PF_ERR_INVALID_ARG, "attention: heads <= 0");
  const int64_t h = (int64_t)heads * head_dim;
  if (kv->row_elems != h) return fail(PF_ERR_INVALID_ARG, "attention: kv row_elems != heads*head_dim");
  if (seq_kv < 1 || seq_kv > kv->rows) return fail(PF_ERR_INVALID_ARG, "attention: seq_kv out of range");
  if (rows < 0) return fail(PF_ERR_INVALID_ARG, "attention: rows < 0");
  if (!q || !o) return fail(PF_ERR_INVALID_ARG, "attention: null pointer");
  if (ldq < h || ldo < h) return fail(PF_ERR_INVALID_ARG, "attention: ldq/ldo < heads*head_dim");
  if (!aligned16(q) || !aligned16(o) || !aligned16(kv->k) || !aligned16(kv->v))
    return fail(PF_ERR_INVALID_ARG, "attention: pointers must be 16-byte aligned");
  if (kv->dtype == PF_BF16) {
    if (kv->v_layout != PF_LAYOUT_K8) return fail(PF_ERR_UNSUPPORTED, "attention: bf16 needs V in PF_LAYOUT_K8");
    if (ldq % 8 || ldo % 4 || kv->k_ld % 8) return fail(PF_ERR_INVALID_ARG, "attention: bf16 strides must keep 16 B rows");
    if (seq_kv * (int64_t)heads > (int64_t)1 << 40) return fail(PF_ERR_UNSUPPORTED, "attention: too large");
  } else {
    if (kv->v_layout != PF_LAYOUT_ROWS) return fail(PF_ERR_UNSUPPORTED, "attention: fp32 needs V in PF_LAYOUT_ROWS");
  }
  const int64_t tiles = (rows + 127) / 128 * heads;
  if (tiles > 0x7fffffff) return fail(PF_ERR_UNSUPPORTED, "attention: grid too large");
  return PF_OK;
}

// ------------------------------------------------------------------------------------
// component entry points
// ------------------------------------------------------------------------------------
extern "C" pf_status pf_ln_modulate(const float* x, int64_t rows, int32_t hidden, const float* shift,
                                    const float* scale, float eps, void* y, int32_t dtype, void* stream) {
  pf_status st = validate_ln(x, rows, hidden, shift, scale, y, dtype);
  if (st != PF_OK) return st;
  if ((st = check_device()) != PF_OK) return st;
  hipError_t e = launch_ln_modulate(x, rows, hidden, shift, scale, eps, y, dtype, (hipStream_t)stream);
  return e == hipSuccess ? PF_OK : hip_fail(e, "ln_modulate launch");
}

extern "C" pf_status pf_gemm(const void* a, int64_t lda, const void* w, const float* bias, int64_t m, int64_t n,
                             int64_t k, int32_t epi, void* c, int64_t ldc, const float* gate, int32_t dtype,
                             void* workspace, uint64_t workspace_bytes, void* stream) {
  pf_status st = validate_gemm(a, lda, w, bias, m, n, k, epi, c, ldc, gate, dtype);
  if (st != PF_OK) return st;
  if (workspace && !aligned16(workspace)) return fail(PF_ERR_INVALID_ARG, "gemm: workspace must be 16-byte aligned");
  if ((st = check_device()) != PF_OK) return st;
  hipError_t e = launch_gemm(a, lda, w, bias, m, n, k, epi, c, ldc, gate, dtype, workspace,
                             workspace ? (size_t)workspace_bytes : 0, (hipStream_t)stream);
  return e == hipSuccess ? PF_OK : hip_fail(e, "gemm launch");
}

extern "C" pf_status pf_gemm_residual_ln(const void* a, int64_t lda, const void* w, const float* bias, int64_t m,
                                         int64_t n, int64_t k, float* x, const float* gate, const float* shift,
                                         const float* scale, float eps, void* y, void* workspace,
                                         uint64_t workspace_bytes, void* stream) {
  pf_status st = validate_gemm(a, lda, w, bias, m, n, k, PF_EPI_GATED_RESIDUAL, x, n, gate, PF_BF16);
  if (st != PF_OK) return st;
  if ((st = validate_ln(x, m, (int32_t)n, shift, scale, y, PF_BF16)) != PF_OK) return st;
  if (workspace && !aligned16(workspace))
    return fail(PF_ERR_INVALID_ARG, "gemm_residual_ln: workspace must be 16-byte aligned");
  if (ranges_overlap(y, (size_t)(m * n) * 2, x, (size_t)(m * n) * 4))
    return fail(PF_ERR_INVALID_ARG, "gemm_residual_ln: y overlaps x");
  if ((st = check_device()) != PF_OK) return st;
  const hipStream_t s = (hipStream_t)stream;
  const LnAfter ln{shift, scale, eps, y};
  bool ln_done = false;
  hipError_t e = launch_gemm(a, lda, w, bias, m, n, k, kEpiGatedResidual, x, n, gate, PF_BF16, workspace,
                             workspace ? (size_t)workspace_bytes : 0, s, nullptr, nullptr, &ln, &ln_done);
  if (e == hipSuccess && !ln_done) e = launch_ln_modulate(x, m, (int)n, shift, scale, eps, y, PF_BF16, s);
  return e == hipSuccess ? PF_OK : hip_fail(e, "gemm_residual_ln launch");
}

extern "C" pf_status pf_gemm_qkv_splice(const void* a, int64_t lda, const void* w, const float* bias, int64_t m,
                                        int64_t hidden, void* q, int64_t ldq, const pf_kv_view* kv,
                                        int64_t row_offset, void* workspace, uint64_t workspace_bytes, void* stream) {
  pf_status st = validate_kv_view(kv, "gemm_qkv_splice");
  if (st != PF_OK) return st;
  if (kv->dtype != PF_BF16) return fail(PF_ERR_UNSUPPORTED, "gemm_qkv_splice: bf16 only");
  if (kv->v_layout != PF_LAYOUT_K8) return fail(PF_ERR_UNSUPPORTED, "gemm_qkv_splice: V must use the K8 layout");
  if (hidden <= 0 || hidden % 64 != 0) return fail(PF_ERR_UNSUPPORTED, "gemm_qkv_splice: hidden %% 64 != 0");
  if (kv->row_elems != hidden || kv->k_ld != hidden)
    return fail(PF_ERR_INVALID_ARG, "gemm_qkv_splice: buffer row_elems and k_ld must equal hidden");
  if (m < 0 || row_offset < 0 || row_offset + m > kv->rows)
    return fail(PF_ERR_INVALID_ARG, "gemm_qkv_splice: rows [%lld, %lld) outside the buffer", (long long)row_offset,
                (long long)(row_offset + m));
  if (!a || !w || !bias || !q) return fail(PF_ERR_INVALID_ARG, "gemm_qkv_splice: null pointer");
  if (lda < hidden || lda % 8 != 0 || ldq < hidden || ldq % 4 != 0)
    return fail(PF_ERR_INVALID_ARG, "gemm_qkv_splice: bad lda or ldq");
  if (!aligned16(a) || !aligned16(w) || !aligned16(bias) || !aligned16(q) || !aligned16(kv->k) || !aligned16(kv->v))
    return fail(PF_ERR_INVALID_ARG, "gemm_qkv_splice: pointers must be 16-byte aligned");
  if (workspace && !aligned16(workspace))
    return fail(PF_ERR_INVALID_ARG, "gemm_qkv_splice: workspace must be 16-byte aligned");
  if ((st = check_device()) != PF_OK) return st;
  const QkvSplice sp{kv->k, kv->v, row_offset, hidden, m > 0 ? m : 1, 0, 0};
  hipError_t e = launch_gemm(a, lda, w, bias, m, 3 * hidden, hidden, kEpiQkvSplice, q, ldq, nullptr, PF_BF16,
                             workspace, workspace ? (size_t)workspace_bytes : 0, (hipStream_t)stream, &sp);
  return e == hipSuccess ? PF_OK : hip_fail(e, "gemm_qkv_splice launch");
}

extern "C" pf_status pf_qk_norm_rope(void* q, int64_t ldq, const pf_kv_view* kv, int64_t row_offset, int64_t rows,
                                     int32_t heads, int32_t head_dim, const float* q_gamma, const float* k_gamma,
                                     const float* angles, uint32_t flags, void* stream) {
  pf_status st = validate_kv_view(kv, "qk_norm_rope");
  if (st != PF_OK) return st;
  if (kv->dtype != PF_BF16) return fail(PF_ERR_UNSUPPORTED, "qk_norm_rope: bf16 only");
  if (flags & ~(PF_STAGE_QK_NORM | PF_STAGE_ROPE)) return fail(PF_ERR_INVALID_ARG, "qk_norm_rope: bad flags");
  if (head_dim != 64 && head_dim != 72 && head_dim != 128)
    return fail(PF_ERR_UNSUPPORTED, "qk_norm_rope: head_dim %d not in {64, 72, 128}", head_dim);
  if (heads <= 0 || kv->row_elems != (int64_t)heads * head_dim)
    return fail(PF_ERR_INVALID_ARG, "qk_norm_rope: kv row_elems != heads * head_dim");
  if (rows < 0 || row_offset < 0 || row_offset + rows > kv->rows)
    return fail(PF_ERR_INVALID_ARG, "qk_norm_rope: rows [%lld, %lld) outside the buffer", (long long)row_offset,
                (long long)(row_offset + rows));
  if (kv->row_elems > kMaxHidden) return fail(PF_ERR_UNSUPPORTED, "qk_norm_rope: heads * head_dim > %d", kMaxHidden);
  if (!q) return fail(PF_ERR_INVALID_ARG, "qk_norm_rope: null q");
  if (ldq < kv->row_elems || (ldq & 7) || (kv->k_ld & 7) || !aligned16(q) || !aligned16(kv->k))
    return fail(PF_ERR_INVALID_ARG,
                "qk_norm_rope: ldq / k_ld must be multiples of 8 (ldq >= row_elems), q and K 16-byte aligned");
  const bool norm = (flags & PF_STAGE_QK_NORM) != 0, rope = (flags & PF_STAGE_ROPE) != 0;
  if ((norm && (!q_gamma || !k_gamma)) || (rope && !angles))
    return fail(PF_ERR_INVALID_ARG, "qk_norm_rope: null gamma or angles for the requested flags");
  if ((norm && (!aligned16(q_gamma) || !aligned16(k_gamma))) || (rope && !aligned16(angles)))
    return fail(PF_ERR_INVALID_ARG, "qk_norm_rope: gammas and angles must be 16-byte aligned");
  if (rows == 0 || flags == 0) return PF_OK;
  uintptr_t klo, khi;
  view_extent(kv, false, row_offset, rows, &klo, &khi);
  const uintptr_t q0 = (uintptr_t)q, q1 = q0 + (uintptr_t)(((rows - 1) * ldq + kv->row_elems) * 2);
  if (q0 < khi && klo < q1) return fail(PF_ERR_INVALID_ARG, "qk_norm_rope: q overlaps the K rows");
  if ((st = check_device()) != PF_OK) return st;
  hipError_t e = launch_qk_norm_rope(q, ldq, kv->k, kv->k_ld, 0, row_offset, rows, 1, heads, head_dim, q_gamma,
                                     k_gamma, angles, norm, rope, (hipStream_t)stream);
  return e == hipSuccess ? PF_OK : hip_fail(e, "qk_norm_rope launch");
}

extern "C" pf_status pf_gemm_workspace_size(int64_t m, int64_t n, int64_t k, uint64_t* bytes) {
  if (!bytes) return fail(PF_ERR_INVALID_ARG, "gemm_workspace_size: null out");
  if (m < 0 || n <= 0 || k <= 0) return fail(PF_ERR_INVALID_ARG, "gemm_workspace_size: bad sizes");
  pf_status st = check_device();   // the plan depends on the device's CU count
  if (st != PF_OK) return st;
  *bytes = gemm_workspace_bytes(m, n, k);
  return PF_OK;
}

extern "C" pf_status pf_attention(const void* q, int64_t ldq, const pf_kv_view* kv, int64_t seq_kv, int64_t rows,
                                  int32_t heads, int32_t head_dim, void* o, int64_t ldo, void* workspace,
                                  uint64_t workspace_bytes, void* stream) {
  pf_status st = validate_attention(q, ldq, kv, seq_kv, rows, heads, head_dim, o, ldo);
  if (st != PF_OK) return st;
  if (workspace && !aligned16(workspace)) return fail(PF_ERR_INVALID_ARG, "attention: workspace must be 16-byte aligned");
  if ((st = check_device()) != PF_OK) return st;
  hipError_t e = launch_attention(q, ldq, kv->k, kv->k_ld, kv->v, kv->v_ld, kv->v_layout, kv->row_elems, seq_kv,
                                  rows, heads, head_dim, o, ldo, kv->dtype, workspace,
                                  workspace ? (size_t)workspace_bytes : 0, (hipStream_t)stream);
  return e == hipSuccess ? PF_OK : hip_fail(e, "attention launch");
}

extern "C" pf_status pf_attention_noalloc(const void* q, int64_t ldq, const pf_kv_view* kv, int64_t seq_kv,
                                          int64_t rows, int32_t heads, int32_t head_dim, void* o, int64_t ldo,
                                          void* stream) {
  pf_status st = validate_attention(q, ldq, kv, seq_kv, rows, heads, head_dim, o, ldo);
  if (st != PF_OK) return st;
  if ((st = check_device()) != PF_OK) return st;
  // the split pf_attention would choose with a workspace of pf_attention_workspace_size bytes
  const size_t need = attention_split_workspace_bytes(rows, seq_kv, kv->row_elems, heads, head_dim, kv->dtype);
  if (need > kStaticScratchBytes)
    return fail(PF_ERR_UNSUPPORTED,
                "attention_noalloc: this launch's key-range split needs %zu bytes of scratch, more than the "
                "library's static %zu bytes (use pf_attention with a workspace)",
                need, kStaticScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = static_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e, "attention_noalloc: static scratch address");
  }
  const hipError_t e = launch_attention(q, ldq, kv->k, kv->k_ld, kv->v, kv->v_ld, kv->v_layout, kv->row_elems, seq_kv,
                                        rows, heads, head_dim, o, ldo, kv->dtype, ws, need, (hipStream_t)stream);
  return e == hipSuccess ? PF_OK : hip_fail(e, "attention_noalloc launch");
}

extern "C" pf_status pf_attention_workspace_size(int64_t rows, int32_t heads, int32_t head_dim, uint64_t* bytes) {
  if (!bytes) return fail(PF_ERR_INVALID_ARG, "attention_workspace_size: null out");
  if (rows < 0 || heads <= 0 || head_dim <= 0) return fail(PF_ERR_INVALID_ARG, "attention_workspace_size: bad sizes");
  *bytes = attention_workspace_bytes(rows, (int64_t)heads * head_dim, heads, kMaxAttnSplit);
  return PF_OK;
}

extern "C" pf_status pf_adaln(const float* cond, const void* w_ada, const float* b_ada, int32_t hidden, float* mod,
                              int32_t dtype, void* stream) {
  if (!dtype_ok(dtype)) return fail(PF_ERR_INVALID_ARG, "adaln: bad dtype");
  if (hidden <= 0 || hidden % 8 != 0 || hidden > 16384)
    return fail(PF_ERR_UNSUPPORTED, "adaln: hidden must be a positive multiple of 8 <= 16384");
  if (!cond || !w_ada || !b_ada || !mod) return fail(PF_ERR_INVALID_ARG, "adaln: null pointer");
  if (!aligned16(w_ada)) return fail(PF_ERR_INVALID_ARG, "adaln: w_ada must be 16-byte aligned");
  pf_status st = check_device();
  if (st != PF_OK) return st;
  hipError_t e = launch_adaln(cond, w_ada, b_ada, hidden, mod, dtype, (hipStream_t)stream);
  return e == hipSuccess ? PF_OK : hip_fail(e, "adaln launch");
}

static hipError_t splice_views(const pf_kv_view* dst, const pf_kv_view* src, int64_t offset, int64_t len,
                               hipStream_t s) {
  KVDesc d[2] = {{dst->k, dst->k_ld, PF_LAYOUT_ROWS}, {dst->v, dst->v_ld, dst->v_layout}};
  KVDesc sr[2] = {{src->k, src->k_ld, PF_LAYOUT_ROWS}, {src->v, src->v_ld, src->v_layout}};
  return launch_splice(d, sr, dst->row_elems, offset, len, (int)dtype_size(dst->dtype), s);
}

extern "C" pf_status kvbuf_splice(const pf_kv_view* dst, const pf_kv_view* src, int64_t offset, int64_t len,
                                  void* stream) {
  pf_status st = validate_splice(dst, src, offset, len);
  if (st != PF_OK) return st;
  if (len == 0) return PF_OK;
  if ((st = check_device()) != PF_OK) return st;
  hipError_t e = splice_views(dst, src, offset, len, (hipStream_t)stream);
  return e == hipSuccess ? PF_OK : hip_fail(e, "kvbuf_splice launch");
}

// ------------------------------------------------------------------------------------
// the stage
// ------------------------------------------------------------------------------------
// One stream's parameters of a layer (the image stream; with PF_STAGE_DUAL_STREAM also the
// text stream) and the modulation computed from them for the current condition.
struct WeightSet {
  void *w_qkv, *w_o, *w1, *w2, *w_ada;
  float *b_qkv, *b_o, *b1, *b2, *b_ada;
  float *q_norm, *k_norm;   // [d] each (PF_STAGE_QK_NORM)
  float* mod;               // [batch][6h]: shift1, scale1, gate1, shift2, scale2, gate2 per sample
  bool loaded;
};

struct LayerMem {
  WeightSet img, txt;   // txt is used only with PF_STAGE_DUAL_STREAM
  void *k, *v;  // sample 0's K and V buffers; sample b's are b * kv_sample_bytes further on
};

struct pf_stage {
  pf_stage_config cfg;
  int device;
  int64_t h, rh, s_kv, s_alloc, patch_rows;
  int64_t batch;            // samples sharing the weights (each with its cond, rows and buffers)
  size_t kv_sample_bytes;   // distance between two samples' K (or V) buffers of one layer
  size_t es;
  void* wmem = nullptr;
  void* kvmem = nullptr;
  void* scratch = nullptr;
  float* modmem = nullptr;
  float* rope = nullptr;     // [s_kv, d/2] rotation angles (PF_STAGE_ROPE)
  bool rope_set = false;
  void *h1, *qkv, *o, *u;
  int64_t ld_o, ld_u;        // row strides of o and u (the parallel block keeps [o, u] side by side)
  int n_mod;                 // modulation vectors per sample: 6 (DiT block) or 3 (parallel block)
  size_t set_bytes = 0;      // distance between two consecutive weight sets (layer by layer, stream by stream)
  void* attn_ws = nullptr;   // key-range split partials of the patch attention
  size_t attn_ws_bytes = 0;
  void* gemm_ws = nullptr;   // k-split partials of the projections
  size_t gemm_ws_bytes = 0;
  std::vector<LayerMem> layers;
  bool cond_set = false;
  bool broken = false;   // a HIP call failed: every later call returns PF_ERR_HIP
  // stage_profile_begin / _end: event pairs recorded around attention launches
  std::vector<hipEvent_t> prof_ev;
  size_t prof_used = 0;
  bool prof_on = false;
};

static size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

static pf_status validate_config(const pf_stage_config* c) {
  if (!c) return fail(PF_ERR_INVALID_ARG, "stage_create: null config");
  if (c->num_layers < 1) return fail(PF_ERR_INVALID_ARG, "stage_create: num_layers < 1");
  if (c->heads < 1) return fail(PF_ERR_INVALID_ARG, "stage_create: heads < 1");
  if (c->head_dim != 64 && c->head_dim != 72 && c->head_dim != 128)
    return fail(PF_ERR_UNSUPPORTED, "stage_create: head_dim %d not in {64, 72, 128}", c->head_dim);
  if ((int64_t)c->hidden != (int64_t)c->heads * c->head_dim)
    return fail(PF_ERR_INVALID_ARG, "stage_create: hidden %d != heads * head_dim", c->hidden);
  if (c->mlp_ratio < 0 || c->mlp_ratio > 16) return fail(PF_ERR_INVALID_ARG, "stage_create: mlp_ratio out of range");
  if (c->num_patches < 1) return fail(PF_ERR_INVALID_ARG, "stage_create: num_patches < 1");
  if (c->seq_img < 1 || c->seq_txt < 0) return fail(PF_ERR_INVALID_ARG, "stage_create: bad sequence lengths");
  if (c->seq_img % c->num_patches != 0)
    return fail(PF_ERR_INVALID_ARG, "stage_create: seq_img %% num_patches != 0");
  if (!dtype_ok(c->dtype)) return fail(PF_ERR_INVALID_ARG, "stage_create: bad dtype");
  if (c->gelu != PF_GELU_TANH && c->gelu != PF_GELU_ERF) return fail(PF_ERR_INVALID_ARG, "stage_create: bad gelu");
  if (!(c->ln_eps > 0.f) || !std::isfinite(c->ln_eps)) return fail(PF_ERR_INVALID_ARG, "stage_create: bad ln_eps");
  if (c->flags & ~(PF_STAGE_QK_NORM | PF_STAGE_DUAL_STREAM | PF_STAGE_ROPE | PF_STAGE_PARALLEL))
    return fail(PF_ERR_INVALID_ARG, "stage_create: unknown flags 0x%x", c->flags);
  if ((c->flags & PF_STAGE_PARALLEL) && (c->flags & PF_STAGE_DUAL_STREAM))
    return fail(PF_ERR_UNSUPPORTED, "stage_create: the parallel block is single-stream (no PF_STAGE_DUAL_STREAM)");
  if (c->flags != 0 && c->dtype != PF_BF16)
    return fail(PF_ERR_UNSUPPORTED, "stage_create: block options need a bf16 stage");
  if ((c->flags & PF_STAGE_DUAL_STREAM) && c->seq_txt < 1)
    return fail(PF_ERR_INVALID_ARG, "stage_create: PF_STAGE_DUAL_STREAM needs a text prefix (seq_txt >= 1)");
  if (c->batch < 0 || c->batch > PF_MAX_STAGE_BATCH)
    return fail(PF_ERR_INVALID_ARG, "stage_create: batch %d outside [0, %d]", c->batch, PF_MAX_STAGE_BATCH);
  if (c->hidden > kMaxHidden) return fail(PF_ERR_UNSUPPORTED, "stage_create: hidden > %d", kMaxHidden);
  if (c->dtype == PF_BF16 && c->hidden % 64 != 0)
    return fail(PF_ERR_UNSUPPORTED, "stage_create: bf16 stages need hidden %% 64 == 0");
  if (c->dtype == PF_FP32 && c->hidden % 8 != 0)
    return fail(PF_ERR_UNSUPPORTED, "stage_create: hidden %% 8 != 0");
  if (c->seq_txt + c->seq_img > ((int64_t)1 << 31))
    return fail(PF_ERR_UNSUPPORTED, "stage_create: sequence too long");
  return PF_OK;
}

static void free_stage_mem(pf_stage* st) {
  if (st->wmem) (void)hipFree(st->wmem);
  if (st->kvmem) (void)hipFree(st->kvmem);
  if (st->scratch) (void)hipFree(st->scratch);
  if (st->modmem) (void)hipFree(st->modmem);
  if (st->rope) (void)hipFree(st->rope);
  st->rope = nullptr;
  if (st->attn_ws) (void)hipFree(st->attn_ws);
  if (st->gemm_ws) (void)hipFree(st->gemm_ws);
  st->attn_ws = st->gemm_ws = nullptr;
  st->wmem = st->kvmem = st->scratch = nullptr;
  st->modmem = nullptr;
}

extern "C" pf_status stage_create(const pf_stage_config* cfg, pf_stage** out) {
  if (!out) return fail(PF_ERR_INVALID_ARG, "stage_create: null out");
  *out = nullptr;
  pf_status vs = validate_config(cfg);
  if (vs != PF_OK) return vs;
  if ((vs = check_device()) != PF_OK) return vs;

  pf_stage* st = new (std::nothrow) pf_stage();
  if (!st) return fail(PF_ERR_OOM, "stage_create: host allocation failed");
  st->cfg = *cfg;
  (void)hipGetDevice(&st->device);
  st->h = cfg->hidden;
  st->rh = (int64_t)cfg->mlp_ratio * cfg->hidden;
  st->s_kv = cfg->seq_txt + cfg->seq_img;
  st->s_alloc = (int64_t)round_up((size_t)st->s_kv, 64);   // K8 groups and key tiles never leave the allocation
  st->patch_rows = cfg->seq_img / cfg->num_patches;
  st->batch = cfg->batch > 0 ? cfg->batch : 1;
  st->es = dtype_size(cfg->dtype);
  const int64_t h = st->h, rh = st->rh, L = cfg->num_layers, nb = st->batch;
  const size_t es = st->es;
  const int64_t n_sets = (cfg->flags & PF_STAGE_DUAL_STREAM) ? 2 : 1;   // weight sets (streams) per layer
  const int64_t d = cfg->head_dim;

  // weights: matrices then fp32 biases, each 256-byte aligned, then the two norm scales
  // (w_qkv, w_o, w1, w2, w_ada; the parallel block has no w_o, a wider w2 and 3 modulation vectors)
  const bool par = (cfg->flags & PF_STAGE_PARALLEL) != 0;
  st->n_mod = par ? 3 : 6;
  const int64_t k2 = par ? h + rh : rh;   // input width of the second MLP matrix
  const size_t mats[5] = {(size_t)(3 * h * h), par ? 0 : (size_t)(h * h), (size_t)(rh * h), (size_t)(h * k2),
                          (size_t)(st->n_mod * h * h)};
  const size_t biases[5] = {(size_t)(3 * h), par ? 0 : (size_t)h, (size_t)rh, (size_t)h, (size_t)(st->n_mod * h)};
  size_t per_set = 0;
  for (int i = 0; i < 5; ++i) per_set += round_up(mats[i] * es, 256) + round_up(biases[i] * 4, 256);
  const size_t norm_bytes = round_up((size_t)d * 4, 256);
  per_set += 2 * norm_bytes;
  const size_t per_layer = per_set * (size_t)n_sets;
  st->set_bytes = per_set;
  const size_t rope_bytes = (cfg->flags & PF_STAGE_ROPE) ? (size_t)(st->s_kv * (d / 2)) * 4 : 0;
  const size_t kv_mat = round_up((size_t)(st->s_alloc * h) * es, 256);
  st->kv_sample_bytes = 2 * kv_mat;   // per layer: K0, V0, K1, V1, ...
  // scratch for a micro-step of up to s_kv rows of every sample
  st->ld_o = par ? h + rh : h;
  st->ld_u = par ? h + rh : rh;
  const size_t scr_h = round_up((size_t)(nb * st->s_alloc * h) * es, 256);
  const size_t scr_o = round_up((size_t)(nb * st->s_alloc * st->ld_o) * es, 256);
  const size_t scr_qkv = round_up((size_t)(nb * st->s_alloc * 3 * h) * es, 256);
  const size_t scr_u = par ? 0 : round_up((size_t)(nb * st->s_alloc * (rh > 0 ? rh : 1)) * es, 256);

  // split partials for a patch or the text prefix of every sample (the warm-up pass fills the
  // GPU unsplit)
  const int64_t split_rows = nb * std::max<int64_t>(st->patch_rows, cfg->seq_txt);
  st->attn_ws_bytes = cfg->dtype == PF_BF16 ? attention_workspace_bytes(split_rows, h, cfg->heads, kMaxAttnSplit) : 0;
  // k-split partials for the projections of a patch or the text prefix of all samples
  st->gemm_ws_bytes = 0;
  if (cfg->dtype == PF_BF16) {
    const int64_t shapes[4][2] = {{3 * h, h}, {par ? 0 : h, h}, {rh, h}, {h, k2}};
    for (const int64_t rows : {nb * st->patch_rows, nb * cfg->seq_txt}) {
      if (rows <= 0) continue;
      for (const auto& nk : shapes)
        if (nk[0] > 0 && nk[1] > 0) st->gemm_ws_bytes = std::max(st->gemm_ws_bytes, gemm_workspace_bytes(rows, nk[0], nk[1]));
    }
  }

  hipError_t e;
  if ((e = hipMalloc(&st->wmem, per_layer * L)) != hipSuccess ||
      (st->attn_ws_bytes && (e = hipMalloc(&st->attn_ws, st->attn_ws_bytes)) != hipSuccess) ||
      (st->gemm_ws_bytes && (e = hipMalloc(&st->gemm_ws, st->gemm_ws_bytes)) != hipSuccess) ||
      (e = hipMalloc(&st->kvmem, 2 * kv_mat * L * nb)) != hipSuccess ||
      (e = hipMalloc(&st->scratch, scr_h + scr_o + scr_qkv + scr_u)) != hipSuccess ||
      (e = hipMalloc((void**)&st->modmem, sizeof(float) * 6 * h * L * nb * n_sets)) != hipSuccess ||
      (rope_bytes && (e = hipMalloc((void**)&st->rope, rope_bytes)) != hipSuccess)) {
    free_stage_mem(st);
    delete st;
    (void)hipGetLastError();
    return e == hipErrorOutOfMemory ? fail(PF_ERR_OOM, "stage_create: device allocation failed")
                                    : hip_fail(e, "stage_create: hipMalloc");
  }
  // zero the KV buffers (including the padding rows past seq_kv) once, synchronously
  if ((e = hipMemset(st->kvmem, 0, 2 * kv_mat * L * nb)) != hipSuccess ||
      (e = hipMemset(st->modmem, 0, sizeof(float) * 6 * h * L * nb * n_sets)) != hipSuccess ||
      (e = hipDeviceSynchronize()) != hipSuccess) {
    free_stage_mem(st);
    delete st;
    return hip_fail(e, "stage_create: hipMemset");
  }
  char* wp = (char*)st->wmem;
  char* kp = (char*)st->kvmem;
  st->layers.resize(L);
  for (int64_t l = 0; l < L; ++l) {
    LayerMem& lm = st->layers[l];
    for (int64_t set = 0; set < 2; ++set) {
      WeightSet& ws = set == 0 ? lm.img : lm.txt;
      ws = WeightSet{};
      if (set >= n_sets) continue;
      void** mp[5] = {&ws.w_qkv, &ws.w_o, &ws.w1, &ws.w2, &ws.w_ada};
      float** bp[5] = {&ws.b_qkv, &ws.b_o, &ws.b1, &ws.b2, &ws.b_ada};
      for (int i = 0; i < 5; ++i) {
        *mp[i] = wp;
        wp += round_up(mats[i] * es, 256);
        *bp[i] = (float*)wp;
        wp += round_up(biases[i] * 4, 256);
      }
      ws.q_norm = (float*)wp;
      wp += norm_bytes;
      ws.k_norm = (float*)wp;
      wp += norm_bytes;
      ws.mod = st->modmem + 6 * h * nb * (l * n_sets + set);
    }
    lm.k = kp;
    lm.v = kp + kv_mat;
    kp += 2 * kv_mat * nb;
  }
  char* sp = (char*)st->scratch;
  st->h1 = sp;
  sp += scr_h;
  st->o = sp;
  sp += scr_o;
  st->qkv = sp;
  sp += scr_qkv;
  st->u = par ? (char*)st->o + h * es : sp;
  *out = st;
  return PF_OK;
}

static void free_profile_events(pf_stage* st) {
  for (hipEvent_t ev : st->prof_ev) (void)hipEventDestroy(ev);
  st->prof_ev.clear();
  st->prof_used = 0;
  st->prof_on = false;
}

extern "C" pf_status stage_destroy(pf_stage* st) {
  if (!st) return PF_OK;
  free_profile_events(st);
  free_stage_mem(st);
  delete st;
  return PF_OK;
}

static pf_status check_stage(pf_stage* st, const char* who) {
  if (!st) return fail(PF_ERR_INVALID_ARG, "%s: null stage", who);
  if (st->broken) return fail(PF_ERR_HIP, "%s: an earlier HIP call on this stage failed", who);
  (void)hipGetLastError();
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != st->device) return fail(PF_ERR_INVALID_ARG, "%s: current device %d is not the stage's device %d", who,
                                     dev, st->device);
  return PF_OK;
}

static pf_status stage_hip_fail(pf_stage* st, hipError_t e, const char* what) {
  st->broken = true;
  return hip_fail(e, what);
}

static pf_status load_set(pf_stage* st, int32_t layer, const pf_layer_weights* w, bool txt, void* stream,
                          const char* who) {
  pf_status s = check_stage(st, who);
  if (s != PF_OK) return s;
  if (layer < 0 || layer >= st->cfg.num_layers) return fail(PF_ERR_INVALID_ARG, "%s: bad layer %d", who, layer);
  if (!w) return fail(PF_ERR_INVALID_ARG, "%s: null weights", who);
  const bool mlp = st->rh > 0;
  const bool qkn = (st->cfg.flags & PF_STAGE_QK_NORM) != 0;
  const bool par = (st->cfg.flags & PF_STAGE_PARALLEL) != 0;
  if (!w->w_qkv || !w->b_qkv || (!par && (!w->w_o || !w->b_o)) || !w->w_ada || !w->b_ada ||
      (mlp && (!w->w1 || !w->b1)) || ((mlp || par) && (!w->w2 || !w->b2)) || (qkn && (!w->q_norm || !w->k_norm)))
    return fail(PF_ERR_INVALID_ARG, "%s: null weight pointer", who);
  const int64_t h = st->h, rh = st->rh, d = st->cfg.head_dim, k2 = par ? h + rh : rh, nm = st->n_mod;
  const size_t es = st->es;
  WeightSet& lm = txt ? st->layers[layer].txt : st->layers[layer].img;
  struct Cp { void* dst; const void* src; size_t bytes; } cps[12] = {
      {lm.w_qkv, w->w_qkv, (size_t)(3 * h * h) * es}, {lm.b_qkv, w->b_qkv, (size_t)(3 * h) * 4},
      {lm.w_o, w->w_o, par ? 0 : (size_t)(h * h) * es}, {lm.b_o, w->b_o, par ? 0 : (size_t)h * 4},
      {lm.w1, w->w1, (size_t)(rh * h) * es},          {lm.b1, w->b1, (size_t)rh * 4},
      {lm.w2, w->w2, (size_t)(h * k2) * es},          {lm.b2, w->b2, (size_t)h * 4},
      {lm.w_ada, w->w_ada, (size_t)(nm * h * h) * es}, {lm.b_ada, w->b_ada, (size_t)(nm * h) * 4},
      {lm.q_norm, w->q_norm, (size_t)d * 4},          {lm.k_norm, w->k_norm, (size_t)d * 4}};
  for (int i = 0; i < 12; ++i) {
    const Cp& c = cps[i];
    if (c.bytes == 0 || (!mlp && i >= 4 && i < (par ? 6 : 8)) || (!qkn && i >= 10)) continue;   // unused parameters
    hipError_t e = hipMemcpyAsync(c.dst, c.src, c.bytes, hipMemcpyDeviceToDevice, (hipStream_t)stream);
    if (e != hipSuccess) return stage_hip_fail(st, e, "stage_load_weights: hipMemcpyAsync");
  }
  lm.loaded = true;
  return PF_OK;
}

extern "C" pf_status stage_load_weights(pf_stage* st, int32_t layer, const pf_layer_weights* w, void* stream) {
  return load_set(st, layer, w, false, stream, "stage_load_weights");
}

extern "C" pf_status stage_load_text_weights(pf_stage* st, int32_t layer, const pf_layer_weights* w, void* stream) {
  if (st && !(st->cfg.flags & PF_STAGE_DUAL_STREAM))
    return fail(PF_ERR_INVALID_ARG, "stage_load_text_weights: the stage was created without PF_STAGE_DUAL_STREAM");
  return load_set(st, layer, w, true, stream, "stage_load_text_weights");
}

extern "C" pf_status stage_set_rope(pf_stage* st, const float* angles, void* stream) {
  pf_status s = check_stage(st, "stage_set_rope");
  if (s != PF_OK) return s;
  if (!(st->cfg.flags & PF_STAGE_ROPE))
    return fail(PF_ERR_INVALID_ARG, "stage_set_rope: the stage was created without PF_STAGE_ROPE");
  if (!angles) return fail(PF_ERR_INVALID_ARG, "stage_set_rope: null angles");
  if ((uintptr_t)angles & 3u) return fail(PF_ERR_INVALID_ARG, "stage_set_rope: angles must be 4-byte aligned");
  if ((uintptr_t)angles < (uintptr_t)st->rope + (st->s_kv * (st->cfg.head_dim / 2)) * sizeof(float) &&
      (uintptr_t)st->rope < (uintptr_t)angles + (st->s_kv * (st->cfg.head_dim / 2)) * sizeof(float))
    return fail(PF_ERR_INVALID_ARG, "stage_set_rope: angles overlap the stage's table");
  const size_t bytes = (size_t)(st->s_kv * (st->cfg.head_dim / 2)) * sizeof(float);
  hipError_t e = hipMemcpyAsync(st->rope, angles, bytes, hipMemcpyDeviceToDevice, (hipStream_t)stream);
  if (e != hipSuccess) return stage_hip_fail(st, e, "stage_set_rope: hipMemcpyAsync");
  st->rope_set = true;
  return PF_OK;
}

static bool dual(const pf_stage* st) { return (st->cfg.flags & PF_STAGE_DUAL_STREAM) != 0; }

static pf_status check_loaded(pf_stage* st, const char* who) {
  for (int l = 0; l < st->cfg.num_layers; ++l) {
    if (!st->layers[l].img.loaded) return fail(PF_ERR_STATE, "%s: layer %d weights not loaded", who, l);
    if (dual(st) && !st->layers[l].txt.loaded)
      return fail(PF_ERR_STATE, "%s: layer %d text-stream weights not loaded", who, l);
  }
  if ((st->cfg.flags & PF_STAGE_ROPE) && !st->rope_set) return fail(PF_ERR_STATE, "%s: stage_set_rope not called", who);
  return PF_OK;
}

// Every layer's (and stream's) modulation for every sample in one launch: the weight sets lie
// set_bytes apart in the weight allocation, their modulation vectors 6h * batch floats apart.
static pf_status set_cond_impl(pf_stage* st, const float* cond, hipStream_t s) {
  const int n_sets = (int)st->layers.size() * (dual(st) ? 2 : 1);
  const WeightSet& first = st->layers[0].img;
  const int64_t h = st->h;
  hipError_t e = launch_adaln_batch(cond, h, (int)st->batch, first.w_ada, (int64_t)(st->set_bytes / st->es),
                                    first.b_ada, (int64_t)(st->set_bytes / sizeof(float)), n_sets, (int)h, first.mod,
                                    6 * h * st->batch, 6 * h, st->cfg.dtype, s, st->n_mod);
  if (e != hipSuccess) return stage_hip_fail(st, e, "stage_set_cond: adaln launch");
  st->cond_set = true;
  return PF_OK;
}

extern "C" pf_status stage_set_cond(pf_stage* st, const float* cond, void* stream) {
  pf_status s = check_stage(st, "stage_set_cond");
  if (s != PF_OK) return s;
  if (!cond) return fail(PF_ERR_INVALID_ARG, "stage_set_cond: null cond");
  if ((s = check_loaded(st, "stage_set_cond")) != PF_OK) return s;
  return set_cond_impl(st, cond, (hipStream_t)stream);
}

// Buffer rows [off, off + n) of every sample through all layers.  Sample b's rows of x (fp32,
// updated in place) are [x + b * x_stride, + n * h).  With PF_STAGE_DUAL_STREAM the rows split
// at seq_txt into a text part and an image part, each with its own weight set; otherwise there
// is one part.  Inside a part the samples' rows are stacked (scratch row srow + b * n_part + i),
// so every projection runs once over batch * n_part rows with shared weights, while each sample
// keeps its own modulation, gates, K/V buffers and attention.  Attention is joint: every part's
// K/V rows are in the buffers before any row attends.
namespace {
struct Part {
  int64_t off, n;        // buffer rows [off, off + n)
  int64_t srow;          // first scratch row (batch-stacked)
  float* x;              // sample 0's first row of x
  const WeightSet* (*pick)(const LayerMem&);
};
const WeightSet* pick_img(const LayerMem& lm) { return &lm.img; }
const WeightSet* pick_txt(const LayerMem& lm) { return &lm.txt; }
}  // namespace

static pf_status run_rows(pf_stage* st, int64_t off, int64_t n, float* x, int64_t x_stride, hipStream_t s) {
  const int64_t h = st->h, rh = st->rh, nb = st->batch;
  const int dt = st->cfg.dtype;
  const size_t es = st->es;
  const float eps = st->cfg.ln_eps;
  const int gelu_epi = st->cfg.gelu == PF_GELU_ERF ? kEpiGeluErf : kEpiGeluTanh;
  const int64_t kv_stride = (int64_t)(st->kv_sample_bytes / es);   // elements between samples' buffers
  const bool qk_norm = (st->cfg.flags & PF_STAGE_QK_NORM) != 0, rope = (st->cfg.flags & PF_STAGE_ROPE) != 0;
  const bool par = (st->cfg.flags & PF_STAGE_PARALLEL) != 0;
  const int64_t ld_o = st->ld_o, ld_u = st->ld_u;
  Part parts[2];
  int n_parts = 0;
  const int64_t split = dual(st) ? std::min(std::max(st->cfg.seq_txt - off, (int64_t)0), n) : 0;
  if (split > 0) parts[n_parts++] = Part{off, split, 0, x, pick_txt};
  if (split < n) parts[n_parts++] = Part{off + split, n - split, nb * split, x + split * h, pick_img};
  char* const qkv = (char*)st->qkv;
  char* const h1 = (char*)st->h1;
  char* const o = (char*)st->o;
  // a k-split residual product whose reduce pass also ran the next LayerNorm leaves that
  // part's h1 ready for the next layer
  bool ln1_ready[2] = {false, false};
  const int n_layers = (int)st->layers.size();
  for (int li = 0; li < n_layers; ++li) {
    LayerMem& lm = st->layers[li];
    const LayerMem* next = li + 1 < n_layers ? &st->layers[li + 1] : nullptr;
    hipError_t e;
    const int v_layout = dt == PF_BF16 ? kLayoutK8 : kLayoutRows;
    for (int pi = 0; pi < n_parts; ++pi) {
      const Part& p = parts[pi];
      const WeightSet& ws = *p.pick(lm);
      const RowGroups xg{p.n, x_stride, 6 * h};   // x rows and modulation vectors per sample
      const int64_t rows = nb * p.n;
      char* h1p = h1 + (size_t)(p.srow * h) * es;
      char* qkvp = qkv + (size_t)(p.srow * 3 * h) * es;
      if (!ln1_ready[pi] &&
          (e = launch_ln_modulate(p.x, rows, (int)h, ws.mod, ws.mod + h, eps, h1p, dt, s, &xg)) != hipSuccess)
        return stage_hip_fail(st, e, "ln_modulate");
      ln1_ready[pi] = false;
      if (dt == PF_BF16) {
        // QKV projection with the splice in its epilogue: Q to the scratch, each sample's fresh K
        // and V straight into rows [p.off, p.off + p.n) of its own buffer (no other row changes)
        const QkvSplice sp{lm.k, lm.v, p.off, h, p.n, kv_stride, kv_stride};
        if ((e = launch_gemm(h1p, h, ws.w_qkv, ws.b_qkv, rows, 3 * h, h, kEpiQkvSplice, qkvp, 3 * h, nullptr, dt,
                             st->gemm_ws, st->gemm_ws_bytes, s, &sp)) != hipSuccess)
          return stage_hip_fail(st, e, "qkv gemm + kv splice");
        // QK-RMSNorm and rotary embedding in place: Q rows in the scratch, K rows in the buffers
        if ((qk_norm || rope) &&
            (e = launch_qk_norm_rope(qkvp, 3 * h, lm.k, h, kv_stride, p.off, p.n, nb, st->cfg.heads,
                                     st->cfg.head_dim, ws.q_norm, ws.k_norm, st->rope, qk_norm, rope, s)) != hipSuccess)
          return stage_hip_fail(st, e, "qk norm / rope");
        // parallel block: the MLP's first projection reads the same modulated rows; its GELU
        // output lands beside the attention output ([o, u] rows of width h + rh)
        if (par && rh > 0 &&
            (e = launch_gemm(h1p, h, ws.w1, ws.b1, rows, rh, h, gelu_epi, (char*)st->u + (size_t)(p.srow * ld_u) * es,
                             ld_u, nullptr, dt, st->gemm_ws, st->gemm_ws_bytes, s)) != hipSuccess)
          return stage_hip_fail(st, e, "mlp up gemm (parallel)");
      } else {
        if ((e = launch_gemm(h1p, h, ws.w_qkv, ws.b_qkv, rows, 3 * h, h, kEpiStore, qkvp, 3 * h, nullptr, dt,
                             st->gemm_ws, st->gemm_ws_bytes, s)) != hipSuccess)
          return stage_hip_fail(st, e, "qkv gemm");
        for (int64_t b = 0; b < nb; ++b) {
          const char* src_row = qkvp + (size_t)(b * p.n * 3 * h) * es;
          KVDesc dst[2] = {{(char*)lm.k + b * st->kv_sample_bytes, h, kLayoutRows},
                           {(char*)lm.v + b * st->kv_sample_bytes, h, kLayoutRows}};
          KVDesc src[2] = {{src_row + h * es, 3 * h, kLayoutRows}, {src_row + 2 * h * es, 3 * h, kLayoutRows}};
          if ((e = launch_splice(dst, src, h, p.off, p.n, (int)es, s)) != hipSuccess)
            return stage_hip_fail(st, e, "kv splice");
        }
      }
    }
    // one launch per part for every sample; each sample's queries attend over its own buffer
    for (int pi = 0; pi < n_parts; ++pi) {
      const Part& p = parts[pi];
      const bool timed = st->prof_on && st->prof_used + 2 <= st->prof_ev.size();
      if (timed && (e = hipEventRecord(st->prof_ev[st->prof_used], s)) != hipSuccess)
        return stage_hip_fail(st, e, "attention timing event");
      if ((e = launch_attention(qkv + (size_t)(p.srow * 3 * h) * es, 3 * h, lm.k, h, lm.v, h, v_layout, h, st->s_kv,
                                p.n, st->cfg.heads, st->cfg.head_dim, o + (size_t)(p.srow * ld_o) * es, ld_o, dt,
                                st->attn_ws, st->attn_ws_bytes, s, nb, kv_stride)) != hipSuccess)
        return stage_hip_fail(st, e, "attention");
      if (timed) {
        if ((e = hipEventRecord(st->prof_ev[st->prof_used + 1], s)) != hipSuccess)
          return stage_hip_fail(st, e, "attention timing event");
        st->prof_used += 2;
      }
    }
    for (int pi = 0; pi < n_parts; ++pi) {
      const Part& p = parts[pi];
      const WeightSet& ws = *p.pick(lm);
      const RowGroups xg{p.n, x_stride, 6 * h};
      const int64_t rows = nb * p.n;
      char* h1p = h1 + (size_t)(p.srow * h) * es;
      char* op = o + (size_t)(p.srow * ld_o) * es;
      char* up = (char*)st->u + (size_t)(p.srow * ld_u) * es;
      // the LayerNorm that follows a layer's last residual product: the next layer's first
      const WeightSet* nws = next ? p.pick(*next) : nullptr;
      const LnAfter ln_next{nws ? nws->mod : nullptr, nws ? nws->mod + h : nullptr, eps, h1p};
      if (par) {
        // x += gate * ([o, u] W2^T + b2): one product over the side-by-side rows
        if ((e = launch_gemm(op, ld_o, ws.w2, ws.b2, rows, h, h + rh, kEpiGatedResidual, p.x, h, ws.mod + 2 * h, dt,
                             st->gemm_ws, st->gemm_ws_bytes, s, nullptr, &xg, nws ? &ln_next : nullptr,
                             &ln1_ready[pi])) != hipSuccess)
          return stage_hip_fail(st, e, "linear2 gemm (parallel)");
        continue;
      }
      const LnAfter ln_mlp{ws.mod + 3 * h, ws.mod + 4 * h, eps, h1p};
      const LnAfter* ln_out = rh > 0 ? &ln_mlp : (nws ? &ln_next : nullptr);
      bool ln_done = false;
      if ((e = launch_gemm(op, h, ws.w_o, ws.b_o, rows, h, h, kEpiGatedResidual, p.x, h, ws.mod + 2 * h, dt,
                           st->gemm_ws, st->gemm_ws_bytes, s, nullptr, &xg, ln_out, &ln_done)) != hipSuccess)
        return stage_hip_fail(st, e, "out-proj gemm");
      if (rh == 0) ln1_ready[pi] = ln_done;
      if (rh > 0) {
        if (!ln_done &&
            (e = launch_ln_modulate(p.x, rows, (int)h, ws.mod + 3 * h, ws.mod + 4 * h, eps, h1p, dt, s, &xg)) !=
                hipSuccess)
          return stage_hip_fail(st, e, "ln_modulate (mlp)");
        if ((e = launch_gemm(h1p, h, ws.w1, ws.b1, rows, rh, h, gelu_epi, up, ld_u, nullptr, dt, st->gemm_ws,
                             st->gemm_ws_bytes, s)) != hipSuccess)
          return stage_hip_fail(st, e, "mlp up gemm");
        if ((e = launch_gemm(up, ld_u, ws.w2, ws.b2, rows, h, rh, kEpiGatedResidual, p.x, h, ws.mod + 5 * h, dt,
                             st->gemm_ws, st->gemm_ws_bytes, s, nullptr, &xg, nws ? &ln_next : nullptr,
                             &ln1_ready[pi])) != hipSuccess)
          return stage_hip_fail(st, e, "mlp down gemm");
      }
    }
  }
  return PF_OK;
}

// x_in / x_out: sample b's n rows at + b * x_stride elements.
static pf_status run_patch_impl(pf_stage* st, int64_t off, int64_t n, const float* x_in, float* x_out,
                                int64_t x_stride, hipStream_t s) {
  if (x_out != x_in) {
    const size_t row_bytes = (size_t)(n * st->h) * sizeof(float);
    hipError_t e = hipMemcpy2DAsync(x_out, (size_t)x_stride * sizeof(float), x_in, (size_t)x_stride * sizeof(float),
                                    row_bytes, (size_t)st->batch, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return stage_hip_fail(st, e, "stage_run_patch: hipMemcpy2DAsync");
  }
  return run_rows(st, off, n, x_out, x_stride, s);
}

extern "C" pf_status stage_run_patch(pf_stage* st, int64_t row_off, int64_t rows, const float* x_in, float* x_out,
                                     void* stream) {
  pf_status s = check_stage(st, "stage_run_patch");
  if (s != PF_OK) return s;
  if (row_off < 0 || rows < 1 || row_off + rows > st->s_kv)
    return fail(PF_ERR_INVALID_ARG, "stage_run_patch: rows [%lld, %lld) outside [0, %lld)", (long long)row_off,
                (long long)(row_off + rows), (long long)st->s_kv);
  if (!x_in || !x_out) return fail(PF_ERR_INVALID_ARG, "stage_run_patch: null x");
  if (!aligned16(x_in) || !aligned16(x_out)) return fail(PF_ERR_INVALID_ARG, "stage_run_patch: x must be 16-byte aligned");
  const size_t bytes = (size_t)(st->batch * rows * st->h) * sizeof(float);
  if (x_in != x_out && ranges_overlap(x_in, bytes, x_out, bytes))
    return fail(PF_ERR_INVALID_ARG, "stage_run_patch: x_in and x_out partially overlap");
  if ((s = check_loaded(st, "stage_run_patch")) != PF_OK) return s;
  if (!st->cond_set) return fail(PF_ERR_STATE, "stage_run_patch: stage_set_cond not called");
  return run_patch_impl(st, row_off, rows, x_in, x_out, rows * st->h, (hipStream_t)stream);
}

extern "C" pf_status stage_run_step(pf_stage* st, const float* x_in, float* x_out, const float* cond, uint32_t flags,
                                    void* stream) {
  pf_status s = check_stage(st, "stage_run_step");
  if (s != PF_OK) return s;
  if (!x_in || !x_out || !cond) return fail(PF_ERR_INVALID_ARG, "stage_run_step: null pointer");
  if (!aligned16(x_in) || !aligned16(x_out)) return fail(PF_ERR_INVALID_ARG, "stage_run_step: x must be 16-byte aligned");
  if (flags & ~PF_STEP_WARMUP) return fail(PF_ERR_INVALID_ARG, "stage_run_step: unknown flags");
  const size_t bytes = (size_t)(st->batch * st->s_kv * st->h) * sizeof(float);
  if (x_in != x_out && ranges_overlap(x_in, bytes, x_out, bytes))
    return fail(PF_ERR_INVALID_ARG, "stage_run_step: x_in and x_out partially overlap");
  if ((s = check_loaded(st, "stage_run_step")) != PF_OK) return s;
  hipStream_t hs = (hipStream_t)stream;
  if ((s = set_cond_impl(st, cond, hs)) != PF_OK) return s;
  // out of place: every row is copied once, then the micro-steps (disjoint rows) run in place
  if (x_out != x_in) {
    hipError_t e = hipMemcpyAsync(x_out, x_in, bytes, hipMemcpyDeviceToDevice, hs);
    if (e != hipSuccess) return stage_hip_fail(st, e, "stage_run_step: hipMemcpyAsync");
  }
  const int64_t h = st->h, xs = st->s_kv * h;   // sample b's rows start b * s_kv rows on
  if (flags & PF_STEP_WARMUP) return run_rows(st, 0, st->s_kv, x_out, xs, hs);
  if (st->cfg.seq_txt > 0 && (s = run_rows(st, 0, st->cfg.seq_txt, x_out, xs, hs)) != PF_OK) return s;
  for (int m = 0; m < st->cfg.num_patches; ++m) {
    const int64_t off = st->cfg.seq_txt + (int64_t)m * st->patch_rows;
    if ((s = run_rows(st, off, st->patch_rows, x_out + off * h, xs, hs)) != PF_OK) return s;
  }
  return PF_OK;
}

extern "C" pf_status stage_profile_begin(pf_stage* st, int32_t max_launches) {
  pf_status s = check_stage(st, "stage_profile_begin");
  if (s != PF_OK) return s;
  if (max_launches < 1 || max_launches > (1 << 20))
    return fail(PF_ERR_INVALID_ARG, "stage_profile_begin: max_launches %d outside [1, 2^20]", max_launches);
  free_profile_events(st);
  st->prof_ev.reserve(2 * (size_t)max_launches);
  for (int32_t i = 0; i < 2 * max_launches; ++i) {
    hipEvent_t ev;
    hipError_t e = hipEventCreate(&ev);
    if (e != hipSuccess) {
      free_profile_events(st);
      return hip_fail(e, "stage_profile_begin: hipEventCreate");
    }
    st->prof_ev.push_back(ev);
  }
  st->prof_on = true;
  return PF_OK;
}

extern "C" pf_status stage_profile_end(pf_stage* st, int64_t* launches, double* attention_ms) {
  pf_status s = check_stage(st, "stage_profile_end");
  if (s != PF_OK) return s;
  if (!launches || !attention_ms) return fail(PF_ERR_INVALID_ARG, "stage_profile_end: null out");
  if (!st->prof_on) return fail(PF_ERR_STATE, "stage_profile_end: stage_profile_begin not called");
  st->prof_on = false;
  double total = 0.0;
  for (size_t i = 0; i + 1 < st->prof_used; i += 2) {
    hipError_t e = hipEventSynchronize(st->prof_ev[i + 1]);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, st->prof_ev[i], st->prof_ev[i + 1]);
    if (e != hipSuccess) {
      free_profile_events(st);
      return stage_hip_fail(st, e, "stage_profile_end: reading events");
    }
    total += ms;
  }
  *launches = (int64_t)(st->prof_used / 2);
  *attention_ms = total;
  free_profile_events(st);
  return PF_OK;
}

extern "C" pf_status stage_get_kvbuf_sample(pf_stage* st, int32_t layer, int32_t sample, pf_kv_view* out) {
  if (!st) return fail(PF_ERR_INVALID_ARG, "stage_get_kvbuf: null stage");
  if (!out) return fail(PF_ERR_INVALID_ARG, "stage_get_kvbuf: null out");
  if (layer < 0 || layer >= st->cfg.num_layers) return fail(PF_ERR_INVALID_ARG, "stage_get_kvbuf: bad layer");
  if (sample < 0 || sample >= st->batch) return fail(PF_ERR_INVALID_ARG, "stage_get_kvbuf: bad sample");
  const LayerMem& lm = st->layers[layer];
  out->k = (char*)lm.k + sample * st->kv_sample_bytes;
  out->v = (char*)lm.v + sample * st->kv_sample_bytes;
  out->rows = st->s_kv;
  out->row_elems = st->h;
  out->k_ld = st->h;
  out->v_ld = st->h;
  out->dtype = st->cfg.dtype;
  out->v_layout = st->cfg.dtype == PF_BF16 ? PF_LAYOUT_K8 : PF_LAYOUT_ROWS;
  return PF_OK;
}

extern "C" pf_status stage_get_config(const pf_stage* st, pf_stage_config* out) {
  if (!st || !out) return fail(PF_ERR_INVALID_ARG, "stage_get_config: null argument");
  *out = st->cfg;
  out->batch = (int32_t)st->batch;
  return PF_OK;
}

extern "C" pf_status stage_get_kvbuf(pf_stage* st, int32_t layer, pf_kv_view* out) {
  return stage_get_kvbuf_sample(st, layer, 0, out);
}
