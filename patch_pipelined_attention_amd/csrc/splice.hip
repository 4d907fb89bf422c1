// KV-buffer splice: bit copy of a block of rows into a K/V buffer pair.
//
// This is the in-place update of PipeFusion's per-layer full-spatial KV buffer (the
// technical summaries' mechanism 2 and 4): the current patch's fresh K/V replace its
// own rows while every other row keeps the previous step's values.  HBM-bound; every
// path moves whole 16-byte units where the layouts allow it.
//
// Paths (chosen per matrix on the host):
//   rows -> rows : one thread per 16-byte chunk of a row.
//   rows -> K8   : one workgroup per (8-row group of the destination, 512 columns): the
//                  rows are read in 16-byte units into LDS, and each thread assembles one
//                  column's 8 rows into a 16-byte K8 unit, so loads and stores both run
//                  along contiguous memory.  Groups cut by the ends of the range merge with
//                  the destination's existing bytes (read-modify-write of that group only).
//   generic      : one thread per element (any other layout pair, e.g. K8 -> rows).
#include "pf_internal.h"

namespace pf {

struct SpliceMat {
  const char* src;
  char* dst;
  int64_t src_ld, dst_ld;    // elements (ROWS layout)
  int src_layout, dst_layout;
};

__device__ __forceinline__ int64_t elem_index(int layout, int64_t ld, int64_t row_elems, int64_t r,
                                              int64_t c) {
  return layout == kLayoutK8 ? ((r >> 3) * row_elems + c) * 8 + (r & 7) : r * ld + c;
}

__global__ __launch_bounds__(256) void splice_rows_kernel(SpliceMat m0, SpliceMat m1, int64_t row_bytes,
                                                          int64_t len, int64_t offset, int esize) {
  const SpliceMat m = blockIdx.y == 0 ? m0 : m1;
  const int64_t chunks = row_bytes >> 4;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= chunks * len) return;
  const int64_t i = id / chunks, ch = id - i * chunks;
  const uint4 v = *reinterpret_cast<const uint4*>(m.src + i * m.src_ld * esize + ch * 16);
  *reinterpret_cast<uint4*>(m.dst + (offset + i) * m.dst_ld * esize + ch * 16) = v;
}

// 16-bit elements only.  Workgroup = one destination group g of 8 rows x kK8Cols columns: the
// group's source rows are read in 16-byte units (a wavefront covers 1 KB of one row) into an
// LDS tile, then thread j assembles column c's 8 rows (one 16-byte K8 unit) and stores it, so
// consecutive threads write consecutive 16-byte units.  Groups cut by the ends of the range
// merge with the destination's existing bytes (read-modify-write of those units only).
constexpr int kK8Cols = 512;
__global__ __launch_bounds__(256) void splice_rows_to_k8_kernel(SpliceMat m0, SpliceMat m1,
                                                                int64_t row_elems, int64_t len,
                                                                int64_t offset) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[8][kK8Cols];
  const SpliceMat m = blockIdx.y == 0 ? m0 : m1;
  const int64_t ncb = (row_elems + kK8Cols - 1) / kK8Cols;
  const int64_t g = (offset >> 3) + (int64_t)blockIdx.x / ncb;
  const int64_t c0 = ((int64_t)blockIdx.x % ncb) * kK8Cols;
  const int ncols = (int)(row_elems - c0 < kK8Cols ? row_elems - c0 : kK8Cols);   // a multiple of 8
  const uint16_t* src = reinterpret_cast<const uint16_t*>(m.src);
  uint16_t* dst = reinterpret_cast<uint16_t*>(m.dst);
  unsigned valid = 0;
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    const int64_t r = g * 8 + rr;
    if (r >= offset && r < offset + len) valid |= 1u << rr;
  }
  // load: 8 rows x ncols / 8 units of 16 bytes
  for (int idx = threadIdx.x; idx < 8 * (kK8Cols / 8); idx += 256) {
    const int rr = idx / (kK8Cols / 8), ch = idx % (kK8Cols / 8);
    if (ch * 8 >= ncols || !(valid & (1u << rr))) continue;
    const int64_t i = g * 8 + rr - offset;
    *reinterpret_cast<uint4*>(&tile[rr][ch * 8]) = *reinterpret_cast<const uint4*>(src + i * m.src_ld + c0 + ch * 8);
  }
  __syncthreads();
  for (int c = threadIdx.x; c < ncols; c += 256) {
    uint16_t* p = dst + (g * row_elems + c0 + c) * 8;
    uint16_t out[8];
    if (valid != 0xFFu) {
      const uint4 old = *reinterpret_cast<const uint4*>(p);
      const uint32_t w[4] = {old.x, old.y, old.z, old.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        out[2 * e] = (uint16_t)(w[e] & 0xFFFFu);
        out[2 * e + 1] = (uint16_t)(w[e] >> 16);
      }
    }
#pragma unroll
    for (int rr = 0; rr < 8; ++rr)
      if (valid & (1u << rr)) out[rr] = tile[rr][c];
    uint4 v;
    v.x = (uint32_t)out[0] | ((uint32_t)out[1] << 16);
    v.y = (uint32_t)out[2] | ((uint32_t)out[3] << 16);
    v.z = (uint32_t)out[4] | ((uint32_t)out[5] << 16);
    v.w = (uint32_t)out[6] | ((uint32_t)out[7] << 16);
    *reinterpret_cast<uint4*>(p) = v;
  }
}

__global__ __launch_bounds__(256) void splice_generic_kernel(SpliceMat m0, SpliceMat m1,
                                                             int64_t row_elems, int64_t len,
                                                             int64_t offset, int esize) {
  const SpliceMat m = blockIdx.y == 0 ? m0 : m1;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= row_elems * len) return;
  const int64_t i = id / row_elems, c = id - i * row_elems;
  const int64_t si = elem_index(m.src_layout, m.src_ld, row_elems, i, c);
  const int64_t di = elem_index(m.dst_layout, m.dst_ld, row_elems, offset + i, c);
  if (esize == 2)
    reinterpret_cast<uint16_t*>(m.dst)[di] = reinterpret_cast<const uint16_t*>(m.src)[si];
  else
    reinterpret_cast<uint32_t*>(m.dst)[di] = reinterpret_cast<const uint32_t*>(m.src)[si];
}

static int path_of(const KVDesc& d, const KVDesc& s, int64_t row_elems, int esize) {
  const bool rows_ok = ((row_elems * esize) % 16 == 0) && ((s.ld * esize) % 16 == 0) &&
                       (((uintptr_t)s.base & 15) == 0);
  if (s.layout == kLayoutRows && d.layout == kLayoutRows && rows_ok && ((d.ld * esize) % 16 == 0) &&
      (((uintptr_t)d.base & 15) == 0))
    return 0;
  if (s.layout == kLayoutRows && d.layout == kLayoutK8 && esize == 2 && rows_ok && row_elems % 8 == 0 &&
      (((uintptr_t)d.base & 15) == 0))
    return 1;
  return 2;
}

hipError_t launch_splice(const KVDesc dst[2], const KVDesc src[2], int64_t row_elems, int64_t offset,
                         int64_t len, int esize, hipStream_t s) {
  if (len <= 0) return hipSuccess;
  SpliceMat m[2];
  for (int t = 0; t < 2; ++t) {
    m[t].src = static_cast<const char*>(src[t].base);
    m[t].dst = static_cast<char*>(const_cast<void*>(dst[t].base));
    m[t].src_ld = src[t].ld;
    m[t].dst_ld = dst[t].ld;
    m[t].src_layout = src[t].layout;
    m[t].dst_layout = dst[t].layout;
  }
  const int p0 = path_of(dst[0], src[0], row_elems, esize);
  const int p1 = path_of(dst[1], src[1], row_elems, esize);
  // Both matrices share one launch when they take the same path; otherwise two launches.
  for (int t = 0; t < 2; ++t) {
    const int p = t == 0 ? p0 : p1;
    if (t == 1 && p1 == p0) break;
    const SpliceMat a = (p0 == p1) ? m[0] : m[t];
    const SpliceMat b = (p0 == p1) ? m[1] : m[t];
    const unsigned ny = (p0 == p1) ? 2u : 1u;
    if (p == 0) {
      const int64_t units = (row_elems * esize / 16) * len;
      hipLaunchKernelGGL(splice_rows_kernel, dim3((unsigned)((units + 255) / 256), ny), dim3(256), 0, s, a,
                         b, row_elems * esize, len, offset, esize);
    } else if (p == 1) {
      const int64_t ngroups = ((offset + len - 1) >> 3) - (offset >> 3) + 1;
      const int64_t blocks = ngroups * ((row_elems + kK8Cols - 1) / kK8Cols);
      hipLaunchKernelGGL(splice_rows_to_k8_kernel, dim3((unsigned)blocks, ny), dim3(256), 0, s, a, b, row_elems,
                         len, offset);
    } else {
      const int64_t units = row_elems * len;
      hipLaunchKernelGGL(splice_generic_kernel, dim3((unsigned)((units + 255) / 256), ny), dim3(256), 0, s,
                         a, b, row_elems, len, offset, esize);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pf
