// Cache append: copy the new tokens' shared rows and per-head latents into
// their slots (slide "Cache shared features and compact per-head latents",
// Eqs. (4)-(5): K_s, V_s and R_h are cached, B_h is not).  A bandwidth-bound
// copy in 16-byte units (4- or 2-byte units for a token latent run of H*r
// elements that is not a whole number of 16-byte chunks); grid.z selects
// which of the four cache arrays.
#include "lrkv_internal.h"

namespace lrkv {

__global__ __launch_bounds__(256) void append_kernel(unsigned char* k_s, unsigned char* v_s, unsigned char* z_k,
                                                     unsigned char* z_v, const int32_t* __restrict__ pos,
                                                     const unsigned char* __restrict__ nk, const unsigned char* __restrict__ nv,
                                                     const unsigned char* __restrict__ nzk, const unsigned char* __restrict__ nzv,
                                                     int n_new, int64_t capacity, int shared_row_bytes, int latent_row_bytes,
                                                     int pos_max) {
  const int which = blockIdx.z;                      // 0 k_s, 1 v_s, 2 z_k, 3 z_v
  const int b = blockIdx.y;
  const int row_bytes = which < 2 ? shared_row_bytes : latent_row_bytes;
  const int unit = row_bytes % 16 == 0 ? 16 : row_bytes % 4 == 0 ? 4 : 2;
  const int chunks = row_bytes / unit;
  if (chunks == 0) return;                           // rank 0: no latent rows
  const long idx = long(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= long(n_new) * chunks) return;
  const int i = int(idx / chunks), c = int(idx % chunks);
  int p0 = pos ? pos[b] : 0;
  p0 = p0 > pos_max ? pos_max : (p0 < 0 && pos_max != INT32_MAX ? 0 : p0);
  const long slot = long(p0) + i;
  if (slot < 0 || slot >= capacity) return;          // outside the cache: dropped
  unsigned char* dst = which == 0 ? k_s : which == 1 ? v_s : which == 2 ? z_k : z_v;
  const unsigned char* src = which == 0 ? nk : which == 1 ? nv : which == 2 ? nzk : nzv;
  const unsigned char* s = src + (size_t(b) * n_new + i) * row_bytes + size_t(c) * unit;
  unsigned char* d = dst + (size_t(b) * capacity + slot) * row_bytes + size_t(c) * unit;
  if (unit == 16) *reinterpret_cast<uint4*>(d) = *reinterpret_cast<const uint4*>(s);
  else if (unit == 4) *reinterpret_cast<uint32_t*>(d) = *reinterpret_cast<const uint32_t*>(s);
  else *reinterpret_cast<uint16_t*>(d) = *reinterpret_cast<const uint16_t*>(s);
}

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
  if (a.n_new <= 0 || a.batch <= 0) return hipSuccess;
  const int es = a.dtype == 1 ? 2 : 4;
  const int shared_row = a.head_dim * es;
  const int latent_row = a.heads * a.rank * es;
  const int latent_unit = latent_row % 16 == 0 ? 16 : latent_row % 4 == 0 ? 4 : 2;
  const int max_chunks = shared_row / 16 > latent_row / latent_unit ? shared_row / 16 : latent_row / latent_unit;
  const long work = long(a.n_new) * max_chunks;
  const dim3 grid(unsigned((work + 255) / 256), unsigned(a.batch), 4);
  hipLaunchKernelGGL(append_kernel, grid, dim3(256), 0, st, static_cast<unsigned char*>(a.k_s),
                     static_cast<unsigned char*>(a.v_s), static_cast<unsigned char*>(a.z_k),
                     static_cast<unsigned char*>(a.z_v), a.pos, static_cast<const unsigned char*>(a.new_k_s),
                     static_cast<const unsigned char*>(a.new_v_s), static_cast<const unsigned char*>(a.new_z_k),
                     static_cast<const unsigned char*>(a.new_z_v), a.n_new, a.capacity, shared_row, latent_row,
                     a.pos_max);
  return hipGetLastError();
}

}  // namespace lrkv
