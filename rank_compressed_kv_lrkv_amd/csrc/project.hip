// Fused projection + append: the cache rows of new tokens computed from their
// hidden states and written straight into the cache.
//
// Method (Low-Rank Key Value Attention, slide discussion of arXiv:2601.11471v3):
// a token's hidden state x (width d) is projected to the shared features
// k_s = x W^K_shared, v_s = x W^V_shared (width d_h) and to the per-head
// latents z^K_h = x U^K_h, z^V_h = x U^V_h (width r), which is all the cache
// keeps (slide "Cache shared features and compact per-head latents",
// Eqs. (4)-(5)).  Concatenated, that is one product
//   y = x . [W^K_shared | W^V_shared | U^K_1 .. U^K_H | U^V_1 .. U^V_H]
// from d to 2(d_h + H r) outputs per token, a dense GEMM over the batch's
// tokens: C[M x N] = X[M x d] . W^T with M = batch * n_new, N = 2(d_h + H r),
// and the weight given output-major (W[N][d], each output's d weights
// contiguous), so both operands are contiguous along the contraction.
//
// Tiling: a workgroup (4 wave64) computes a 128 x 128 block of C; each wave a
// 64 x 64 quarter as 2 x 2 tiles of v_mfma_f32_32x32x16_bf16.  The contraction
// advances 32 at a time; the X and W slices of a step (128 rows x 64 bytes
// each) are copied global -> LDS (buffer loads into LDS), double-buffered,
// rows swizzled so the operand reads are free of bank conflicts.  Rows past
// M or N clamp to the last row (their results are not stored).
//
// Epilogue: each output is rounded once to bf16 and stored at cache slot
// pos[b] + i of token (b, i) in the array its column belongs to; the array
// boundaries (d_h, 2 d_h, 2 d_h + H r) are multiples of 32, so every 32-column
// MFMA tile belongs to one array.  Slots outside [0, capacity) are dropped,
// as for the append.
#include "lrkv_device.h"
#include "lrkv_internal.h"

namespace lrkv {

constexpr int kPjThreads = 256;
constexpr int kPjBM = 128, kPjBN = 128, kPjBK = 32;     // block tile and contraction step
constexpr int kPjRowBytes = kPjBK * 2;                   // one row of a step slice: 64 bytes
constexpr int kPjSlice = kPjBM * kPjRowBytes;            // 8 KB per operand and step
constexpr int kPjChunks = kPjRowBytes / 16;              // 16-byte chunks per slice row

struct ProjectParams {
  const uint16_t* x; const uint16_t* w;
  uint16_t* k_s; uint16_t* v_s; uint16_t* z_k; uint16_t* z_v;
  const int32_t* pos;
  int M, N, K, n_new, head_dim, hr;   // hr = H * r
  int64_t capacity;
};

__global__ __launch_bounds__(kPjThreads) void project_append_kernel(ProjectParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char s_a[2][kPjSlice];
  __shared__ __attribute__((aligned(1024))) unsigned char s_b[2][kPjSlice];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;                 // the wave's 64 x 64 quarter
  const int n_lane = lane & 31, hf = lane >> 5;
  const int m0 = blockIdx.y * kPjBM, nb0 = blockIdx.x * kPjBN;

  // operand sources: rows m0.. of X and nb0.. of W, the whole contraction
  const __amdgpu_buffer_rsrc_t xres = buffer_resource(p.x + size_t(m0) * p.K, uint32_t(min(kPjBM, p.M - m0)) * p.K * 2);
  const __amdgpu_buffer_rsrc_t wres = buffer_resource(p.w + size_t(nb0) * p.K, uint32_t(min(kPjBN, p.N - nb0)) * p.K * 2);
  const int last_m = min(kPjBM, p.M - m0) - 1, last_n = min(kPjBN, p.N - nb0) - 1;

  // Transfer x of a slice carries LDS bytes [1024x, 1024x + 1024): 16 rows of
  // 64 bytes; lane i the chunk at position i % 4 of row 16x + i / 4, i.e.
  // source chunk pos ^ lds_swz(row, 4).  Each wave moves 2 of the 8.
  uint32_t a_off[2], b_off[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int xfer = wave * 2 + t, row = xfer * 16 + lane / 4, pos = lane % 4;
    const int ch = pos ^ lds_swz(row, kPjChunks);
    a_off[t] = uint32_t(min(row, last_m)) * p.K * 2 + ch * 16;
    b_off[t] = uint32_t(min(row, last_n)) * p.K * 2 + ch * 16;
  }
  auto load_step = [&](int ks, int buf) {
    const uint32_t k_off = uint32_t(ks) * kPjRowBytes;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int xfer = wave * 2 + t;
      dma16(xres, a_off[t] + k_off, 0u, &s_a[buf][xfer * 1024]);
      dma16(wres, b_off[t] + k_off, 0u, &s_b[buf][xfer * 1024]);
    }
  };

  // operand reads: lane (row n_lane of a 32-row tile, half hf) takes 16-byte
  // chunk 2c + hf of its row for contraction chunk c (k = 16c + 8hf ..)
  int a_rd[2][2], b_rd[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int ra = wm * 64 + t * 32 + n_lane, rb = wn * 64 + t * 32 + n_lane;
      a_rd[t][c] = ra * kPjRowBytes + ((2 * c + hf) ^ lds_swz(ra, kPjChunks)) * 16;
      b_rd[t][c] = rb * kPjRowBytes + ((2 * c + hf) ^ lds_swz(rb, kPjChunks)) * 16;
    }

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

  const int nsteps = p.K / kPjBK;
  load_step(0, 0);
  for (int ks = 0; ks < nsteps; ++ks) {
    const int buf = ks & 1;
    __builtin_amdgcn_s_waitcnt(0x0F70);                     // this wave's transfers of step ks have landed
    __syncthreads();                                        // everyone's have; buffer buf^1 is free
    if (ks + 1 < nsteps) load_step(ks + 1, buf ^ 1);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4 av[2], bv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        av[t] = *reinterpret_cast<const u32x4*>(&s_a[buf][a_rd[t][c]]);
        bv[t] = *reinterpret_cast<const u32x4*>(&s_b[buf][b_rd[t][c]]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(as_bf16x8(av[i]), as_bf16x8(bv[j]), acc[i][j]);
    }
  }

  // ---- epilogue: element e of tile (i, j) is row 8(e/4) + 4hf + e%4, column n_lane ----
  uint16_t* base[2];
  int col0[2], width[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n0 = nb0 + wn * 64 + j * 32;                 // first column of this 32-column tile
    if (n0 < p.head_dim) { base[j] = p.k_s; col0[j] = n0; width[j] = p.head_dim; }
    else if (n0 < 2 * p.head_dim) { base[j] = p.v_s; col0[j] = n0 - p.head_dim; width[j] = p.head_dim; }
    else if (n0 < 2 * p.head_dim + p.hr) { base[j] = p.z_k; col0[j] = n0 - 2 * p.head_dim; width[j] = p.hr; }
    else { base[j] = p.z_v; col0[j] = n0 - 2 * p.head_dim - p.hr; width[j] = p.hr; }
  }
  const bool col_ok[2] = {nb0 + wn * 64 < p.N, nb0 + wn * 64 + 32 < p.N};
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m0 + wm * 64 + i * 32 + 8 * (e / 4) + 4 * hf + (e % 4);
      if (m >= p.M) continue;
      const int b = m / p.n_new, tok = m - b * p.n_new;
      const long slot = long(p.pos ? p.pos[b] : 0) + tok;
      if (slot < 0 || slot >= p.capacity) continue;        // outside the cache: dropped
      const size_t row = size_t(b) * p.capacity + slot;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (col_ok[j]) base[j][row * width[j] + col0[j] + n_lane] = f32_to_bf16(acc[i][j][e]);
    }
}

// ---------------------------------------------------------------------------
// Vector-ALU projection for the shapes the MFMA kernel does not take (fp32,
// or bf16 with array widths that are not multiples of 32): a 64 x 64 block of
// C per workgroup, 4 x 4 outputs per lane, the contraction staged through LDS
// 16 at a time, fp32 fused multiply-adds.  Same output placement.
// ---------------------------------------------------------------------------
constexpr int kPvT = 64, kPvK = 16;

template <class E>
__global__ __launch_bounds__(256) void project_append_valu_kernel(ProjectParams p) {
  using T = typename E::T;
  __shared__ float s_x[kPvK][kPvT + 4];
  __shared__ float s_w[kPvK][kPvT + 4];
  const T* x = reinterpret_cast<const T*>(p.x);
  const T* w = reinterpret_cast<const T*>(p.w);
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  const int m0 = blockIdx.y * kPvT, n0 = blockIdx.x * kPvT;
  // staging: lane loads row tid / 4 at contraction offsets 4(tid % 4) .. +3
  const int lrow = tid / 4, lk = (tid % 4) * 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < p.K; k0 += kPvK) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = k0 + lk + u, mr = m0 + lrow, nr = n0 + lrow;
      s_x[lk + u][lrow] = (mr < p.M && k < p.K) ? E::to_f32(x[size_t(mr) * p.K + k]) : 0.f;
      s_w[lk + u][lrow] = (nr < p.N && k < p.K) ? E::to_f32(w[size_t(nr) * p.K + k]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPvK; ++k) {
      float a[4], bb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) { a[u] = s_x[k][ty * 4 + u]; bb[u] = s_w[k][tx * 4 + u]; }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(a[u], bb[v], acc[u][v]);
    }
    __syncthreads();
  }
  T* outs[4] = {reinterpret_cast<T*>(p.k_s), reinterpret_cast<T*>(p.v_s), reinterpret_cast<T*>(p.z_k),
                reinterpret_cast<T*>(p.z_v)};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int m = m0 + ty * 4 + u;
    if (m >= p.M) continue;
    const int b = m / p.n_new, tok = m - b * p.n_new;
    const long slot = long(p.pos ? p.pos[b] : 0) + tok;
    if (slot < 0 || slot >= p.capacity) continue;
    const size_t row = size_t(b) * p.capacity + slot;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int n = n0 + tx * 4 + v;
      if (n >= p.N) continue;
      int which, col, width;
      if (n < p.head_dim) { which = 0; col = n; width = p.head_dim; }
      else if (n < 2 * p.head_dim) { which = 1; col = n - p.head_dim; width = p.head_dim; }
      else if (n < 2 * p.head_dim + p.hr) { which = 2; col = n - 2 * p.head_dim; width = p.hr; }
      else { which = 3; col = n - 2 * p.head_dim - p.hr; width = p.hr; }
      outs[which][row * width + col] = E::from_f32(acc[u][v]);
    }
  }
}

// ---------------------------------------------------------------------------
// Packing of the projection weights into the output-major matrix the
// projection reads: row n of W holds the d_model weights of output n, for
// n < d_h the columns of W^K_shared [d][d_h], then W^V_shared, then column j
// of U^K_h [H][d][r] at row 2 d_h + h r + j, then U^V_h.  A transpose through
// LDS in 32 x 32 tiles; elements are copied bit-exactly.
// ---------------------------------------------------------------------------
struct PackParams {
  const unsigned char* wk; const unsigned char* wv; const unsigned char* uk; const unsigned char* uv;
  unsigned char* out;
  int d_model, head_dim, rank, hr, N, es;
};

__device__ __forceinline__ const unsigned char* pack_src(const PackParams& p, int k, int n) {
  if (n < p.head_dim) return p.wk + (size_t(k) * p.head_dim + n) * p.es;
  if (n < 2 * p.head_dim) return p.wv + (size_t(k) * p.head_dim + n - p.head_dim) * p.es;
  const bool is_k = n < 2 * p.head_dim + p.hr;
  const int c = n - 2 * p.head_dim - (is_k ? 0 : p.hr), h = c / p.rank, j = c - h * p.rank;
  return (is_k ? p.uk : p.uv) + ((size_t(h) * p.d_model + k) * p.rank + j) * p.es;
}

__global__ __launch_bounds__(256) void pack_projection_kernel(PackParams p) {
  __shared__ uint32_t tile[32][33];
  const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;
  const int n0 = blockIdx.x * 32, k0 = blockIdx.y * 32;
#pragma unroll
  for (int u = 0; u < 4; ++u) {                           // read: consecutive lanes along n
    const int k = k0 + ty + 8 * u, n = n0 + tx;
    uint32_t v = 0;
    if (k < p.d_model && n < p.N) {
      const unsigned char* s = pack_src(p, k, n);
      v = p.es == 2 ? uint32_t(*reinterpret_cast<const uint16_t*>(s)) : *reinterpret_cast<const uint32_t*>(s);
    }
    tile[ty + 8 * u][tx] = v;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u) {                           // write: consecutive lanes along k
    const int n = n0 + ty + 8 * u, k = k0 + tx;
    if (k >= p.d_model || n >= p.N) continue;
    unsigned char* d = p.out + (size_t(n) * p.d_model + k) * p.es;
    const uint32_t v = tile[tx][ty + 8 * u];
    if (p.es == 2) *reinterpret_cast<uint16_t*>(d) = uint16_t(v);
    else *reinterpret_cast<uint32_t*>(d) = v;
  }
}

bool project_mfma_supported(int dtype, int head_dim, int rank, int heads, int d_model) {
  return dtype == 1 && head_dim % 32 == 0 && (heads * rank) % 32 == 0 && d_model % kPjBK == 0 && d_model > 0;
}

hipError_t launch_project_append(const ProjectArgs& a, hipStream_t st) {
  ProjectParams p;
  p.x = static_cast<const uint16_t*>(a.x);
  p.w = static_cast<const uint16_t*>(a.w);
  p.k_s = static_cast<uint16_t*>(a.k_s); p.v_s = static_cast<uint16_t*>(a.v_s);
  p.z_k = static_cast<uint16_t*>(a.z_k); p.z_v = static_cast<uint16_t*>(a.z_v);
  p.pos = a.pos;
  p.M = a.batch * a.n_new;
  p.hr = a.heads * a.rank;
  p.N = 2 * (a.head_dim + p.hr);
  p.K = a.d_model;
  p.n_new = a.n_new;
  p.head_dim = a.head_dim;
  p.capacity = a.capacity;
  if (p.M <= 0) return hipSuccess;
  if (project_mfma_supported(a.dtype, a.head_dim, a.rank, a.heads, a.d_model)) {
    const dim3 grid((p.N + kPjBN - 1) / kPjBN, (p.M + kPjBM - 1) / kPjBM);
    hipLaunchKernelGGL(project_append_kernel, grid, dim3(kPjThreads), 0, st, p);
  } else {
    const dim3 grid((p.N + kPvT - 1) / kPvT, (p.M + kPvT - 1) / kPvT);
    if (a.dtype == 1) hipLaunchKernelGGL(project_append_valu_kernel<BF16>, grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL(project_append_valu_kernel<F32>, grid, dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_pack_projection(const PackArgs& a, hipStream_t st) {
  PackParams p;
  p.wk = static_cast<const unsigned char*>(a.wk_shared); p.wv = static_cast<const unsigned char*>(a.wv_shared);
  p.uk = static_cast<const unsigned char*>(a.u_k); p.uv = static_cast<const unsigned char*>(a.u_v);
  p.out = static_cast<unsigned char*>(a.w_packed);
  p.d_model = a.d_model; p.head_dim = a.head_dim; p.rank = a.rank; p.hr = a.heads * a.rank;
  p.N = 2 * (a.head_dim + p.hr);
  p.es = a.dtype == 1 ? 2 : 4;
  if (p.d_model <= 0) return hipSuccess;
  const dim3 grid((p.N + 31) / 32, (p.d_model + 31) / 32);
  hipLaunchKernelGGL(pack_projection_kernel, grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace lrkv
