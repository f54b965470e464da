// LRKV decode for any rank: the split-K scan and merge of decode.hip for
// latent widths the tuned scans do not take (ranks that are not multiples
// of 8 or 4, ranks up to 128, head counts up to 1024).
//
// Method (Low-Rank Key Value Attention, slide discussion of arXiv:2601.11471v3):
//   logits  s_t = scale ( q_h.k_{s,t} + (B^K_h^T q_h).z^K_{t,h} )     slide "Compute logits
//           without expanding historical keys", Eq. (6);
//   output  o_h = sum_t a_t v_{s,t} + B^V_h ( sum_t a_t z^V_{t,h} )     slide "Aggregate values
//           before the residual up-projection", Eq. (7);
// at the ranks of slides "The rank directly sets the theoretical cache
// budget" (Table 7) and "Backup: the complete rank sweep clarifies the
// trade-off" (Table 8), where a token's latent run of H*r elements need not
// fill whole 16-byte chunks.
//
// Work decomposition: a workgroup is 256 lanes = 32 heads x 8 lanes (grid.z
// runs further groups of 32 heads), over one split of one sequence.  The
// shared rows of 64 tokens are staged in LDS and read by every head; lane g
// of a head owns shared dims [g d_h/8, (g+1) d_h/8) and latent dims j = g +
// 8i.  Per token the head's 8 lanes add their partial logits through DPP,
// run the online softmax (all 8 hold the same m and l) and fold the token
// into their dims.  Latents are read element by element: the 64 lanes of a
// wave cover 8 heads x 8 consecutive elements, so each load instruction
// reads 8 runs of 8 contiguous elements.  The next token's latents are in
// flight while a token is computed.
//
// Numerics: fp32 throughout (the absorbed query B^K_h^T q_h is kept in fp32;
// bf16 elements are widened exactly).
#include "lrkv_device.h"
#include "lrkv_internal.h"

namespace lrkv {

namespace {

constexpr int kGnThreads = 256;
constexpr int kGnG = 8;                          // lanes per head
constexpr int kGnHeads = kGnThreads / kGnG;      // heads per workgroup
constexpr int kGnTile = 64;                      // tokens staged per tile
constexpr int kGnRPL = kGenericMaxRank / kGnG;   // latent dims per lane, at most

struct GnParams {
  const void* k_s; const void* v_s; const void* z_k; const void* z_v;
  const int32_t* seq_lens; const void* q; const void* b_k;
  float scale_log2;
  int heads, rank, max_len, split_tokens, partials;
  int64_t capacity;
  float* ws_ml; float* ws_acc;
};

template <class E>
__device__ __forceinline__ float gn_load(__amdgpu_buffer_rsrc_t res, uint32_t byte_off) {
  if constexpr (E::kBytes == 2)
    return bf16_to_f32(uint16_t(__builtin_amdgcn_raw_buffer_load_b16(res, int(byte_off), 0, kStream)));
  else
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(res, int(byte_off), 0, kStream));
}

template <class E>
__device__ __forceinline__ float gn_elem(const void* base, size_t i) {
  if constexpr (E::kBytes == 2) return bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
  else return static_cast<const float*>(base)[i];
}

}  // namespace

template <class E, int DH>
__global__ __launch_bounds__(kGnThreads) void decode_generic_kernel(GnParams p) {
  constexpr int G = kGnG, DPL = DH / G;
  constexpr int ES = E::kBytes, ROW = DH * ES, ROW_CH = ROW / 16;
  static_assert(DH % G == 0 && ROW % 16 == 0, "shared rows");
  __shared__ __attribute__((aligned(16))) unsigned char s_k[kGnTile * ROW];
  __shared__ __attribute__((aligned(16))) unsigned char s_v[kGnTile * ROW];
  const int tid = threadIdx.x, g = tid % G;
  const int split = blockIdx.x, b = blockIdx.y;
  const int H = p.heads, R = p.rank;
  const int h = blockIdx.z * kGnHeads + tid / G;
  const bool active = h < H;
  const int hh = active ? h : H - 1;

  int len = p.seq_lens[b];
  len = len < 0 ? 0 : (len > p.max_len ? p.max_len : len);
  const int t0 = split * p.split_tokens;
  if (t0 >= len) return;                                    // uniform: the merge reads no state here
  const int t1 = min(t0 + p.split_tokens, len);
  const int ntok = t1 - t0;
  const int nz = R > g ? (R - g + G - 1) / G : 0;          // latent dims of this lane

  // ---- this lane's slice of q_h and its latent dims of B^K_h^T q_h ----
  const size_t qbase = (size_t(b) * H + hh) * DH;
  float q[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) q[i] = gn_elem<E>(p.q, qbase + g * DPL + i);
  float qt[kGnRPL];
#pragma unroll
  for (int i = 0; i < kGnRPL; ++i) qt[i] = 0.f;
  if (R > 0) {
    const size_t bk0 = size_t(hh) * DH * R;
    for (int d = 0; d < DH; ++d) {
      const float qd = gn_elem<E>(p.q, qbase + d);
#pragma unroll
      for (int i = 0; i < kGnRPL; ++i)
        if (i < nz) qt[i] = __builtin_fmaf(qd, gn_elem<E>(p.b_k, bk0 + size_t(d) * R + g + G * i), qt[i]);
    }
  }

  // ---- resources over the split's tokens ----
  const size_t row0 = size_t(b) * p.capacity + size_t(t0);
  const uint32_t ztok = uint32_t(H) * uint32_t(R) * ES;     // latent bytes per token
  const __amdgpu_buffer_rsrc_t kres =
      buffer_resource(static_cast<const unsigned char*>(p.k_s) + row0 * ROW, uint32_t(ntok) * ROW);
  const __amdgpu_buffer_rsrc_t vres =
      buffer_resource(static_cast<const unsigned char*>(p.v_s) + row0 * ROW, uint32_t(ntok) * ROW);
  const __amdgpu_buffer_rsrc_t zkres =
      buffer_resource(static_cast<const unsigned char*>(p.z_k) + row0 * ztok, uint32_t(ntok) * ztok);
  const __amdgpu_buffer_rsrc_t zvres =
      buffer_resource(static_cast<const unsigned char*>(p.z_v) + row0 * ztok, uint32_t(ntok) * ztok);
  const uint32_t zlane = (uint32_t(hh) * R + g) * ES;       // byte offset of latent dim g of head hh in a token

  // latents of token tt (relative to t0) of this lane's dims
  auto zload = [&](float (&zk)[kGnRPL], float (&zv)[kGnRPL], int tt) __attribute__((always_inline)) {
    const uint32_t off = uint32_t(tt) * ztok + zlane;
#pragma unroll
    for (int i = 0; i < kGnRPL; ++i) {
      if (i < nz) {
        zk[i] = gn_load<E>(zkres, off + uint32_t(G * i * ES));
        zv[i] = gn_load<E>(zvres, off + uint32_t(G * i * ES));
      }
    }
  };

  float m = -INFINITY, l = 0.f;
  float acc_s[DPL], acc_z[kGnRPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc_s[i] = 0.f;
#pragma unroll
  for (int i = 0; i < kGnRPL; ++i) acc_z[i] = 0.f;
  float zk[2][kGnRPL], zv[2][kGnRPL];
#pragma unroll
  for (int i = 0; i < kGnRPL; ++i) zk[0][i] = zv[0][i] = zk[1][i] = zv[1][i] = 0.f;
  if (active) zload(zk[0], zv[0], 0);

  // One token: logit, online softmax, aggregation.  Buffer `cur` holds its
  // latents; the next token's go into the other buffer first.
  auto token = [&](int tt, int j, float (&zkc)[kGnRPL], float (&zvc)[kGnRPL], float (&zkn)[kGnRPL],
                   float (&zvn)[kGnRPL]) __attribute__((always_inline)) {
    if (active && tt + 1 < ntok) zload(zkn, zvn, tt + 1);
    float part = 0.f;
    {
      const unsigned char* kr = s_k + j * ROW + g * DPL * ES;
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        const float kv = ES == 2 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(kr)[i])
                                 : reinterpret_cast<const float*>(kr)[i];
        part = __builtin_fmaf(q[i], kv, part);
      }
    }
#pragma unroll
    for (int i = 0; i < kGnRPL; ++i)
      if (i < nz) part = __builtin_fmaf(qt[i], zkc[i], part);
    const float s = group_sum<G>(part) * p.scale_log2;
    if (s > m + 8.f) {                                       // lazy running max (log2 units)
      const float alpha = fast_exp2(m - s);                  // 0 on the first token (m = -inf)
      l *= alpha;
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc_s[i] *= alpha;
#pragma unroll
      for (int i = 0; i < kGnRPL; ++i) acc_z[i] *= alpha;
      m = s;
    }
    const float pe = fast_exp2(s - m);
    l += pe;
    const unsigned char* vr = s_v + j * ROW + g * DPL * ES;
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      const float vv = ES == 2 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(vr)[i])
                               : reinterpret_cast<const float*>(vr)[i];
      acc_s[i] = __builtin_fmaf(pe, vv, acc_s[i]);
    }
#pragma unroll
    for (int i = 0; i < kGnRPL; ++i)
      if (i < nz) acc_z[i] = __builtin_fmaf(pe, zvc[i], acc_z[i]);
  };

  for (int tile0 = 0; tile0 < ntok; tile0 += kGnTile) {
    const int nt = min(kGnTile, ntok - tile0);
    __syncthreads();                                         // the previous tile is consumed
    for (int idx = tid; idx < kGnTile * ROW_CH; idx += kGnThreads) {
      const int r = idx / ROW_CH, c = idx % ROW_CH;
      const uint32_t off = uint32_t(tile0 + min(r, nt - 1)) * ROW + uint32_t(c) * 16;
      *reinterpret_cast<u32x4*>(s_k + r * ROW + c * 16) =
          __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kres, int(off), 0, kStream));
      *reinterpret_cast<u32x4*>(s_v + r * ROW + c * 16) =
          __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vres, int(off), 0, kStream));
    }
    __syncthreads();
    if (!active) continue;
    int j = 0;
    for (; j + 1 < nt; j += 2) {
      token(tile0 + j, j, zk[0], zv[0], zk[1], zv[1]);
      token(tile0 + j + 1, j + 1, zk[1], zv[1], zk[0], zv[0]);
    }
    if (j < nt) {                                            // odd tile length: swap the buffers' roles
      token(tile0 + j, j, zk[0], zv[0], zk[1], zv[1]);
#pragma unroll
      for (int i = 0; i < kGnRPL; ++i) {
        zk[0][i] = zk[1][i];
        zv[0][i] = zv[1][i];
      }
    }
  }

  if (!active) return;
  // ---- partial state of this (split, head); same layout as decode_split_kernel ----
  const size_t pidx = (size_t(b) * p.partials + size_t(split)) * H + h;
  if (g == 0) {
    p.ws_ml[2 * pidx] = m;
    p.ws_ml[2 * pidx + 1] = l;
  }
  float* dst = p.ws_acc + pidx * size_t(DH + R);
#pragma unroll
  for (int i = 0; i < DPL; ++i) dst[g * DPL + i] = acc_s[i];
#pragma unroll
  for (int i = 0; i < kGnRPL; ++i)
    if (i < nz) dst[DH + g + G * i] = acc_z[i];
}

// Merge of the partial states of one (sequence, head), with the residual
// up-projection applied once (Eq. (7)): o = (sum_j w_j acc_s_j + B^V_h sum_j
// w_j acc_z_j) / L, w_j = 2^(m_j - M), L = sum_j w_j l_j.  Thread t folds
// merged dims t, t + 256, ... (d_h + r of them).
template <class E>
__global__ __launch_bounds__(kGnThreads) void decode_merge_generic_kernel(
    const float* __restrict__ ws_ml, const float* __restrict__ ws_acc, const int32_t* __restrict__ seq_lens,
    const void* b_v, void* out, int heads, int head_dim, int rank, int partials, int split_tokens, int max_len) {
  using T = typename E::T;
  __shared__ float s_a[kGenericMaxDims];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int D = head_dim + rank;
  int len = seq_lens[b];
  len = len < 0 ? 0 : (len > max_len ? max_len : len);
  T* o = static_cast<T*>(out) + (size_t(b) * heads + h) * head_dim;
  if (len == 0) {
    for (int d = tid; d < head_dim; d += kGnThreads) o[d] = E::from_f32(0.f);
    return;
  }
  const int n = (len + split_tokens - 1) / split_tokens;
  const float2* ml = reinterpret_cast<const float2*>(ws_ml) + size_t(b) * partials * heads + h;
  float M = -INFINITY;
  for (int j = 0; j < n; ++j) M = fmaxf(M, ml[size_t(j) * heads].x);
  float L = 0.f;
  for (int j = 0; j < n; ++j) {
    const float2 v = ml[size_t(j) * heads];
    L = __builtin_fmaf(fast_exp2(v.x - M), v.y, L);
  }
  for (int d = tid; d < D; d += kGnThreads) {
    float a = 0.f;
    for (int j = 0; j < n; ++j) {
      const size_t st = (size_t(b) * partials + j) * heads + h;
      a = __builtin_fmaf(fast_exp2(ml[size_t(j) * heads].x - M), ws_acc[st * D + d], a);
    }
    s_a[d] = a;
  }
  __syncthreads();
  for (int d = tid; d < head_dim; d += kGnThreads) {
    float a = s_a[d];
    for (int i = 0; i < rank; ++i)
      a = __builtin_fmaf(gn_elem<E>(b_v, (size_t(h) * head_dim + d) * rank + i), s_a[head_dim + i], a);
    o[d] = E::from_f32(a / L);
  }
}

bool decode_generic_supported(int dtype, int head_dim, int rank, int heads) {
  return (dtype == 0 || dtype == 1) && (head_dim == 16 || head_dim == 32 || head_dim == 64 || head_dim == 128) &&
         rank >= 0 && rank <= kGenericMaxRank && heads >= 1 && heads <= kGenericMaxHeads;
}

template <class E, int DH>
static hipError_t launch_generic_t(const DecodePlan& pl, const DecodeArgs& a, int phase, hipStream_t st) {
  if ((phase & 1) && pl.n_splits > 0) {
    GnParams kp;
    kp.k_s = a.k_s; kp.v_s = a.v_s; kp.z_k = a.z_k; kp.z_v = a.z_v;
    kp.seq_lens = a.seq_lens; kp.q = a.q; kp.b_k = a.b_k;
    kp.scale_log2 = a.scale_log2;
    kp.heads = pl.heads; kp.rank = pl.rank; kp.max_len = pl.max_len; kp.split_tokens = pl.split_tokens;
    kp.partials = pl.partials; kp.capacity = pl.capacity;
    kp.ws_ml = a.ws_ml; kp.ws_acc = a.ws_acc;
    const dim3 grid(unsigned(pl.n_splits), unsigned(pl.batch), unsigned((pl.heads + kGnHeads - 1) / kGnHeads));
    hipLaunchKernelGGL((decode_generic_kernel<E, DH>), grid, dim3(kGnThreads), 0, st, kp);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!(phase & 2)) return hipSuccess;
  hipLaunchKernelGGL((decode_merge_generic_kernel<E>), dim3(pl.heads, pl.batch), dim3(kGnThreads), 0, st, a.ws_ml,
                     a.ws_acc, a.seq_lens, a.b_v, a.out, pl.heads, pl.head_dim, pl.rank, pl.partials,
                     pl.split_tokens, pl.max_len);
  return hipGetLastError();
}

hipError_t launch_decode_generic(const DecodePlan& pl, const DecodeArgs& a, int phase, hipStream_t st) {
#define LRKV_GN(DHV)                                                                                   \
  if (pl.head_dim == DHV)                                                                              \
    return pl.dtype == 1 ? launch_generic_t<BF16, DHV>(pl, a, phase, st) : launch_generic_t<F32, DHV>(pl, a, phase, st);
  LRKV_GN(16) LRKV_GN(32) LRKV_GN(64) LRKV_GN(128)
#undef LRKV_GN
  return hipErrorInvalidValue;
}

}  // namespace lrkv
