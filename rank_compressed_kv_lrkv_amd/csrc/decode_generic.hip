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
// Work decomposition: a workgroup is 256 lanes = (256 / G) heads x G lanes
// (G = 8, 16 or 32 lanes per head, more lanes per head when there are few
// heads; grid.z runs further head groups), over one split of one sequence.
// The split's tokens go through LDS in tiles of T tokens (T chosen on the
// host so that a tile fits 64 KB): the shared rows, and for every token the
// contiguous run of the group's latents, [h0 r, (h0 + heads) r) of its H r
// elements, copied with 16-byte loads from the 16-byte boundary at or below
// its start (the run's offset inside the copy is kept per token).  So every
// global load is a whole 16-byte chunk whatever the rank, except the one
// chunk that crosses the split's last byte, read in 2-byte pieces that each
// lie inside the split.  Lane g of a head owns shared dims
// [g d_h/G, (g+1) d_h/G) and latent dims j = g + G i.  Per token the head's
// G lanes add their partial logits through DPP, run the online softmax (all
// G hold the same m and l) and fold the token into their dims; two tokens
// are interleaved.  Two or more workgroups are resident per compute unit,
// so one's tile copy overlaps another's arithmetic.
//
// Numerics: fp32 throughout (the absorbed query B^K_h^T q_h is kept in fp32;
// bf16 elements are widened exactly).
#include "lrkv_device.h"
#include "lrkv_internal.h"

namespace lrkv {

namespace {

constexpr int kGnThreads = 256;
constexpr int kGnTileMax = 64;                   // tokens per tile, at most
constexpr int kGnLdsBudget = 64 * 1024;          // bytes of LDS per workgroup, at most

struct GnParams {
  const void* k_s; const void* v_s; const void* z_k; const void* z_v;
  const int32_t* seq_lens; const void* q; const void* b_k;
  float scale_log2;
  int heads, rank, max_len, split_tokens, partials;
  int tile, zrow;                                // tokens per tile; LDS bytes per token's latent copy
  int64_t capacity;
  float* ws_ml; float* ws_acc;
};

template <class E>
__device__ __forceinline__ float gn_elem(const void* base, size_t i) {
  if constexpr (E::kBytes == 2) return bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
  else return static_cast<const float*>(base)[i];
}

template <class E>
__device__ __forceinline__ float gn_lds(const unsigned char* p) {
  if constexpr (E::kBytes == 2) return bf16_to_f32(*reinterpret_cast<const uint16_t*>(p));
  else return *reinterpret_cast<const float*>(p);
}

// Sum over aligned groups of G lanes (G up to 32): DPP within 8 lanes, row
// mirror for 16, a bit-mode swizzle (xor 16) for 32.
template <int G>
__device__ __forceinline__ float gn_group_sum(float v) {
  v = group_sum<(G < 8 ? G : 8)>(v);
  if constexpr (G >= 16) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  if constexpr (G >= 32) v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
  return v;
}

}  // namespace

// Lanes per head of the any-rank scan.
int generic_lanes_per_head(int heads, int head_dim) {
  const int g = heads > 16 ? 8 : heads > 8 ? 16 : 32;
  return g > head_dim ? head_dim : g;
}

template <class E, int DH, int G>
__global__ __launch_bounds__(kGnThreads) void decode_generic_kernel(GnParams p) {
  constexpr int DPL = DH / G, HW = kGnThreads / G;
  constexpr int ES = E::kBytes, ROW = DH * ES, ROW_CH = ROW / 16;
  static_assert(DH % G == 0 && ROW % 16 == 0, "shared rows");
  constexpr int RPL = (kGenericMaxRank + G - 1) / G;      // latent dims per lane, at most
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int T = p.tile, ZR = p.zrow;
  unsigned char* const s_k = smem;
  unsigned char* const s_v = s_k + T * ROW;
  unsigned char* const s_zk = s_v + T * ROW;
  unsigned char* const s_zv = s_zk + size_t(T) * ZR;
  int* const s_off = reinterpret_cast<int*>(s_zv + size_t(T) * ZR);   // run offset inside each token's copy
  const int tid = threadIdx.x, g = tid % G, hl = tid / G;
  const int split = blockIdx.x, b = blockIdx.y;
  const int H = p.heads, R = p.rank;
  const int h0 = blockIdx.z * HW;
  const int h = h0 + hl;
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
  float qt[RPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i) qt[i] = 0.f;
  if (R > 0) {
    const size_t bk0 = size_t(hh) * DH * R;
    for (int d = 0; d < DH; ++d) {
      const float qd = gn_elem<E>(p.q, qbase + d);
#pragma unroll
      for (int i = 0; i < RPL; ++i)
        if (i < nz) qt[i] = __builtin_fmaf(qd, gn_elem<E>(p.b_k, bk0 + size_t(d) * R + g + G * i), qt[i]);
    }
  }

  // ---- resources over the split's tokens ----
  const size_t row0 = size_t(b) * p.capacity + size_t(t0);
  const int nh = min(HW, H - h0);                           // heads of this group
  const uint32_t ztok = uint32_t(H) * uint32_t(R) * ES;    // latent bytes per token (all heads)
  const uint32_t zrun = uint32_t(nh) * uint32_t(R) * ES;   // the group's run in a token
  const size_t zstart = (row0 * size_t(H) + size_t(h0)) * size_t(R) * ES;   // byte of the split's first run
  const size_t zbase = zstart & ~size_t(15);
  const uint32_t zlead = uint32_t(zstart - zbase);          // < 16
  const __amdgpu_buffer_rsrc_t kres =
      buffer_resource(static_cast<const unsigned char*>(p.k_s) + row0 * ROW, uint32_t(ntok) * ROW);
  const __amdgpu_buffer_rsrc_t vres =
      buffer_resource(static_cast<const unsigned char*>(p.v_s) + row0 * ROW, uint32_t(ntok) * ROW);
  // the split's latent bytes from the aligned start to the end of its last run
  const uint32_t zbytes = zlead + uint32_t(ntok - 1) * ztok + zrun;
  const __amdgpu_buffer_rsrc_t zkres =
      buffer_resource(static_cast<const unsigned char*>(p.z_k) + (R > 0 ? zbase : 0), R > 0 ? zbytes : 0u);
  const __amdgpu_buffer_rsrc_t zvres =
      buffer_resource(static_cast<const unsigned char*>(p.z_v) + (R > 0 ? zbase : 0), R > 0 ? zbytes : 0u);
  const int zch = ZR / 16;                                  // 16-byte chunks per token copy
  const uint32_t zlane = (uint32_t(hl) * R + g) * ES;       // byte of latent dim g of this head in the run

  float m = -INFINITY, l = 0.f;
  float acc_s[DPL], acc_z[RPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc_s[i] = 0.f;
#pragma unroll
  for (int i = 0; i < RPL; ++i) acc_z[i] = 0.f;

  // One token j of the tile: logit, online softmax, aggregation.
  auto token = [&](int j) __attribute__((always_inline)) {
    float part = 0.f;
    {
      const unsigned char* kr = s_k + j * ROW + g * DPL * ES;
#pragma unroll
      for (int i = 0; i < DPL; ++i) part = __builtin_fmaf(q[i], gn_lds<E>(kr + i * ES), part);
    }
    const unsigned char* zkr = s_zk + size_t(j) * ZR + s_off[j] + zlane;
#pragma unroll
    for (int i = 0; i < RPL; ++i)
      if (i < nz) part = __builtin_fmaf(qt[i], gn_lds<E>(zkr + G * i * ES), part);
    const float s = gn_group_sum<G>(part) * p.scale_log2;
    if (s > m + 8.f) {                                       // lazy running max (log2 units)
      const float alpha = fast_exp2(m - s);                  // 0 on the first token (m = -inf)
      l *= alpha;
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc_s[i] *= alpha;
#pragma unroll
      for (int i = 0; i < RPL; ++i) acc_z[i] *= alpha;
      m = s;
    }
    const float pe = fast_exp2(s - m);
    l += pe;
    const unsigned char* vr = s_v + j * ROW + g * DPL * ES;
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc_s[i] = __builtin_fmaf(pe, gn_lds<E>(vr + i * ES), acc_s[i]);
    const unsigned char* zvr = s_zv + size_t(j) * ZR + s_off[j] + zlane;
#pragma unroll
    for (int i = 0; i < RPL; ++i)
      if (i < nz) acc_z[i] = __builtin_fmaf(pe, gn_lds<E>(zvr + G * i * ES), acc_z[i]);
  };

  for (int tile0 = 0; tile0 < ntok; tile0 += T) {
    const int nt = min(T, ntok - tile0);
    __syncthreads();                                         // the previous tile is consumed
    // shared rows (rows past the split repeat its last token)
    for (int idx = tid; idx < T * ROW_CH; idx += kGnThreads) {
      const int r = idx / ROW_CH, c = idx % ROW_CH;
      const uint32_t off = uint32_t(tile0 + min(r, nt - 1)) * ROW + uint32_t(c) * 16;
      const u32x4 kv = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kres, int(off), 0, kStream));
      const u32x4 vv = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vres, int(off), 0, kStream));
      *reinterpret_cast<u32x4*>(s_k + r * ROW + c * 16) = kv;
      *reinterpret_cast<u32x4*>(s_v + r * ROW + c * 16) = vv;
    }
    // latent runs: token r's run starts `lead` bytes into its 16-byte-aligned
    // copy; bytes past the split's last run are zero
    if (R > 0) {
      for (int idx0 = tid; idx0 < T * zch; idx0 += 4 * kGnThreads) {
        u32x4 zk4[4], zv4[4];
        int at[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int idx = idx0 + u * kGnThreads;
          at[u] = -1;
          zk4[u] = zv4[u] = u32x4{0u, 0u, 0u, 0u};
          if (idx < T * zch) {
            const int r = idx / zch, c = idx % zch;
            const uint32_t rel = zlead + uint32_t(tile0 + min(r, nt - 1)) * ztok;
            const uint32_t off = (rel & ~15u) + uint32_t(c) * 16;
            if (off + 16 <= zbytes) {
              zk4[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(zkres, int(off), 0, kStream));
              zv4[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(zvres, int(off), 0, kStream));
            } else if (off < zbytes) {
              // the chunk that crosses the split's last byte: 2-byte loads,
              // each inside the range (no load partly out of it)
              uint32_t wk[4] = {0u, 0u, 0u, 0u}, wv[4] = {0u, 0u, 0u, 0u};
              for (int e = 0; e < 8; ++e)
                if (off + 2 * e < zbytes) {
                  wk[e >> 1] |= uint32_t(uint16_t(__builtin_amdgcn_raw_buffer_load_b16(zkres, int(off + 2 * e), 0,
                                                                                        kStream))) << (16 * (e & 1));
                  wv[e >> 1] |= uint32_t(uint16_t(__builtin_amdgcn_raw_buffer_load_b16(zvres, int(off + 2 * e), 0,
                                                                                        kStream))) << (16 * (e & 1));
                }
              zk4[u] = u32x4{wk[0], wk[1], wk[2], wk[3]};
              zv4[u] = u32x4{wv[0], wv[1], wv[2], wv[3]};
            }
            at[u] = r * ZR + c * 16;
            if (c == 0) s_off[r] = int(rel & 15u);
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (at[u] >= 0) {
            *reinterpret_cast<u32x4*>(s_zk + at[u]) = zk4[u];
            *reinterpret_cast<u32x4*>(s_zv + at[u]) = zv4[u];
          }
      }
    } else if (tid < T) {
      s_off[tid] = 0;
    }
    __syncthreads();
    if (!active) continue;
    int j = 0;
    for (; j + 1 < nt; j += 2) {
      token(j);
      token(j + 1);
    }
    if (j < nt) token(j);
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
  for (int i = 0; i < RPL; ++i)
    if (i < nz) dst[DH + g + G * i] = acc_z[i];
}

// Merge of the partial states of one (sequence, head), with the residual
// up-projection applied once (Eq. (7)): o = (sum_j w_j acc_s_j + B^V_h sum_j
// w_j acc_z_j) / L, w_j = 2^(m_j - M), L = sum_j w_j l_j.  The partials' maxima
// and weights are spread over the threads (block reductions), each thread
// folds merged dims t, t + 256, ... (d_h + r of them) with the weights from
// LDS, and for bf16 B^V_h is staged in LDS (coalesced) before thread d < d_h
// forms its row's product.
constexpr int kMgW = 1024;                          // partial weights held in LDS per pass

static __device__ __forceinline__ float block_reduce(float v, float* s_red, bool is_max) {
  for (int o = 32; o >= 1; o >>= 1) {
    const float u = __shfl_xor(v, o);
    v = is_max ? fmaxf(v, u) : v + u;
  }
  const int w = threadIdx.x >> 6;
  __syncthreads();                                  // s_red free from any earlier use
  if ((threadIdx.x & 63) == 0) s_red[w] = v;
  __syncthreads();
  return is_max ? fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]))
                : (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
}

template <class E>
__global__ __launch_bounds__(kGnThreads) void decode_merge_generic_kernel(
    const float* __restrict__ ws_ml, const float* __restrict__ ws_acc, const int32_t* __restrict__ seq_lens,
    const void* b_v, void* out, int heads, int head_dim, int rank, int partials, int split_tokens, int max_len) {
  using T = typename E::T;
  static_assert(kGnThreads == 256, "four waves");
  constexpr bool kStageBv = E::kBytes == 2;
  __shared__ float s_a[kGenericMaxDims];
  __shared__ float s_w[kMgW];
  __shared__ float s_red[4];
  __shared__ __attribute__((aligned(16))) uint16_t s_bv[kStageBv ? 128 * kGenericMaxRank : 8];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int D = head_dim + rank;
  int len = seq_lens[b];
  len = len < 0 ? 0 : (len > max_len ? max_len : len);
  T* o = static_cast<T*>(out) + (size_t(b) * heads + h) * head_dim;
  if (len == 0) {
    for (int d = tid; d < head_dim; d += kGnThreads) o[d] = E::from_f32(0.f);
    return;
  }
  // B^V_h staged while the partial states are merged: head_dim rows of rank
  // bf16, 16-byte aligned as a whole (head_dim a multiple of 16), in 16-byte
  // chunks, all of a thread's loads issued before any store
  constexpr int kMaxCh = kStageBv ? 128 * kGenericMaxRank * 2 / 16 / kGnThreads : 1;
  const int nch = kStageBv ? head_dim * rank * 2 / 16 : 0;
  u32x4 c[kMaxCh];
  if constexpr (kStageBv) {
    const u32x4* bv = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(b_v) + size_t(h) * head_dim * rank);
#pragma unroll
    for (int k = 0; k < kMaxCh; ++k) {
      const int i = tid + k * kGnThreads;
      if (i < nch) c[k] = bv[i];
    }
  }
  const int n = (len + split_tokens - 1) / split_tokens;
  const float2* ml = reinterpret_cast<const float2*>(ws_ml) + size_t(b) * partials * heads + h;
  float mloc = -INFINITY;
  for (int j = tid; j < n; j += kGnThreads) mloc = fmaxf(mloc, ml[size_t(j) * heads].x);
  if constexpr (kStageBv) {                         // stored once the partials' maxima are in flight
#pragma unroll
    for (int k = 0; k < kMaxCh; ++k) {
      const int i = tid + k * kGnThreads;
      if (i < nch) reinterpret_cast<u32x4*>(s_bv)[i] = c[k];
    }
  }
  const float M = block_reduce(mloc, s_red, true);
  float acc[(kGenericMaxDims + kGnThreads - 1) / kGnThreads];
#pragma unroll
  for (int k = 0; k < (kGenericMaxDims + kGnThreads - 1) / kGnThreads; ++k) acc[k] = 0.f;
  float lloc = 0.f;
  for (int j0 = 0; j0 < n; j0 += kMgW) {
    const int nj = min(kMgW, n - j0);
    __syncthreads();                                // s_w free from the previous pass
    for (int j = tid; j < nj; j += kGnThreads) {
      const float2 v = ml[size_t(j0 + j) * heads];
      const float w = fast_exp2(v.x - M);
      s_w[j] = w;
      lloc = __builtin_fmaf(w, v.y, lloc);
    }
    __syncthreads();
    const float* src = ws_acc + ((size_t(b) * partials + j0) * heads + h) * D;
    const size_t step = size_t(heads) * D;
#pragma unroll
    for (int k = 0; k < (kGenericMaxDims + kGnThreads - 1) / kGnThreads; ++k) {
      const int d = tid + k * kGnThreads;
      if (d < D) {
        float a = acc[k];
        int j = 0;
        for (; j + 8 <= nj; j += 8) {               // eight partial loads in flight
          float x[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) x[u] = src[size_t(j + u) * step + d];
#pragma unroll
          for (int u = 0; u < 8; ++u) a = __builtin_fmaf(s_w[j + u], x[u], a);
        }
        for (; j < nj; ++j) a = __builtin_fmaf(s_w[j], src[size_t(j) * step + d], a);
        acc[k] = a;
      }
    }
  }
  const float L = block_reduce(lloc, s_red, false);
#pragma unroll
  for (int k = 0; k < (kGenericMaxDims + kGnThreads - 1) / kGnThreads; ++k) {
    const int d = tid + k * kGnThreads;
    if (d < D) s_a[d] = acc[k];
  }
  __syncthreads();
  for (int d = tid; d < head_dim; d += kGnThreads) {
    float a = s_a[d];
    if constexpr (kStageBv) {
      const uint16_t* row = s_bv + d * rank;
      for (int i = 0; i < rank; ++i) a = __builtin_fmaf(bf16_to_f32(row[i]), s_a[head_dim + i], a);
    } else {
      for (int i = 0; i < rank; ++i)
        a = __builtin_fmaf(gn_elem<E>(b_v, (size_t(h) * head_dim + d) * rank + i), s_a[head_dim + i], a);
    }
    o[d] = E::from_f32(a / L);
  }
}

bool decode_generic_supported(int dtype, int head_dim, int rank, int heads) {
  return (dtype == 0 || dtype == 1) && (head_dim == 16 || head_dim == 32 || head_dim == 64 || head_dim == 128) &&
         rank >= 0 && rank <= kGenericMaxRank && heads >= 1 && heads <= kGenericMaxHeads;
}

// Tokens per tile and the LDS bytes of one token's latent copy, for lanes
// per head G: the largest power of two up to kGnTileMax whose tile (shared
// rows, the two latent copies, the run offsets) fits kGnLdsBudget.
static void generic_tile(const DecodePlan& pl, int G, int* tile, int* zrow, int* lds) {
  const int es = pl.dtype == 1 ? 2 : 4;
  const int hw = kGnThreads / G;
  const int nh = pl.heads < hw ? pl.heads : hw;
  const int zr = pl.rank > 0 ? (nh * pl.rank * es + 15 + 15) / 16 * 16 : 0;
  auto bytes = [&](int t) { return 2 * t * pl.head_dim * es + 2 * t * zr + 4 * t; };
  int t = kGnTileMax;
  while (t > 1 && bytes(t) > kGnLdsBudget) t /= 2;
  *tile = t;
  *zrow = zr;
  *lds = bytes(t);
}

template <class E, int DH, int G>
static hipError_t launch_generic_t(const DecodePlan& pl, const DecodeArgs& a, int phase, hipStream_t st) {
  if ((phase & 1) && pl.n_splits > 0) {
    GnParams kp;
    kp.k_s = a.k_s; kp.v_s = a.v_s; kp.z_k = a.z_k; kp.z_v = a.z_v;
    kp.seq_lens = a.seq_lens; kp.q = a.q; kp.b_k = a.b_k;
    kp.scale_log2 = a.scale_log2;
    kp.heads = pl.heads; kp.rank = pl.rank; kp.max_len = pl.max_len; kp.split_tokens = pl.split_tokens;
    kp.partials = pl.partials; kp.capacity = pl.capacity;
    kp.ws_ml = a.ws_ml; kp.ws_acc = a.ws_acc;
    int lds = 0;
    generic_tile(pl, G, &kp.tile, &kp.zrow, &lds);
    constexpr int HW = kGnThreads / G;
    const dim3 grid(unsigned(pl.n_splits), unsigned(pl.batch), unsigned((pl.heads + HW - 1) / HW));
    hipLaunchKernelGGL((decode_generic_kernel<E, DH, G>), grid, dim3(kGnThreads), size_t(lds), st, kp);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!(phase & 2)) return hipSuccess;
  hipLaunchKernelGGL((decode_merge_generic_kernel<E>), dim3(pl.heads, pl.batch), dim3(kGnThreads), 0, st, a.ws_ml,
                     a.ws_acc, a.seq_lens, a.b_v, a.out, pl.heads, pl.head_dim, pl.rank, pl.partials,
                     pl.split_tokens, pl.max_len);
  return hipGetLastError();
}

template <class E, int DH>
static hipError_t launch_generic_g(const DecodePlan& pl, const DecodeArgs& a, int phase, hipStream_t st) {
  switch (generic_lanes_per_head(pl.heads, DH)) {
    case 8: return launch_generic_t<E, DH, 8>(pl, a, phase, st);
    case 16: return launch_generic_t<E, DH, 16>(pl, a, phase, st);
    case 32:
      if constexpr (DH >= 32) return launch_generic_t<E, DH, 32>(pl, a, phase, st);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_generic(const DecodePlan& pl, const DecodeArgs& a, int phase, hipStream_t st) {
#define LRKV_GN(DHV)                                                                                   \
  if (pl.head_dim == DHV)                                                                              \
    return pl.dtype == 1 ? launch_generic_g<BF16, DHV>(pl, a, phase, st) : launch_generic_g<F32, DHV>(pl, a, phase, st);
  LRKV_GN(16) LRKV_GN(32) LRKV_GN(64) LRKV_GN(128)
#undef LRKV_GN
  return hipErrorInvalidValue;
}

}  // namespace lrkv
