// LRKV causal prefill on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16).
//
// Method (Low-Rank Key Value Attention, slide discussion of arXiv:2601.11471v3):
// with L fresh tokens, every query row i of head h attends to keys j <= i
// (slide "Compute logits without expanding historical keys", Eq. (6), causal
// mask) through the absorbed forms
//   S = scale * [Q_h | Q_h B^K_h] . [K_s | R^K_h]^T           (inner dim d_h + r)
//   [O_s | O_z] = softmax(S) . [V_s | R^V_h]
//   O = O_s + O_z (B^V_h)^T, normalised by the softmax sum   (Eq. (7)).
// Per-head keys and values are never formed; the shared K_s/V_s tiles staged
// in LDS serve the four heads of a workgroup.
//
// Work decomposition: a workgroup is 4 wave64, one head each (heads 4g..4g+3)
// over the same 32 query rows; key tiles of 32 tokens run from 0 to the
// diagonal.  Each wave computes, per key tile:
//   S^T (32 tokens x 32 queries) = Kaug (32 x Daug) . Qaug^T (Daug x 32),
//   Daug = d_h + r rounded up to 16: (d_h + r)/16 MFMAs with A = key rows from
//   LDS and B = the wave's query rows held in registers;
//   online softmax per query (a lane owns one query column: 16 tokens, the
//   other 16 are in lane ^ 32);
//   O^T (features x 32 queries) += Vaug^T . P^T: P^T is reused directly from
//   the S^T accumulators as the B operand (tokens inside each 16-token chunk
//   are taken in the order the accumulator layout provides, and the value
//   tile is stored in LDS transposed with its token columns in that order).
// The absorbed query Q B^K_h and the residual up-projection O_z (B^V_h)^T are
// MFMA products too.  Softmax runs in fp32 in the log2 domain; P, the absorbed
// query and O_z enter MFMAs rounded to bf16.
#include "lrkv_device.h"
#include "lrkv_internal.h"

namespace lrkv {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int kPfWaves = 4;                 // heads per workgroup
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfTile = 32;                 // key tokens per tile, query rows per wave
constexpr float kPfStale = 8.f;             // running-max refresh threshold (log2 units)

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8_t, v); }

// Position of token u (0..15) of a 16-token chunk in the MFMA k-slot order
// that the 32x32 accumulator layout produces: lanes 0-31 carry tokens
// {0-3, 8-11}, lanes 32-63 carry {4-7, 12-15}.
__device__ __forceinline__ int kslot_pos(int u) { return (u & 3) | ((u >> 3) << 2) | (((u >> 2) & 1) << 3); }

template <int DH, int R>
struct PrefillShape {
  static constexpr int RK = (R + 15) / 16 * 16;          // latent dims padded for the K-dim chunks
  static constexpr int KCH = DH / 16 + RK / 16;           // 16-wide chunks of the augmented key
  static constexpr int VBLK = DH / 32 + (R > 0 ? 1 : 0);  // 32-row blocks of the augmented value
  static constexpr int K_STRIDE = DH * 2 + 16;            // LDS row of a shared key (padded)
  static constexpr int ZK_STRIDE = (R > 0 ? R * 2 : 16) + 16;   // LDS row of one head's key latent
  static constexpr int VT_STRIDE = kPfTile * 2 + 16;      // LDS row of the transposed value tile
  static constexpr int S_K = kPfTile * K_STRIDE;
  static constexpr int S_ZK = kPfWaves * kPfTile * ZK_STRIDE;
  static constexpr int S_VT = DH * VT_STRIDE;
  static constexpr int S_ZVT = kPfWaves * (R > 0 ? R : 1) * VT_STRIDE;
  static constexpr int STAGE = S_K + S_ZK + S_VT + S_ZVT;
  // 16-byte chunks staged per tile
  static constexpr int K_CHUNKS = kPfTile * DH / 8;
  static constexpr int Z_CHUNKS = kPfTile * kPfWaves * R / 8;
  static constexpr int K_PER = (K_CHUNKS + kPfThreads - 1) / kPfThreads;
  static constexpr int Z_PER = (Z_CHUNKS + kPfThreads - 1) / kPfThreads;
  static_assert(DH % 32 == 0 && R <= 32 && R % 8 == 0, "prefill envelope");
};

struct PrefillKernelParams {
  const uint16_t* q; const uint16_t* k_s; const uint16_t* v_s; const uint16_t* z_k; const uint16_t* z_v;
  const uint16_t* b_k; const uint16_t* b_v;
  uint16_t* out;
  int heads, seq_len, n_qblocks;
  float scale_log2;
};

// Registers holding one key tile on its way from HBM to LDS.
template <class P>
struct PfStage {
  u32x4 k[P::K_PER], v[P::K_PER], zk[P::Z_PER > 0 ? P::Z_PER : 1], zv[P::Z_PER > 0 ? P::Z_PER : 1];
};

// Load key tile `kt` (tokens 32kt..32kt+31, clamped to the last token) of
// sequence b for heads [4hg, 4hg+4).
template <int DH, int R>
__device__ __forceinline__ void pf_load(PfStage<PrefillShape<DH, R>>& st, const PrefillKernelParams& p, int b, int hg,
                                        int kt, int tid) {
  using P = PrefillShape<DH, R>;
  const int L = p.seq_len, H = p.heads;
#pragma unroll
  for (int i = 0; i < P::K_PER; ++i) {
    const int c = tid + i * kPfThreads;
    if (c < P::K_CHUNKS) {
      const int t = min(kt * kPfTile + c % kPfTile, L - 1), ch = c / kPfTile;   // token fastest across lanes
      const size_t row = (size_t(b) * L + t) * DH + ch * 8;
      st.k[i] = *reinterpret_cast<const u32x4*>(p.k_s + row);
      st.v[i] = *reinterpret_cast<const u32x4*>(p.v_s + row);
    }
  }
  if constexpr (R > 0) {
#pragma unroll
    for (int i = 0; i < P::Z_PER; ++i) {
      const int c = tid + i * kPfThreads;                 // (token, head in group, 8-dim chunk)
      if (c < P::Z_CHUNKS) {
        const int t = min(kt * kPfTile + c % kPfTile, L - 1), rem = c / kPfTile;     // token fastest
        const int hh = min(hg * kPfWaves + rem / (R / 8), H - 1), ch = rem % (R / 8);
        const size_t off = ((size_t(b) * L + t) * H + hh) * R + ch * 8;
        st.zk[i] = *reinterpret_cast<const u32x4*>(p.z_k + off);
        st.zv[i] = *reinterpret_cast<const u32x4*>(p.z_v + off);
      }
    }
  }
}

// Write a staged tile to LDS: keys row-major, values transposed (feature rows,
// token columns in MFMA k-slot order).
template <int DH, int R>
__device__ __forceinline__ void pf_store(const PfStage<PrefillShape<DH, R>>& st, unsigned char* buf, int tid) {
  using P = PrefillShape<DH, R>;
  unsigned char* sK = buf;
  unsigned char* sZK = buf + P::S_K;
  unsigned char* sVT = sZK + P::S_ZK;
  unsigned char* sZVT = sVT + P::S_VT;
#pragma unroll
  for (int i = 0; i < P::K_PER; ++i) {
    const int c = tid + i * kPfThreads;
    if (c < P::K_CHUNKS) {
      const int t = c % kPfTile, ch = c / kPfTile;
      *reinterpret_cast<u32x4*>(sK + t * P::K_STRIDE + ch * 16) = st.k[i];
      const int col = ((t >> 4) << 4) | kslot_pos(t & 15);
      const uint32_t w[4] = {st.v[i].x, st.v[i].y, st.v[i].z, st.v[i].w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<uint16_t*>(sVT + (ch * 8 + e) * P::VT_STRIDE + col * 2) =
            uint16_t((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu));
    }
  }
  if constexpr (R > 0) {
#pragma unroll
    for (int i = 0; i < P::Z_PER; ++i) {
      const int c = tid + i * kPfThreads;
      if (c < P::Z_CHUNKS) {
        const int t = c % kPfTile, rem = c / kPfTile, w = rem / (R / 8), ch = rem % (R / 8);
        *reinterpret_cast<u32x4*>(sZK + (w * kPfTile + t) * P::ZK_STRIDE + ch * 16) = st.zk[i];
        const int col = ((t >> 4) << 4) | kslot_pos(t & 15);
        const uint32_t wv[4] = {st.zv[i].x, st.zv[i].y, st.zv[i].z, st.zv[i].w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          *reinterpret_cast<uint16_t*>(sZVT + ((w * R) + ch * 8 + e) * P::VT_STRIDE + col * 2) =
              uint16_t((e & 1) ? (wv[e >> 1] >> 16) : (wv[e >> 1] & 0xffffu));
      }
    }
  }
}

template <int DH, int R>
__global__ __attribute__((amdgpu_flat_work_group_size(kPfThreads, kPfThreads), amdgpu_waves_per_eu(2)))
void prefill_kernel(PrefillKernelParams p) {
  using P = PrefillShape<DH, R>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, half = lane >> 5;
  const int qb = p.n_qblocks - 1 - int(blockIdx.x);      // heaviest query blocks first
  const int hg = blockIdx.y, b = blockIdx.z;
  const int H = p.heads, L = p.seq_len;
  const int h = hg * kPfWaves + wave;
  const bool head_ok = h < H;
  const int hh = head_ok ? h : H - 1;
  const int q0 = qb * kPfTile;
  const int qrow = min(q0 + n, L - 1);

  // ---- query rows (B operands, K-dim = features): lane (query n, half) ----
  bf16x8_t qop[P::KCH];
  {
    const uint16_t* qr = p.q + ((size_t(b) * L + qrow) * H + hh) * DH;
#pragma unroll
    for (int c = 0; c < DH / 16; ++c) qop[c] = as_bf16x8(*reinterpret_cast<const u32x4*>(qr + 16 * c + 8 * half));
  }
  if constexpr (R > 0) {
    // absorbed query, transposed: (latent j x query n) = (B^K_h)^T (j x d) . Q^T (d x n), rows j >= R zero
    f32x16_t qt = {};
    const uint16_t* bk = p.b_k + size_t(hh) * DH * R;
#pragma unroll
    for (int c = 0; c < DH / 16; ++c) {
      bf16x8_t a;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint16_t v = n < R ? bk[size_t(16 * c + 8 * half + i) * R + n] : uint16_t(0);
        a[i] = __builtin_bit_cast(__bf16, v);
      }
      qt = mfma32(a, qop[c], qt);
    }
    // accumulator rows 8(r/4)+4half+r%4 are the latent dims this lane feeds as
    // k-slots of the latent chunks (same order as the key latents in LDS)
#pragma unroll
    for (int c = 0; c < P::RK / 16; ++c) {
      bf16x8_t v;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (__bf16)qt[8 * c + i];
      qop[DH / 16 + c] = v;
    }
  }

  f32x16_t oacc[P::VBLK];
#pragma unroll
  for (int f = 0; f < P::VBLK; ++f) oacc[f] = f32x16_t{};
  float m = -INFINITY, lsum = 0.f;

  PfStage<P> st;
  pf_load<DH, R>(st, p, b, hg, 0, tid);
  pf_store<DH, R>(st, smem, tid);
  __syncthreads();

  for (int kt = 0; kt <= qb; ++kt) {
    if (kt < qb) pf_load<DH, R>(st, p, b, hg, kt + 1, tid);
    const unsigned char* buf = smem + (kt & 1) * P::STAGE;
    const unsigned char* sK = buf;
    const unsigned char* sZK = buf + P::S_K;
    const unsigned char* sVT = sZK + P::S_ZK;
    const unsigned char* sZVT = sVT + P::S_VT;

    // S^T = Kaug . Qaug^T: lane (query n, half) gets tokens 8(r/4)+4half+r%4.
    // All key operands are read from LDS first, then the MFMAs run back to back.
    u32x4 ka[P::KCH];
#pragma unroll
    for (int c = 0; c < DH / 16; ++c)
      ka[c] = *reinterpret_cast<const u32x4*>(sK + n * P::K_STRIDE + (16 * c + 8 * half) * 2);
    if constexpr (R > 0) {
#pragma unroll
      for (int c = 0; c < P::RK / 16; ++c) {
        // key latent k-slots in accumulator order: lanes 0-31 dims {0-3, 8-11}, lanes 32-63 {4-7, 12-15}
        const unsigned char* zr = sZK + (wave * kPfTile + n) * P::ZK_STRIDE + c * 32;
        const uint2 lo = *reinterpret_cast<const uint2*>(zr + half * 8);
        const uint2 hi = *reinterpret_cast<const uint2*>(zr + 16 + half * 8);
        ka[DH / 16 + c] = (16 * c + 8 >= R) ? u32x4{lo.x, lo.y, 0u, 0u}     // R = 8: dims 8..15 are padding
                                            : u32x4{lo.x, lo.y, hi.x, hi.y};
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x16_t s = {};
#pragma unroll
    for (int c = 0; c < P::KCH; ++c) s = mfma32(as_bf16x8(ka[c]), qop[c], s);
    // value operands for this tile, read while the softmax runs
    u32x4 va[P::VBLK][2];
#pragma unroll
    for (int f = 0; f < DH / 32; ++f)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        va[f][c] = *reinterpret_cast<const u32x4*>(sVT + (32 * f + n) * P::VT_STRIDE + (16 * c + 8 * half) * 2);
    if constexpr (R > 0) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        va[DH / 32][c] = u32x4{0u, 0u, 0u, 0u};
        if (n < R) va[DH / 32][c] = *reinterpret_cast<const u32x4*>(sZVT + (wave * R + n) * P::VT_STRIDE + (16 * c + 8 * half) * 2);
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // online softmax (log2 domain) for query q0+n.  Only the diagonal tile and
    // a tile reaching past the sequence end need the mask.  The running max is
    // refreshed only when a score exceeds it by more than kPfStale (log2
    // units): weights then stay <= 2^kPfStale, and since the sum and the
    // output use the same reference the result is unchanged.
    float sv[16];
    float mx = -INFINITY;
    const bool masked = (kt == qb) || (kt * kPfTile + kPfTile > L);
    if (masked) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = kt * kPfTile + 8 * (r >> 2) + 4 * half + (r & 3);
        sv[r] = (tok <= q0 + n && tok < L) ? s[r] : -INFINITY;
        mx = fmaxf(mx, sv[r]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sv[r] = s[r];
        mx = fmaxf(mx, sv[r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * p.scale_log2;   // finite: token kt*32 <= q0 + n always
    if (mx > m + kPfStale) {
      const float alpha = fast_exp2(m - mx);               // 0 on the first tile (m = -inf)
      m = mx;
      lsum *= alpha;
#pragma unroll
      for (int f = 0; f < P::VBLK; ++f) oacc[f] *= alpha;
    }
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sv[r] = fast_exp2(__builtin_fmaf(sv[r], p.scale_log2, -m));
      ps += sv[r];
    }
    lsum += ps + __shfl_xor(ps, 32);
    bf16x8_t pb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[c][i] = (__bf16)sv[8 * c + i];

    // O^T += Vaug^T . P^T
#pragma unroll
    for (int f = 0; f < P::VBLK; ++f)
#pragma unroll
      for (int c = 0; c < 2; ++c) oacc[f] = mfma32(as_bf16x8(va[f][c]), pb[c], oacc[f]);

    if (kt < qb) pf_store<DH, R>(st, smem + ((kt + 1) & 1) * P::STAGE, tid);
    __syncthreads();
  }

  if (!head_ok) return;
  // ---- epilogue: O_s += B^V_h . O_z^T, then divide by the softmax sum ----
  if constexpr (R > 0) {
#pragma unroll
    for (int c = 0; c < P::RK / 16; ++c) {
      bf16x8_t bz;                                          // O_z^T k-slots, accumulator order
#pragma unroll
      for (int i = 0; i < 8; ++i) bz[i] = (__bf16)oacc[DH / 32][8 * c + i];
#pragma unroll
      for (int f = 0; f < DH / 32; ++f) {
        const uint16_t* bv = p.b_v + (size_t(hh) * DH + 32 * f + n) * R + 16 * c;
        const uint2 lo = *reinterpret_cast<const uint2*>(bv + 4 * half);
        uint2 hi = {0u, 0u};
        if (16 * c + 8 < R) hi = *reinterpret_cast<const uint2*>(bv + 8 + 4 * half);
        oacc[f] = mfma32(as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y}), bz, oacc[f]);
      }
    }
  }
  if (q0 + n >= L) return;
  const float inv = 1.f / lsum;
  uint16_t* orow = p.out + ((size_t(b) * L + q0 + n) * H + h) * DH;
#pragma unroll
  for (int f = 0; f < DH / 32; ++f)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 32 * f + 8 * j + 4 * half;
      const uint32_t lo = pack_bf16x2(oacc[f][4 * j] * inv, oacc[f][4 * j + 1] * inv);
      const uint32_t hi = pack_bf16x2(oacc[f][4 * j + 2] * inv, oacc[f][4 * j + 3] * inv);
      *reinterpret_cast<uint2*>(orow + d) = make_uint2(lo, hi);
    }
}

template <int DH, int R>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  using P = PrefillShape<DH, R>;
  PrefillKernelParams kp;
  kp.q = static_cast<const uint16_t*>(a.q);
  kp.k_s = static_cast<const uint16_t*>(a.k_s);
  kp.v_s = static_cast<const uint16_t*>(a.v_s);
  kp.z_k = static_cast<const uint16_t*>(a.z_k);
  kp.z_v = static_cast<const uint16_t*>(a.z_v);
  kp.b_k = static_cast<const uint16_t*>(a.b_k);
  kp.b_v = static_cast<const uint16_t*>(a.b_v);
  kp.out = static_cast<uint16_t*>(a.out);
  kp.heads = a.heads;
  kp.seq_len = a.seq_len;
  kp.n_qblocks = (a.seq_len + kPfTile - 1) / kPfTile;
  kp.scale_log2 = a.scale_log2;
  const dim3 grid(kp.n_qblocks, (a.heads + kPfWaves - 1) / kPfWaves, a.batch);
  const size_t lds = 2 * size_t(P::STAGE);
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<DH, R>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((prefill_kernel<DH, R>), grid, dim3(kPfThreads), lds, st, kp);
  return hipGetLastError();
}

bool prefill_supported(int dtype, int head_dim, int rank, int heads) {
  return dtype == 1 && (head_dim == 64 || head_dim == 128) &&
         (rank == 0 || rank == 8 || rank == 16 || rank == 32) && heads >= 1;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
#define LRKV_PF(DHV, RV) \
  if (a.head_dim == DHV && a.rank == RV) return launch_prefill_t<DHV, RV>(a, st);
  LRKV_PF(64, 0) LRKV_PF(64, 8) LRKV_PF(64, 16) LRKV_PF(64, 32)
  LRKV_PF(128, 0) LRKV_PF(128, 8) LRKV_PF(128, 16) LRKV_PF(128, 32)
#undef LRKV_PF
  return hipErrorInvalidValue;
}

}  // namespace lrkv
