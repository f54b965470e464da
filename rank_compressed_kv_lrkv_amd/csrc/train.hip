// LRKV attention backward for training, on bf16 MFMA (gfx950
// v_mfma_f32_32x32x16_bf16), fp32 gradients.
//
// Method (Low-Rank Key Value Attention, slide discussion of arXiv:2601.11471v3):
// training learns W_shared, U_h and B_h together (slide "Training learns the
// base and residuals together"); a layer's attention is the causal prefill of
// slides "Compute logits without expanding historical keys", Eq. (6), and
// "Aggregate values before the residual up-projection", Eq. (7).  For a loss
// with upstream gradient dO, per head h (K_h = K_s + Z^K_h B^K_h^T,
// V_h = V_s + Z^V_h B^V_h^T, causal softmax P = exp(S - lse)):
//   dV_h = P^T dO,  dP = dO V_h^T,  dS = P o (dP - D),  D = rowsum(dO o O),
//   dQ = scale dS K_h,  dK_h = scale dS^T Q,
//   dK_s = sum_h dK_h,  dZ^K_h = dK_h B^K_h,  dB^K_h = dK_h^T Z^K_h  (V alike).
// Every product runs in the absorbed form, as in the forward pass: with the
// augmented rows Kaug = [K_s | Z^K_h], Vaug = [V_s | Z^V_h], Qaug = [Q | Q B^K_h]
// and dOaug = [dO | dO B^V_h],
//   S = scale Qaug Kaug^T,   dP = dOaug Vaug^T,
//   [dK_h | dZ^K_h] = scale dS^T Qaug,   [dV_h | dZ^V_h] = P^T dOaug,
//   dQ = scale (dS K_s + (dS Z^K_h) B^K_h^T),
// so per-head keys and values are never formed.
//
// Kernels (one backward call):
//   train_prep_kernel   Q B^K_h and dO B^V_h (bf16), D and log2-scaled lse;
//   train_dq_kernel     per (query block, 4 heads): keys streamed through
//                       LDS, S^T and dP^T on MFMA (lane = query), dQ^T
//                       accumulated as Kaug^T dS^T, B^K epilogue;
//   train_dkv_kernel    per (key block, 4 heads): queries and dO streamed
//                       through LDS, S and dP on MFMA (lane = key), Kaug and
//                       Vaug gradients accumulated as dS^T Qaug and P^T dOaug;
//                       per-head-group partial sums of dK_s, dV_s and
//                       per-key-block partial dB^K, dB^V;
//   train_reduce_kernel the partial sums added up (deterministic order).
// P and dS enter MFMAs rounded to bf16; everything is accumulated in fp32.
#include "lrkv_device.h"
#include "lrkv_internal.h"

namespace lrkv {

namespace {

constexpr int kTrWaves = 4;                 // heads per workgroup, one per wave
constexpr int kTrThreads = 64 * kTrWaves;
constexpr int kTrTile = 32;                 // tokens per block

template <int DH, int R>
struct TrShape {
  static constexpr int RK = (R + 15) / 16 * 16;           // latent dims padded to the K-dim chunk
  static constexpr int KCH = DH / 16 + RK / 16;            // 16-wide chunks of an augmented row
  static constexpr int ZCH = RK / 16 > 0 ? RK / 16 : 1;
  static constexpr int VBLK = DH / 32 + (R > 0 ? 1 : 0);   // 32-row blocks of an augmented row
  static constexpr int RB = DH * 2, CR = RB / 16;          // bytes and 16-byte chunks of a d_h row
  static constexpr int ZB = kTrWaves * R * 2, CZ = ZB / 16; // the 4 heads' latents of one token
  static constexpr int ROWS = kTrTile * RB;                 // a 32-row tile of d_h rows
  static constexpr int LATS = kTrTile * ZB;                 // a 32-token tile of latents
  static constexpr int LDS_DQ = 2 * (ROWS + LATS);                     // dQ kernel: key and value tiles
  static constexpr int LDS_RED = kTrWaves * (DH / 32) * 16 * 64 * 4;    // dK/dV kernel: head-sum exchange
  static constexpr int LDS_KV = 2 * (kTrWaves * ROWS + LATS) > LDS_RED ? 2 * (kTrWaves * ROWS + LATS) : LDS_RED;
  static_assert(DH % 32 == 0 && R <= 32 && R % 8 == 0, "training envelope");
  static_assert(CR >= 4 && (R == 0 || CZ >= 4), "swizzle needs 4 chunks per row");
};

struct TrParams {
  const uint16_t* q; const uint16_t* k_s; const uint16_t* v_s; const uint16_t* z_k; const uint16_t* z_v;
  const uint16_t* b_k; const uint16_t* b_v;
  const uint16_t* out; const float* lse; const uint16_t* d_out;
  float* dq; float* dz_k; float* dz_v;
  // workspace
  uint16_t* qb; uint16_t* dob;      // [B][L][H][R] bf16: Q B^K_h and dO B^V_h
  float* lse2; float* dd;           // [B][H][Lp]: lse * log2(e) and rowsum(dO o O); rows >= L hold 0
  float* dks_part; float* dvs_part; // [n_hgroups][B][L][DH]
  float* dbk_part; float* dbv_part; // [B][n_kblocks][H][DH][R]
  int batch, heads, seq_len, seq_pad, n_blocks, n_hgroups;
  float scale, scale_log2;
};

// Copy a 32-row tile into LDS: row t (t < 32) is `chunks` 16-byte chunks at
// src + t * stride (bytes); chunk ch of row t lands at position
// ch ^ lds_swz(t, chunks).  Rows t >= valid are zero.  All threads of the
// workgroup take part.
__device__ __forceinline__ void tr_fill(unsigned char* dst, const unsigned char* src, size_t stride, int chunks,
                                        int valid, int tid) {
  for (int idx = tid; idx < kTrTile * chunks; idx += kTrThreads) {
    const int t = idx / chunks, ch = idx % chunks;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (t < valid) v = *reinterpret_cast<const u32x4*>(src + size_t(t) * stride + size_t(ch) * 16);
    *reinterpret_cast<u32x4*>(dst + t * chunks * 16 + (ch ^ lds_swz(t, chunks)) * 16) = v;
  }
}

// Per-lane LDS offsets of the operand reads (the layouts of the forward
// prefill kernel): row-major 16-byte reads of chunk c of row n (koff) and of
// this wave's head's latent chunk c (zoff); transpose reads of a 16-token
// chunk of d_h rows (voff) and of latents (zvoff), giving lane (feature n,
// half) the tokens {4half..+3, 8+4half..+3} of the chunk, the k-slot order
// of an MFMA accumulator used as the other operand.
template <int DH, int R>
struct TrOffsets {
  using P = TrShape<DH, R>;
  int koff[DH / 16], zoff[P::ZCH], voff[DH / 32][2], zvoff[2][2];
  __device__ __forceinline__ TrOffsets(int lane, int wave) {
    const int n = lane & 31, half = lane >> 5;
#pragma unroll
    for (int c = 0; c < DH / 16; ++c) koff[c] = n * P::RB + ((2 * c + half) ^ lds_swz(n, P::CR)) * 16;
#pragma unroll
    for (int c = 0; c < P::ZCH; ++c) {
      zoff[c] = 0;
      if constexpr (R > 0) {
        const int ch = wave * (R / 8) + (R == 8 ? 0 : 2 * c + half);
        zoff[c] = n * P::ZB + (ch ^ lds_swz(n, P::CZ)) * 16;
      }
    }
    const int tr_tok = 4 * half + ((lane >> 2) & 3);
#pragma unroll
    for (int f = 0; f < DH / 32; ++f) {
      const int ch = 4 * f + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = tr_tok + 8 * j;
        voff[f][j] = row * P::RB + (ch ^ lds_swz(row, P::CR)) * 16 + 8 * (lane & 1);
      }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        zvoff[c][j] = 0;
        if constexpr (R > 0) {
          const int feat = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
          const int byte = wave * R * 2 + (feat < R ? feat : 0) * 2;   // rows >= R: any valid row (unused)
          const int row = 16 * c + tr_tok + 8 * j;
          zvoff[c][j] = row * P::ZB + ((byte / 16) ^ lds_swz(row, P::CZ)) * 16 + byte % 16;
        }
      }
  }
};

// Row-major operand chunk c of an augmented row: d_h part from `rows`, latent
// part from `lats` (this wave's head).
template <int DH, int R>
__device__ __forceinline__ bf16x8_t tr_row_chunk(const unsigned char* rows, const unsigned char* lats,
                                                 const TrOffsets<DH, R>& o, int c, int half) {
  if (c < DH / 16) return as_bf16x8(*reinterpret_cast<const u32x4*>(rows + o.koff[c]));
  if constexpr (R > 0) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(lats + o.zoff[c - DH / 16]);
    return as_bf16x8((R == 8 && half) ? u32x4{0u, 0u, 0u, 0u} : v);   // R = 8: dims 8..15 are padding
  }
  return as_bf16x8(u32x4{0u, 0u, 0u, 0u});
}

// Transposed operand of 32-row block f of an augmented row, 16-token chunk c.
template <int DH, int R>
__device__ __forceinline__ bf16x8_t tr_col_chunk(const unsigned char* rows, const unsigned char* lats,
                                                 const TrOffsets<DH, R>& o, int f, int c) {
  if (f < DH / 32) {
    const uint2 lo = lds_read_tr16(rows + 16 * c * TrShape<DH, R>::RB + o.voff[f][0]);
    const uint2 hi = lds_read_tr16(rows + 16 * c * TrShape<DH, R>::RB + o.voff[f][1]);
    return as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
  }
  const uint2 lo = lds_read_tr16(lats + o.zvoff[c][0]), hi = lds_read_tr16(lats + o.zvoff[c][1]);
  return as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
}

// A 16-byte operand of an augmented row straight from global memory: dims
// 16c + 8half..+7 of [row (d_h) | lat (R)].
template <int DH, int R>
__device__ __forceinline__ bf16x8_t tr_global_chunk(const uint16_t* row, const uint16_t* lat, int c, int half) {
  if (c < DH / 16) return as_bf16x8(*reinterpret_cast<const u32x4*>(row + 16 * c + 8 * half));
  if constexpr (R > 0) {
    if (R == 8 && half) return as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    return as_bf16x8(*reinterpret_cast<const u32x4*>(lat + 16 * (c - DH / 16) + 8 * half));
  }
  return as_bf16x8(u32x4{0u, 0u, 0u, 0u});
}

}  // namespace

// ---------------------------------------------------------------------------
// Per token row: Q B^K_h and dO B^V_h for every head (bf16), D = rowsum(dO o O)
// and lse * log2(e) (fp32, [B][H][Lp]; the padding rows get 0).
// ---------------------------------------------------------------------------
template <int DH, int R>
__global__ __launch_bounds__(kTrThreads) void train_prep_kernel(TrParams p) {
  const int row = int(blockIdx.x), tid = threadIdx.x;
  const int H = p.heads, L = p.seq_len;
  const int b = row / L, i = row % L;
  const uint16_t* qr = p.q + size_t(row) * H * DH;
  const uint16_t* dr = p.d_out + size_t(row) * H * DH;
  const uint16_t* orow = p.out + size_t(row) * H * DH;
  if constexpr (R > 0) {
    for (int idx = tid; idx < 2 * H * R; idx += kTrThreads) {
      const int which = idx / (H * R), hj = idx % (H * R), h = hj / R, j = hj % R;
      const uint16_t* x = (which ? dr : qr) + h * DH;
      const uint16_t* w = (which ? p.b_v : p.b_k) + size_t(h) * DH * R + j;
      float acc = 0.f;
#pragma unroll 8
      for (int d = 0; d < DH; ++d) acc = __builtin_fmaf(bf16_to_f32(x[d]), bf16_to_f32(w[size_t(d) * R]), acc);
      (which ? p.dob : p.qb)[size_t(row) * H * R + hj] = f32_to_bf16(acc);
    }
  }
  for (int h = tid; h < H; h += kTrThreads) {
    float acc = 0.f;
    for (int d = 0; d < DH; ++d) acc = __builtin_fmaf(bf16_to_f32(dr[h * DH + d]), bf16_to_f32(orow[h * DH + d]), acc);
    const size_t o = (size_t(b) * H + h) * p.seq_pad + i;
    p.dd[o] = acc;
    p.lse2[o] = p.lse[size_t(row) * H + h] * 1.4426950408889634f;
    if (i == L - 1)
      for (int t = L; t < p.seq_pad; ++t) {
        p.dd[o + (t - i)] = 0.f;
        p.lse2[o + (t - i)] = 0.f;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ: workgroup = (query block, 4 heads, sequence), one head per wave.
// ---------------------------------------------------------------------------
template <int DH, int R>
__global__ __launch_bounds__(kTrThreads) void train_dq_kernel(TrParams p) {
  using P = TrShape<DH, R>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  unsigned char* const krows = smem;
  unsigned char* const klats = smem + P::ROWS;
  unsigned char* const vrows = klats + P::LATS;
  unsigned char* const vlats = vrows + P::ROWS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, half = lane >> 5;
  const int per_level = p.n_hgroups * p.batch;
  const int qb = p.n_blocks - 1 - int(blockIdx.x) / per_level;    // heaviest first
  const int rem = int(blockIdx.x) % per_level;
  const int b = rem % p.batch, hg = rem / p.batch;
  const int H = p.heads, L = p.seq_len;
  const int h = hg * kTrWaves + wave;
  const int q0 = qb * kTrTile;
  const int qrow = min(q0 + n, L - 1);
  const int kt_last = min(q0 + kTrTile - 1, L - 1) / kTrTile;
  const TrOffsets<DH, R> o(lane, wave);

  // B operands: the wave's query rows [Q | Q B^K_h] and [dO | dO B^V_h]
  bf16x8_t qop[P::KCH], dop[P::KCH];
  {
    const size_t r = size_t(b) * L + qrow;
#pragma unroll
    for (int c = 0; c < P::KCH; ++c) {
      qop[c] = tr_global_chunk<DH, R>(p.q + (r * H + h) * DH, p.qb + (r * H + h) * R, c, half);
      dop[c] = tr_global_chunk<DH, R>(p.d_out + (r * H + h) * DH, p.dob + (r * H + h) * R, c, half);
    }
  }
  const size_t lrow = (size_t(b) * H + h) * p.seq_pad + qrow;
  const float lse2 = p.lse2[lrow], dd = p.dd[lrow];

  f32x16_t acc[P::VBLK];
#pragma unroll
  for (int f = 0; f < P::VBLK; ++f) acc[f] = f32x16_t{};
  for (int kt = 0; kt <= kt_last; ++kt) {
    const int t0 = kt * kTrTile, valid = min(kTrTile, L - t0);
    const size_t tok = size_t(b) * L + t0;
    tr_fill(krows, reinterpret_cast<const unsigned char*>(p.k_s + tok * DH), P::RB, P::CR, valid, tid);
    tr_fill(vrows, reinterpret_cast<const unsigned char*>(p.v_s + tok * DH), P::RB, P::CR, valid, tid);
    if constexpr (R > 0) {
      tr_fill(klats, reinterpret_cast<const unsigned char*>(p.z_k + (tok * H + hg * kTrWaves) * R), size_t(H) * R * 2,
              P::CZ, valid, tid);
      tr_fill(vlats, reinterpret_cast<const unsigned char*>(p.z_v + (tok * H + hg * kTrWaves) * R), size_t(H) * R * 2,
              P::CZ, valid, tid);
    }
    __syncthreads();
    // S^T = Kaug Qaug^T and dP^T = Vaug dOaug^T: lane (query n, half) holds
    // keys 8(i/4) + 4half + i%4
    f32x16_t s = {}, dp = {};
#pragma unroll
    for (int c = 0; c < P::KCH; ++c) {
      s = mfma32(tr_row_chunk<DH, R>(krows, klats, o, c, half), qop[c], s);
      dp = mfma32(tr_row_chunk<DH, R>(vrows, vlats, o, c, half), dop[c], dp);
    }
    bf16x8_t pb[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = t0 + 8 * (i >> 2) + 4 * half + (i & 3);
      const bool ok = key <= q0 + n && key < L;
      const float pv = ok ? fast_exp2(__builtin_fmaf(s[i], p.scale_log2, -lse2)) : 0.f;
      pb[i >> 3][i & 7] = (__bf16)(pv * (dp[i] - dd));
    }
    // dQaug^T += Kaug^T dS^T
#pragma unroll
    for (int f = 0; f < P::VBLK; ++f)
#pragma unroll
      for (int c = 0; c < 2; ++c) acc[f] = mfma32(tr_col_chunk<DH, R>(krows, klats, o, f, c), pb[c], acc[f]);
    __syncthreads();
  }
  // dQ^T = scale (dQ_s^T + B^K_h dQ_z^T)
  if constexpr (R > 0) {
#pragma unroll
    for (int c = 0; c < P::RK / 16; ++c) {
      bf16x8_t bz;
#pragma unroll
      for (int i = 0; i < 8; ++i) bz[i] = (__bf16)acc[DH / 32][8 * c + i];
#pragma unroll
      for (int f = 0; f < DH / 32; ++f) {
        const uint16_t* bk = p.b_k + (size_t(h) * DH + 32 * f + n) * R + 16 * c;
        const uint2 lo = *reinterpret_cast<const uint2*>(bk + 4 * half);
        uint2 hi = {0u, 0u};
        if (16 * c + 8 < R) hi = *reinterpret_cast<const uint2*>(bk + 8 + 4 * half);
        acc[f] = mfma32(as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y}), bz, acc[f]);
      }
    }
  }
  if (q0 + n >= L) return;
  float* dqr = p.dq + ((size_t(b) * L + q0 + n) * H + h) * DH;
#pragma unroll
  for (int f = 0; f < DH / 32; ++f)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 32 * f + 8 * j + 4 * half;
      *reinterpret_cast<float4*>(dqr + d) = make_float4(acc[f][4 * j] * p.scale, acc[f][4 * j + 1] * p.scale,
                                                        acc[f][4 * j + 2] * p.scale, acc[f][4 * j + 3] * p.scale);
    }
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup = (key block, 4 heads, sequence), one head per wave.
// ---------------------------------------------------------------------------
template <int DH, int R>
__global__ __launch_bounds__(kTrThreads) void train_dkv_kernel(TrParams p) {
  using P = TrShape<DH, R>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  // query side: the 4 heads' Q rows, then [Q B^K] latents; dO side alike
  unsigned char* const qrows = smem;                               // 4 x ROWS
  unsigned char* const qlats = smem + kTrWaves * P::ROWS;
  unsigned char* const drows = qlats + P::LATS;                    // 4 x ROWS
  unsigned char* const dlats = drows + kTrWaves * P::ROWS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, half = lane >> 5;
  const int per_level = p.n_hgroups * p.batch;
  const int kb = int(blockIdx.x) / per_level;                      // key block 0 scans every query block
  const int rem = int(blockIdx.x) % per_level;
  const int b = rem % p.batch, hg = rem / p.batch;
  const int H = p.heads, L = p.seq_len;
  const int h = hg * kTrWaves + wave;
  const int k0 = kb * kTrTile;
  const int krow = min(k0 + n, L - 1);
  const TrOffsets<DH, R> o(lane, wave);

  // B operands: the wave's key rows [K_s | Z^K_h] and [V_s | Z^V_h] (lane = key n)
  bf16x8_t kop[P::KCH], vop[P::KCH];
  {
    const size_t r = size_t(b) * L + krow;
#pragma unroll
    for (int c = 0; c < P::KCH; ++c) {
      kop[c] = tr_global_chunk<DH, R>(p.k_s + r * DH, p.z_k + (r * H + h) * R, c, half);
      vop[c] = tr_global_chunk<DH, R>(p.v_s + r * DH, p.z_v + (r * H + h) * R, c, half);
    }
  }
  // accumulators C[key][feature], lane = feature column: [dK_h | dZ^K_h] / scale, [dV_h | dZ^V_h]
  f32x16_t dk[P::VBLK], dv[P::VBLK];
#pragma unroll
  for (int f = 0; f < P::VBLK; ++f) dk[f] = dv[f] = f32x16_t{};
  const int nqb = (L + kTrTile - 1) / kTrTile;
  for (int qb = kb; qb < nqb; ++qb) {
    const int q0 = qb * kTrTile, valid = min(kTrTile, L - q0);
    const size_t tok = size_t(b) * L + q0;
#pragma unroll
    for (int w = 0; w < kTrWaves; ++w) {
      const size_t hr = (tok * H + hg * kTrWaves + w) * DH;
      tr_fill(qrows + w * P::ROWS, reinterpret_cast<const unsigned char*>(p.q + hr), size_t(H) * DH * 2, P::CR, valid,
              tid);
      tr_fill(drows + w * P::ROWS, reinterpret_cast<const unsigned char*>(p.d_out + hr), size_t(H) * DH * 2, P::CR,
              valid, tid);
    }
    if constexpr (R > 0) {
      tr_fill(qlats, reinterpret_cast<const unsigned char*>(p.qb + (tok * H + hg * kTrWaves) * R), size_t(H) * R * 2,
              P::CZ, valid, tid);
      tr_fill(dlats, reinterpret_cast<const unsigned char*>(p.dob + (tok * H + hg * kTrWaves) * R), size_t(H) * R * 2,
              P::CZ, valid, tid);
    }
    __syncthreads();
    const unsigned char* qw = qrows + wave * P::ROWS;
    const unsigned char* dw = drows + wave * P::ROWS;
    // S = Qaug Kaug^T and dP = dOaug Vaug^T: lane (key n, half) holds queries
    // 8(i/4) + 4half + i%4
    f32x16_t s = {}, dp = {};
#pragma unroll
    for (int c = 0; c < P::KCH; ++c) {
      s = mfma32(tr_row_chunk<DH, R>(qw, qlats, o, c, half), kop[c], s);
      dp = mfma32(tr_row_chunk<DH, R>(dw, dlats, o, c, half), vop[c], dp);
    }
    // the 16 rows' lse and D: 4 runs of 4 consecutive queries
    const size_t lbase = (size_t(b) * H + h) * p.seq_pad + q0 + 4 * half;
    float lse2[16], dd[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 l4 = *reinterpret_cast<const float4*>(p.lse2 + lbase + 8 * j);
      const float4 d4 = *reinterpret_cast<const float4*>(p.dd + lbase + 8 * j);
      lse2[4 * j] = l4.x; lse2[4 * j + 1] = l4.y; lse2[4 * j + 2] = l4.z; lse2[4 * j + 3] = l4.w;
      dd[4 * j] = d4.x; dd[4 * j + 1] = d4.y; dd[4 * j + 2] = d4.z; dd[4 * j + 3] = d4.w;
    }
    bf16x8_t pp[2], ps[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int qi = q0 + 8 * (i >> 2) + 4 * half + (i & 3);
      const bool ok = k0 + n <= qi && qi < L && k0 + n < L;
      const float pv = ok ? fast_exp2(__builtin_fmaf(s[i], p.scale_log2, -lse2[i])) : 0.f;
      pp[i >> 3][i & 7] = (__bf16)pv;
      ps[i >> 3][i & 7] = (__bf16)(pv * (dp[i] - dd[i]));
    }
    // [dV_h | dZ^V_h] += P^T dOaug, [dK_h | dZ^K_h] / scale += dS^T Qaug
#pragma unroll
    for (int f = 0; f < P::VBLK; ++f)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        dv[f] = mfma32(pp[c], tr_col_chunk<DH, R>(dw, dlats, o, f, c), dv[f]);
        dk[f] = mfma32(ps[c], tr_col_chunk<DH, R>(qw, qlats, o, f, c), dk[f]);
      }
    __syncthreads();
  }
#pragma unroll
  for (int f = 0; f < P::VBLK; ++f) dk[f] *= p.scale;

  // ---- per-key gradients of this head: dZ^K_h, dZ^V_h (columns n < R) ----
  if constexpr (R > 0) {
    if (n < R) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 8 * (i >> 2) + 4 * half + (i & 3);
        if (key < L) {
          const size_t zo = ((size_t(b) * L + key) * H + h) * R + n;
          p.dz_k[zo] = dk[DH / 32][i];
          p.dz_v[zo] = dv[DH / 32][i];
        }
      }
    }
    // ---- dB^K_h, dB^V_h over this key block: C[d][j] = sum_key dK_h[key][d] Z^K[key][h][j] ----
    // A = dK_h^T (lane = feature row, k-slots = keys in accumulator order),
    // B = Z^K (lane = latent column n, the same keys).
    bf16x8_t zk[2], zv[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8) {
        const int i = 8 * c + s8;
        const int key = k0 + 8 * (i >> 2) + 4 * half + (i & 3);
        uint16_t zkv = 0, zvv = 0;
        if (n < R && key < L) {
          const size_t zo = ((size_t(b) * L + key) * H + h) * R + n;
          zkv = p.z_k[zo];
          zvv = p.z_v[zo];
        }
        zk[c][s8] = __builtin_bit_cast(__bf16, zkv);
        zv[c][s8] = __builtin_bit_cast(__bf16, zvv);
      }
    float* dbk = p.dbk_part + ((size_t(b) * p.n_blocks + kb) * H + h) * DH * R;
    float* dbv = p.dbv_part + ((size_t(b) * p.n_blocks + kb) * H + h) * DH * R;
#pragma unroll
    for (int f = 0; f < DH / 32; ++f) {
      f32x16_t ck = {}, cv = {};
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bf16x8_t ak, av;
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
          ak[s8] = (__bf16)dk[f][8 * c + s8];
          av[s8] = (__bf16)dv[f][8 * c + s8];
        }
        ck = mfma32(ak, zk[c], ck);
        cv = mfma32(av, zv[c], cv);
      }
      if (n < R) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int d = 32 * f + 8 * (i >> 2) + 4 * half + (i & 3);
          dbk[size_t(d) * R + n] = ck[i];
          dbv[size_t(d) * R + n] = cv[i];
        }
      }
    }
  }

  // ---- dK_s, dV_s: the 4 heads summed through LDS, one partial per head group ----
  float* red = reinterpret_cast<float*>(smem);                     // [wave][f][16][64]
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int f = 0; f < DH / 32; ++f)
#pragma unroll
      for (int i = 0; i < 16; ++i) red[((wave * (DH / 32) + f) * 16 + i) * 64 + lane] = pass ? dv[f][i] : dk[f][i];
    __syncthreads();
    float* part = (pass ? p.dvs_part : p.dks_part) + (size_t(hg) * p.batch + b) * size_t(L) * DH;
    for (int f = wave; f < DH / 32; f += kTrWaves) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kTrWaves; ++w) sum += red[((w * (DH / 32) + f) * 16 + i) * 64 + lane];
        const int key = k0 + 8 * (i >> 2) + 4 * half + (i & 3);
        if (key < L) part[size_t(key) * DH + 32 * f + n] = sum;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Sums of the partials, each output element added in a fixed order:
// dK_s, dV_s over the head groups; dB^K, dB^V over (sequence, key block).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void train_reduce_kernel(const float* part, float* out, long long n, int parts) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  float s = 0.f;
  for (int k = 0; k < parts; ++k) s += part[(long long)k * n + e];
  out[e] = s;
}

size_t train_backward_ws_bytes(int batch, int heads, int head_dim, int rank, int seq_len) {
  const size_t B = size_t(batch), H = size_t(heads), D = size_t(head_dim), R = size_t(rank), L = size_t(seq_len);
  const size_t nb = (L + kTrTile - 1) / kTrTile, lp = nb * kTrTile, ng = (H + kTrWaves - 1) / kTrWaves;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  return 2 * al(B * L * H * R * 2) + 2 * al(B * H * lp * 4) + 2 * al(ng * B * L * D * 4) + 2 * al(B * nb * H * D * R * 4);
}

template <int DH, int R>
static hipError_t launch_train_backward_t(const TrainArgs& a, hipStream_t st) {
  using P = TrShape<DH, R>;
  const size_t B = size_t(a.batch), H = size_t(a.heads), L = size_t(a.seq_len);
  if (B == 0 || L == 0) {                  // no tokens: dB^K = dB^V = 0, nothing else to write
    if constexpr (R > 0) {
      const long long nb = (long long)(H * DH * R);
      hipLaunchKernelGGL(train_reduce_kernel, dim3(unsigned((nb + 255) / 256)), dim3(256), 0, st, nullptr, a.db_k, nb, 0);
      hipLaunchKernelGGL(train_reduce_kernel, dim3(unsigned((nb + 255) / 256)), dim3(256), 0, st, nullptr, a.db_v, nb, 0);
    }
    return hipGetLastError();
  }
  TrParams kp;
  kp.q = static_cast<const uint16_t*>(a.q);
  kp.k_s = static_cast<const uint16_t*>(a.k_s);
  kp.v_s = static_cast<const uint16_t*>(a.v_s);
  kp.z_k = static_cast<const uint16_t*>(a.z_k);
  kp.z_v = static_cast<const uint16_t*>(a.z_v);
  kp.b_k = static_cast<const uint16_t*>(a.b_k);
  kp.b_v = static_cast<const uint16_t*>(a.b_v);
  kp.out = static_cast<const uint16_t*>(a.out);
  kp.lse = a.lse;
  kp.d_out = static_cast<const uint16_t*>(a.d_out);
  kp.dq = a.dq; kp.dz_k = a.dz_k; kp.dz_v = a.dz_v;
  kp.batch = a.batch; kp.heads = a.heads; kp.seq_len = a.seq_len;
  kp.n_blocks = int((L + kTrTile - 1) / kTrTile);
  kp.seq_pad = kp.n_blocks * kTrTile;
  kp.n_hgroups = int((H + kTrWaves - 1) / kTrWaves);
  kp.scale = a.scale;
  kp.scale_log2 = a.scale * 1.4426950408889634f;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  unsigned char* w = static_cast<unsigned char*>(a.ws);
  kp.qb = reinterpret_cast<uint16_t*>(w); w += al(B * L * H * R * 2);
  kp.dob = reinterpret_cast<uint16_t*>(w); w += al(B * L * H * R * 2);
  kp.lse2 = reinterpret_cast<float*>(w); w += al(B * H * size_t(kp.seq_pad) * 4);
  kp.dd = reinterpret_cast<float*>(w); w += al(B * H * size_t(kp.seq_pad) * 4);
  kp.dks_part = reinterpret_cast<float*>(w); w += al(size_t(kp.n_hgroups) * B * L * DH * 4);
  kp.dvs_part = reinterpret_cast<float*>(w); w += al(size_t(kp.n_hgroups) * B * L * DH * 4);
  kp.dbk_part = reinterpret_cast<float*>(w); w += al(B * size_t(kp.n_blocks) * H * DH * R * 4);
  kp.dbv_part = reinterpret_cast<float*>(w);

  hipLaunchKernelGGL((train_prep_kernel<DH, R>), dim3(unsigned(B * L)), dim3(kTrThreads), 0, st, kp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned grid = unsigned(size_t(kp.n_blocks) * kp.n_hgroups * B);
  const int lds_dq = P::LDS_DQ;
  e = allow_dynamic_lds<&train_dq_kernel<DH, R>>(lds_dq);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((train_dq_kernel<DH, R>), dim3(grid), dim3(kTrThreads), size_t(lds_dq), st, kp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int lds_kv = P::LDS_KV;
  e = allow_dynamic_lds<&train_dkv_kernel<DH, R>>(lds_kv);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((train_dkv_kernel<DH, R>), dim3(grid), dim3(kTrThreads), size_t(lds_kv), st, kp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long nrow = (long long)(B * L * DH);
  hipLaunchKernelGGL(train_reduce_kernel, dim3(unsigned((nrow + 255) / 256)), dim3(256), 0, st, kp.dks_part, a.dk_s,
                     nrow, kp.n_hgroups);
  hipLaunchKernelGGL(train_reduce_kernel, dim3(unsigned((nrow + 255) / 256)), dim3(256), 0, st, kp.dvs_part, a.dv_s,
                     nrow, kp.n_hgroups);
  if constexpr (R > 0) {
    const long long nb = (long long)(H * DH * R);
    const int parts = int(B) * kp.n_blocks;
    hipLaunchKernelGGL(train_reduce_kernel, dim3(unsigned((nb + 255) / 256)), dim3(256), 0, st, kp.dbk_part, a.db_k,
                       nb, parts);
    hipLaunchKernelGGL(train_reduce_kernel, dim3(unsigned((nb + 255) / 256)), dim3(256), 0, st, kp.dbv_part, a.db_v,
                       nb, parts);
  }
  return hipGetLastError();
}

bool train_supported(int dtype, int head_dim, int rank, int heads) {
  return dtype == 1 && (head_dim == 64 || head_dim == 128) && (rank == 0 || rank == 8 || rank == 16 || rank == 32) &&
         heads >= 1 && heads % kTrWaves == 0;
}

hipError_t launch_train_backward(const TrainArgs& a, hipStream_t st) {
#define LRKV_TR(DHV, RV) \
  if (a.head_dim == DHV && a.rank == RV) return launch_train_backward_t<DHV, RV>(a, st);
  LRKV_TR(64, 0) LRKV_TR(64, 8) LRKV_TR(64, 16) LRKV_TR(64, 32)
  LRKV_TR(128, 0) LRKV_TR(128, 8) LRKV_TR(128, 16) LRKV_TR(128, 32)
#undef LRKV_TR
  return hipErrorInvalidValue;
}

hipError_t train_prepare() {
  hipError_t e = hipSuccess;
#define LRKV_TR(DHV, RV)                                                                                      \
  if (e == hipSuccess) e = allow_dynamic_lds<&train_dq_kernel<DHV, RV>>(TrShape<DHV, RV>::LDS_DQ);              \
  if (e == hipSuccess) e = allow_dynamic_lds<&train_dkv_kernel<DHV, RV>>(TrShape<DHV, RV>::LDS_KV);
  LRKV_TR(64, 0) LRKV_TR(64, 8) LRKV_TR(64, 16) LRKV_TR(64, 32)
  LRKV_TR(128, 0) LRKV_TR(128, 8) LRKV_TR(128, 16) LRKV_TR(128, 32)
#undef LRKV_TR
  return e;
}

}  // namespace lrkv
