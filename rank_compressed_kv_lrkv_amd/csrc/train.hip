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
//                       LDS (software pipelined), S^T and dP^T on MFMA
//                       (lane = query), dQ^T
//                       accumulated as Kaug^T dS^T, B^K epilogue;
//   train_dkv_kernel    per (128 keys, head): the head's queries and dO
//                       streamed through LDS (software pipelined), S and dP on
//                       MFMA (lane = key), Kaug and Vaug gradients
//                       accumulated as dS^T Qaug and P^T dOaug; per-head
//                       partials of dK_s, dV_s and per-key-block partial
//                       dB^K, dB^V;
//   train_reduce_kernel the partial sums added up (deterministic order).
// P and dS enter MFMAs rounded to bf16; everything is accumulated in fp32.
#include <type_traits>

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
  static constexpr int LDS_DQ1 = 2 * (ROWS + LATS);        // dQ kernel: a key and a value tile
  static constexpr int LDS_DQ = 3 * LDS_DQ1;                // a three-stage pipeline
  // dK/dV kernel: three query-side tiles of one head (a software pipeline),
  // each Q rows, Q B^K latents, dO rows, dO B^V latents, then lse and D of
  // its 32 queries; after them the B-gradient exchange area (32 x R fp32)
  static constexpr int ZB1 = R * 2, CZ1 = ZB1 / 16;         // one head's latents of a token
  static constexpr int LATS1 = kTrTile * ZB1;
  static constexpr int KV_TILE1 = 2 * (ROWS + LATS1) + 2 * kTrTile * 4;
  static constexpr int KV_BUFS = 3;
  static constexpr int LDS_KV = KV_BUFS * KV_TILE1 + (R > 0 ? kTrTile * R * 4 : 16);
  static_assert(DH % 32 == 0 && R <= 32 && R % 8 == 0, "training envelope");
  static_assert(CR >= 4 && (R == 0 || CZ >= 4), "swizzle needs 4 chunks per row");
  static_assert(LDS_KV <= 160 * 1024, "LDS");
};

constexpr int kTrKeyWaves = 4;                // dK/dV kernel: waves over the keys of a block
constexpr int kTrKeyBlock = kTrKeyWaves * kTrTile;

struct TrParams {
  const uint16_t* q; const uint16_t* k_s; const uint16_t* v_s; const uint16_t* z_k; const uint16_t* z_v;
  const uint16_t* b_k; const uint16_t* b_v;
  const uint16_t* out; const float* lse; const uint16_t* d_out;
  float* dq; float* dz_k; float* dz_v;
  // workspace
  uint16_t* qb; uint16_t* dob;      // [B][L][H][R] bf16: Q B^K_h and dO B^V_h
  float* lse2; float* dd;           // [B][H][Lp]: lse * log2(e) and rowsum(dO o O); rows >= L: +inf, 0
  float* dks_part; float* dvs_part; // [H][B][L][DH]: per-head dK_h, dV_h
  float* dbk_part; float* dbv_part; // [B][n_kb][H][DH][R], key blocks of kTrKeyBlock tokens
  int batch, heads, seq_len, seq_pad, n_blocks, n_hgroups, n_kb;
  float scale, scale_log2;
};

// Per-lane LDS offsets of the operand reads (the layouts of the forward
// prefill kernel): row-major 16-byte reads of chunk c of row n (koff) and of
// latent chunk c (zoff) of head slot `slot` in a latent tile holding NH
// heads' latents per token; transpose reads of a 16-token chunk of d_h rows
// (voff) and of latents (zvoff), giving lane (feature n, half) the tokens
// {4half..+3, 8+4half..+3} of the chunk, the k-slot order of an MFMA
// accumulator used as the other operand.
template <int DH, int R, int NH>
struct TrOffsets {
  using P = TrShape<DH, R>;
  static constexpr int ZB = NH * R * 2, CZ = ZB / 16;       // latent bytes and chunks per token
  int koff[DH / 16], zoff[P::ZCH], voff[DH / 32][2], zvoff[2][2];
  __device__ __forceinline__ TrOffsets(int lane, int slot) {
    const int n = lane & 31, half = lane >> 5;
#pragma unroll
    for (int c = 0; c < DH / 16; ++c) koff[c] = n * P::RB + ((2 * c + half) ^ lds_swz(n, P::CR)) * 16;
#pragma unroll
    for (int c = 0; c < P::ZCH; ++c) {
      zoff[c] = 0;
      if constexpr (R > 0) {
        const int ch = slot * (R / 8) + (R == 8 ? 0 : 2 * c + half);
        zoff[c] = n * ZB + (ch ^ lds_swz(n, CZ)) * 16;
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
          const int byte = slot * R * 2 + (feat < R ? feat : 0) * 2;   // rows >= R: any valid row (unused)
          const int row = 16 * c + tr_tok + 8 * j;
          zvoff[c][j] = row * ZB + ((byte / 16) ^ lds_swz(row, CZ)) * 16 + byte % 16;
        }
      }
  }
};

// Row-major operand chunk c of an augmented row: d_h part from `rows`, latent
// part from `lats` (the offsets' head slot).
template <int DH, int R, int NH>
__device__ __forceinline__ bf16x8_t tr_row_chunk(const unsigned char* rows, const unsigned char* lats,
                                                 const TrOffsets<DH, R, NH>& o, int c, int half) {
  if (c < DH / 16) return as_bf16x8(*reinterpret_cast<const u32x4*>(rows + o.koff[c]));
  if constexpr (R > 0) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(lats + o.zoff[c - DH / 16]);
    return as_bf16x8((R == 8 && half) ? u32x4{0u, 0u, 0u, 0u} : v);   // R = 8: dims 8..15 are padding
  }
  return as_bf16x8(u32x4{0u, 0u, 0u, 0u});
}

// Transposed operand of 32-row block f of an augmented row, 16-token chunk c.
template <int DH, int R, int NH>
__device__ __forceinline__ bf16x8_t tr_col_chunk(const unsigned char* rows, const unsigned char* lats,
                                                 const TrOffsets<DH, R, NH>& o, int f, int c) {
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
// Per (token, head): Q B^K_h and dO B^V_h (bf16), D = rowsum(dO o O) and
// lse * log2(e) (fp32, [B][H][Lp]; the padding rows get D = 0, lse = +inf).  Workgroup = 128
// tokens (4 blocks of 32) x 4 heads, one head per wave.  The products run on
// MFMA as C[j][token] = sum_d B_h[d][j] X[token][d]: A = B_h^T (lane = latent
// column j, read once per wave), B = the tokens' rows straight from global
// memory (lane = token), so lane (token n, half) ends up holding latent
// columns 8(i/4) + 4half + i%4 of its token.
// ---------------------------------------------------------------------------
constexpr int kPrepBlocks = 4;                 // 32-token blocks per workgroup

template <int DH, int R>
__global__ __launch_bounds__(kTrThreads) void train_prep_kernel(TrParams p) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, half = lane >> 5;
  const int H = p.heads, L = p.seq_len;
  const int h = int(blockIdx.y) * kTrWaves + wave;
  const long long ntok = (long long)p.batch * L;
  constexpr int NC = DH / 16;
  bf16x8_t wk[NC], wv[NC];
  if constexpr (R > 0) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const size_t at = (size_t(h) * DH + 16 * c + 8 * half + e) * R + n;
        wk[c][e] = __builtin_bit_cast(__bf16, n < R ? p.b_k[at] : uint16_t(0));
        wv[c][e] = __builtin_bit_cast(__bf16, n < R ? p.b_v[at] : uint16_t(0));
      }
  }
#pragma unroll 1
  for (int sb = 0; sb < kPrepBlocks; ++sb) {
    const long long t = ((long long)blockIdx.x * kPrepBlocks + sb) * kTrTile + n;   // this lane's token
    const bool ok = t < ntok;
    const size_t row = (size_t(ok ? t : ntok - 1) * H + h) * DH + 8 * half;
    f32x16_t cq = {}, cd = {};
    float dsum = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const u32x4 qv = *reinterpret_cast<const u32x4*>(p.q + row + 16 * c);
      const u32x4 dv = *reinterpret_cast<const u32x4*>(p.d_out + row + 16 * c);
      const u32x4 ov = *reinterpret_cast<const u32x4*>(p.out + row + 16 * c);
      if constexpr (R > 0) {
        cq = mfma32(wk[c], as_bf16x8(qv), cq);
        cd = mfma32(wv[c], as_bf16x8(dv), cd);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dsum = __builtin_fmaf(__uint_as_float(dv[e] << 16), __uint_as_float(ov[e] << 16), dsum);
        dsum = __builtin_fmaf(__uint_as_float(dv[e] & 0xffff0000u), __uint_as_float(ov[e] & 0xffff0000u), dsum);
      }
    }
    dsum += __shfl_xor(dsum, 32);
    if (!ok) continue;
    const int b = int(t / L), i = int(t % L);
    if (half == 0) {
      const size_t o = (size_t(b) * H + h) * p.seq_pad + i;
      p.dd[o] = dsum;
      p.lse2[o] = p.lse[size_t(t) * H + h] * 1.4426950408889634f;
      if (i == L - 1)
        for (int u = L; u < p.seq_pad; ++u) {
          p.dd[o + (u - i)] = 0.f;
          p.lse2[o + (u - i)] = __builtin_inff();   // probability 0 for every key
        }
    }
    if constexpr (R > 0) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j0 = 8 * g + 4 * half;
        if (j0 < R) {
          const size_t zo = (size_t(t) * H + h) * R + j0;
          *reinterpret_cast<uint2*>(p.qb + zo) = uint2{pack_bf16x2(cq[4 * g], cq[4 * g + 1]),
                                                       pack_bf16x2(cq[4 * g + 2], cq[4 * g + 3])};
          *reinterpret_cast<uint2*>(p.dob + zo) = uint2{pack_bf16x2(cd[4 * g], cd[4 * g + 1]),
                                                        pack_bf16x2(cd[4 * g + 2], cd[4 * g + 3])};
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ: workgroup = (query block, 4 heads, sequence), one head per wave.  The
// key tiles from 0 to the diagonal (K_s and V_s rows, the 4 heads' Z^K and
// Z^V latents) stream through three LDS buffers: tile kt's dS (vector ALU)
// overlaps tile kt + 1's scores (MFMA), tile kt + 2's global loads are in
// flight in registers.
// ---------------------------------------------------------------------------
template <int DH, int R>
__global__ __launch_bounds__(kTrThreads) void train_dq_kernel(TrParams p) {
  using P = TrShape<DH, R>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
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
  const TrOffsets<DH, R, kTrWaves> o(lane, wave);

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

  // key tile kt: global loads into registers, then stores to LDS buffer
  // `buf`.  Rows past the sequence repeat its last row (finite values; those
  // keys are later than every query, so the causal mask removes them).
  constexpr int NRL = kTrTile * P::CR / kTrThreads;         // row chunks per thread and array
  constexpr int NZL = R > 0 ? (kTrTile * P::CZ + kTrThreads - 1) / kTrThreads : 1;   // latent chunks per thread
  static_assert(NRL >= 1 && (kTrTile * P::CR) % kTrThreads == 0, "row chunks per thread");
  u32x4 pre_k[NRL], pre_v[NRL], pre_zk[NZL], pre_zv[NZL];
  // element offsets of this thread's latent chunks from a tile's first token
  uint32_t zoffs[NZL];
#pragma unroll
  for (int i = 0; i < NZL; ++i) {
    const int idx = tid + i * kTrThreads;
    zoffs[i] = R > 0 ? uint32_t(((idx / P::CZ) * H + hg * kTrWaves) * R + (idx % P::CZ) * 8) : 0u;
  }
  auto tile_load = [&](int kt) __attribute__((always_inline)) {
    const int t0 = kt * kTrTile;
    const size_t tok = size_t(b) * L + t0;
    if (t0 + kTrTile <= L) {                                 // a whole tile: uniform base + offsets
#pragma unroll
      for (int i = 0; i < NRL; ++i) {
        const uint32_t off = uint32_t(tid + i * kTrThreads) * 8;
        pre_k[i] = *reinterpret_cast<const u32x4*>(p.k_s + tok * DH + off);
        pre_v[i] = *reinterpret_cast<const u32x4*>(p.v_s + tok * DH + off);
      }
      if constexpr (R > 0) {
#pragma unroll
        for (int i = 0; i < NZL; ++i)
          if (tid + i * kTrThreads < kTrTile * P::CZ) {
            pre_zk[i] = *reinterpret_cast<const u32x4*>(p.z_k + tok * H * R + zoffs[i]);
            pre_zv[i] = *reinterpret_cast<const u32x4*>(p.z_v + tok * H * R + zoffs[i]);
          }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NRL; ++i) {
        const int idx = tid + i * kTrThreads, t = idx / P::CR, ch = idx % P::CR;
        const size_t off = (size_t(b) * L + min(t0 + t, L - 1)) * DH + ch * 8;
        pre_k[i] = *reinterpret_cast<const u32x4*>(p.k_s + off);
        pre_v[i] = *reinterpret_cast<const u32x4*>(p.v_s + off);
      }
      if constexpr (R > 0) {
#pragma unroll
        for (int i = 0; i < NZL; ++i) {
          const int idx = tid + i * kTrThreads, t = idx / P::CZ, ch = idx % P::CZ;
          if (idx < kTrTile * P::CZ) {
            const size_t off = ((size_t(b) * L + min(t0 + t, L - 1)) * H + hg * kTrWaves) * R + ch * 8;
            pre_zk[i] = *reinterpret_cast<const u32x4*>(p.z_k + off);
            pre_zv[i] = *reinterpret_cast<const u32x4*>(p.z_v + off);
          }
        }
      }
    }
  };
  auto tile_store = [&](int buf) __attribute__((always_inline)) {
    unsigned char* const kr = smem + buf * P::LDS_DQ1;
    unsigned char* const kl = kr + P::ROWS;
    unsigned char* const vr = kl + P::LATS;
    unsigned char* const vl = vr + P::ROWS;
#pragma unroll
    for (int i = 0; i < NRL; ++i) {
      const int idx = tid + i * kTrThreads, t = idx / P::CR, ch = idx % P::CR;
      const int pos = t * P::RB + (ch ^ lds_swz(t, P::CR)) * 16;
      *reinterpret_cast<u32x4*>(kr + pos) = pre_k[i];
      *reinterpret_cast<u32x4*>(vr + pos) = pre_v[i];
    }
    if constexpr (R > 0) {
#pragma unroll
      for (int i = 0; i < NZL; ++i) {
        const int idx = tid + i * kTrThreads, t = idx / P::CZ, ch = idx % P::CZ;
        if (idx < kTrTile * P::CZ) {
          const int pos = t * P::ZB + (ch ^ lds_swz(t, P::CZ)) * 16;
          *reinterpret_cast<u32x4*>(kl + pos) = pre_zk[i];
          *reinterpret_cast<u32x4*>(vl + pos) = pre_zv[i];
        }
      }
    }
  };

  // Software pipeline over the key tiles, three LDS buffers: while tile
  // kt's dS is formed (vector ALU), the scores of tile kt + 1 run on MFMA;
  // tile kt + 2 is in flight from global memory.
  auto rows_of = [&](int buf) __attribute__((always_inline)) { return smem + buf * P::LDS_DQ1; };
  f32x16_t acc[P::VBLK];
#pragma unroll
  for (int f = 0; f < P::VBLK; ++f) acc[f] = f32x16_t{};
  tile_load(0);
  tile_store(0);
  tile_load(min(1, kt_last));
  tile_store(1);
  __syncthreads();
  // S^T = Kaug Qaug^T and dP^T = Vaug dOaug^T: lane (query n, half) holds
  // keys 8(i/4) + 4half + i%4
  f32x16_t s = {}, dp = {};
  {
    const unsigned char* const kr = rows_of(0);
#pragma unroll
    for (int c = 0; c < P::KCH; ++c) {
      s = mfma32(tr_row_chunk(kr, kr + P::ROWS, o, c, half), qop[c], s);
      dp = mfma32(tr_row_chunk(kr + P::ROWS + P::LATS, kr + 2 * P::ROWS + P::LATS, o, c, half), dop[c], dp);
    }
  }
  // causal mask: key t0 + 8j + 4half + e is seen by query q0 + n iff
  // (q0 + n - 4half - t0) - (8j + e) >= 0 (keys past the sequence are later
  // than every query)
  const int mask_base = q0 + n - 4 * half;
  int cur = 0;
  for (int kt = 0; kt <= kt_last; ++kt) {
    const int nxt = cur == 2 ? 0 : cur + 1, nn = nxt == 2 ? 0 : nxt + 1;
    if (kt + 2 <= kt_last) tile_load(kt + 2);
    const unsigned char* const krows = rows_of(cur);
    const unsigned char* const klats = krows + P::ROWS;
    const int mb = mask_base - kt * kTrTile;
    // dS of tile kt (bf16), formed between the MFMAs of tile kt + 1's scores
    // (past the end: a stale buffer, not used): chunk c's two MFMAs, then
    // elements [16c / KCH, 16(c + 1) / KCH); the next chunk's operands are
    // read one step ahead.  Scheduling barriers keep the groups in order.
    const unsigned char* const nk = rows_of(nxt);
    const unsigned char* const nkl = nk + P::ROWS;
    const unsigned char* const nv = nkl + P::LATS;
    const unsigned char* const nvl = nv + P::ROWS;
    bf16x8_t pb[2];
    f32x16_t s2 = {}, dp2 = {};
    bf16x8_t ak = tr_row_chunk(nk, nkl, o, 0, half), av = tr_row_chunk(nv, nvl, o, 0, half);
#pragma unroll
    for (int c = 0; c < P::KCH; ++c) {
      bf16x8_t ak1 = ak, av1 = av;
      if (c + 1 < P::KCH) {
        ak1 = tr_row_chunk(nk, nkl, o, c + 1, half);
        av1 = tr_row_chunk(nv, nvl, o, c + 1, half);
      }
      s2 = mfma32(ak, qop[c], s2);
      dp2 = mfma32(av, dop[c], dp2);
#pragma unroll
      for (int i = 16 * c / P::KCH; i < 16 * (c + 1) / P::KCH; ++i) {
        const float ev = fast_exp2(__builtin_fmaf(s[i], p.scale_log2, -lse2));
        float sv = mb >= 8 * (i >> 2) + (i & 3) ? ev * (dp[i] - dd) : 0.f;
        asm volatile("" : "+v"(sv));
        pb[i >> 3][i & 7] = (__bf16)sv;
      }
      __builtin_amdgcn_sched_barrier(0);
      ak = ak1;
      av = av1;
    }
    // dQaug^T += Kaug^T dS^T, block f's MFMAs with block f + 1's operands
    // read one step ahead
    bf16x8_t ok[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) ok[c] = tr_col_chunk(krows, klats, o, 0, c);
#pragma unroll
    for (int f = 0; f < P::VBLK; ++f) {
      bf16x8_t ok1[2] = {ok[0], ok[1]};
      if (f + 1 < P::VBLK) {
#pragma unroll
        for (int c = 0; c < 2; ++c) ok1[c] = tr_col_chunk(krows, klats, o, f + 1, c);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) acc[f] = mfma32(ok[c], pb[c], acc[f]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < 2; ++c) ok[c] = ok1[c];
    }
    // buffer nn held tile kt - 1, read before the previous barrier
    if (kt + 2 <= kt_last) tile_store(nn);
    __syncthreads();
    s = s2;
    dp = dp2;
    cur = nxt;
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
// dK, dV: workgroup = (block of 128 keys, head, sequence); wave w owns keys
// k0 + 32w .. k0 + 32w + 31.  The query blocks from the key block's diagonal
// to the end stream through LDS as one tile (the head's Q rows and Q B^K
// latents, dO rows and dO B^V latents, lse and D of the 32 queries) that all
// four waves read.  Three LDS buffers carry a software pipeline: tile qb's
// probabilities (vector ALU) overlap tile qb + 1's scores (MFMA), and tile
// qb + 2's global loads are in flight in registers.  A
// wave keeps its keys' [dK_h | dZ^K_h] and [dV_h | dZ^V_h] in registers; at
// the end it writes dZ^K_h, dZ^V_h, the head's dK_h, dV_h as one partial of
// dK_s, dV_s (summed over the heads afterwards) and its share of dB^K_h,
// dB^V_h over the block (summed over the waves in a fixed order through LDS).
// ---------------------------------------------------------------------------
template <int DH, int R>
__global__ __launch_bounds__(kTrThreads) void train_dkv_kernel(TrParams p) {
  using P = TrShape<DH, R>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  float* const bx = reinterpret_cast<float*>(smem + P::KV_BUFS * P::KV_TILE1);   // B-gradient exchange
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, half = lane >> 5;
  const int H = p.heads, L = p.seq_len;
  const int per_level = H * p.batch;
  const int kb = int(blockIdx.x) / per_level;                // key block 0 (the heaviest) first
  const int rem = int(blockIdx.x) % per_level;
  const int b = rem % p.batch, h = rem / p.batch;
  const int k0 = kb * kTrKeyBlock + wave * kTrTile;          // this wave's first key
  const int krow = min(k0 + n, L - 1);
  const int nqb = (L + kTrTile - 1) / kTrTile;
  const int qb_first = (kb * kTrKeyBlock) / kTrTile;
  const TrOffsets<DH, R, 1> o(lane, 0);

  // the lane's key rows [K_s | Z^K_h] and [V_s | Z^V_h] (B operands, lane = key n)
  bf16x8_t kop[P::KCH], vop[P::KCH];
  {
    const size_t kr = size_t(b) * L + krow;
#pragma unroll
    for (int c = 0; c < P::KCH; ++c) {
      kop[c] = tr_global_chunk<DH, R>(p.k_s + kr * DH, p.z_k + (kr * H + h) * R, c, half);
      vop[c] = tr_global_chunk<DH, R>(p.v_s + kr * DH, p.z_v + (kr * H + h) * R, c, half);
    }
  }

  // query-side tile qb: global loads into registers, then stores to LDS
  // buffer `buf`.  Rows past the sequence repeat its last row: their
  // probabilities are 0 and every value is finite, so they add nothing.
  constexpr int NRL = kTrTile * P::CR / kTrThreads;         // row chunks per thread and array
  static_assert(NRL >= 1 && (kTrTile * P::CR) % kTrThreads == 0, "row chunks per thread");
  static_assert(kTrTile * P::CZ1 <= kTrThreads, "latent chunks per thread");
  u32x4 pre_q[NRL], pre_d[NRL], pre_zq = {0u, 0u, 0u, 0u}, pre_zd = {0u, 0u, 0u, 0u};
  float pre_l = 0.f;
  const size_t lrow = (size_t(b) * H + h) * p.seq_pad;
  // element offsets of this thread's chunks from a tile's first token
  uint32_t roff[NRL], zoff1 = 0;
#pragma unroll
  for (int i = 0; i < NRL; ++i) {
    const int idx = tid + i * kTrThreads;
    roff[i] = uint32_t(((idx / P::CR) * H + h) * DH + (idx % P::CR) * 8);
  }
  if constexpr (R > 0) zoff1 = uint32_t(((tid / P::CZ1) * H + h) * R + (tid % P::CZ1) * 8);
  auto tile_load = [&](int qb) __attribute__((always_inline)) {
    const int q0 = qb * kTrTile;
    const size_t tok = size_t(b) * L + q0;
    if (q0 + kTrTile <= L) {                                 // a whole tile: uniform base + offsets
#pragma unroll
      for (int i = 0; i < NRL; ++i) {
        pre_q[i] = *reinterpret_cast<const u32x4*>(p.q + tok * H * DH + roff[i]);
        pre_d[i] = *reinterpret_cast<const u32x4*>(p.d_out + tok * H * DH + roff[i]);
      }
      if constexpr (R > 0) {
        if (tid < kTrTile * P::CZ1) {
          pre_zq = *reinterpret_cast<const u32x4*>(p.qb + tok * H * R + zoff1);
          pre_zd = *reinterpret_cast<const u32x4*>(p.dob + tok * H * R + zoff1);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NRL; ++i) {
        const int idx = tid + i * kTrThreads, t = idx / P::CR, ch = idx % P::CR;
        const size_t off = ((size_t(b) * L + min(q0 + t, L - 1)) * H + h) * DH + ch * 8;
        pre_q[i] = *reinterpret_cast<const u32x4*>(p.q + off);
        pre_d[i] = *reinterpret_cast<const u32x4*>(p.d_out + off);
      }
      if constexpr (R > 0) {
        if (tid < kTrTile * P::CZ1) {
          const int t = tid / P::CZ1, ch = tid % P::CZ1;
          const size_t off = ((size_t(b) * L + min(q0 + t, L - 1)) * H + h) * R + ch * 8;
          pre_zq = *reinterpret_cast<const u32x4*>(p.qb + off);
          pre_zd = *reinterpret_cast<const u32x4*>(p.dob + off);
        }
      }
    }
    // lse and D of the 32 queries (padding rows: +inf and 0)
    if (tid < 2 * kTrTile) pre_l = (tid < kTrTile ? p.lse2 : p.dd)[lrow + q0 + (tid & (kTrTile - 1))];
  };
  auto tile_store = [&](int buf) __attribute__((always_inline)) {
    unsigned char* const qrows = smem + buf * P::KV_TILE1;
    unsigned char* const qlats = qrows + P::ROWS;
    unsigned char* const drows = qlats + P::LATS1;
    unsigned char* const dlats = drows + P::ROWS;
#pragma unroll
    for (int i = 0; i < NRL; ++i) {
      const int idx = tid + i * kTrThreads, t = idx / P::CR, ch = idx % P::CR;
      const int pos = t * P::RB + (ch ^ lds_swz(t, P::CR)) * 16;
      *reinterpret_cast<u32x4*>(qrows + pos) = pre_q[i];
      *reinterpret_cast<u32x4*>(drows + pos) = pre_d[i];
    }
    if constexpr (R > 0) {
      if (tid < kTrTile * P::CZ1) {
        const int t = tid / P::CZ1, ch = tid % P::CZ1;
        const int pos = t * P::ZB1 + (ch ^ lds_swz(t, P::CZ1)) * 16;
        *reinterpret_cast<u32x4*>(qlats + pos) = pre_zq;
        *reinterpret_cast<u32x4*>(dlats + pos) = pre_zd;
      }
    }
    if (tid < 2 * kTrTile) reinterpret_cast<float*>(dlats + P::LATS1)[tid] = pre_l;
  };
  // S = Qaug Kaug^T and dP = dOaug Vaug^T of the tile in buffer `buf`: lane
  // (key n, half) holds queries 8(i/4) + 4half + i%4
  auto scores = [&](int buf, f32x16_t& s, f32x16_t& dp) __attribute__((always_inline)) {
    const unsigned char* const qrows = smem + buf * P::KV_TILE1;
    const unsigned char* const qlats = qrows + P::ROWS;
    const unsigned char* const drows = qlats + P::LATS1;
    const unsigned char* const dlats = drows + P::ROWS;
    s = f32x16_t{};
    dp = f32x16_t{};
#pragma unroll
    for (int c = 0; c < P::KCH; ++c) {
      s = mfma32(tr_row_chunk(qrows, qlats, o, c, half), kop[c], s);
      dp = mfma32(tr_row_chunk(drows, dlats, o, c, half), vop[c], dp);
    }
  };

  // Software pipeline over the query tiles, three LDS buffers: while tile
  // qb's probabilities are formed (vector ALU), the scores of tile qb + 1 run
  // on MFMA; tile qb + 2 is in flight from global memory.
  f32x16_t dk[P::VBLK], dv[P::VBLK];
#pragma unroll
  for (int f = 0; f < P::VBLK; ++f) dk[f] = dv[f] = f32x16_t{};
  tile_load(qb_first);
  tile_store(0);
  tile_load(min(qb_first + 1, nqb - 1));
  tile_store(1);
  __syncthreads();
  f32x16_t s, dp;
  scores(0, s, dp);
  // causal mask: query q0 + 8j + 4half + e sees key k0 + n iff
  // (q0 - k0 + 4half - n) + 8j + e >= 0; queries past the sequence have
  // lse = +inf (probability 0), keys past it are later than every query
  const int mask_base = 4 * half - n - k0;
  int cur = 0;
  for (int qb = qb_first; qb < nqb; ++qb) {
    const int nxt = cur == 2 ? 0 : cur + 1, nn = nxt == 2 ? 0 : nxt + 1;
    if (qb + 2 < nqb) tile_load(qb + 2);
    const unsigned char* const qrows = smem + cur * P::KV_TILE1;
    const unsigned char* const qlats = qrows + P::ROWS;
    const unsigned char* const drows = qlats + P::LATS1;
    const unsigned char* const dlats = drows + P::ROWS;
    const float* const lsd = reinterpret_cast<const float*>(dlats + P::LATS1);   // lse2[32], then D[32]
    const int mb = qb * kTrTile + mask_base;
    // P and dS of tile qb (bf16), formed between the MFMAs of tile qb + 1's
    // scores (past the end: a stale buffer, not used): chunk c's two MFMAs,
    // then elements [16c / KCH, 16(c + 1) / KCH) of the probabilities; the
    // next chunk's operands are read from LDS one step ahead.  Scheduling
    // barriers keep the groups in this order.
    float4 l4[4], d4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      l4[j] = *reinterpret_cast<const float4*>(lsd + 8 * j + 4 * half);
      d4[j] = *reinterpret_cast<const float4*>(lsd + kTrTile + 8 * j + 4 * half);
    }
    const unsigned char* const nq = smem + nxt * P::KV_TILE1;
    const unsigned char* const nql = nq + P::ROWS;
    const unsigned char* const nd = nql + P::LATS1;
    const unsigned char* const ndl = nd + P::ROWS;
    bf16x8_t pp[2], ps[2];
    f32x16_t s2 = {}, dp2 = {};
    bf16x8_t aq = tr_row_chunk(nq, nql, o, 0, half), ad = tr_row_chunk(nd, ndl, o, 0, half);
#pragma unroll
    for (int c = 0; c < P::KCH; ++c) {
      bf16x8_t aq1 = aq, ad1 = ad;
      if (c + 1 < P::KCH) {
        aq1 = tr_row_chunk(nq, nql, o, c + 1, half);
        ad1 = tr_row_chunk(nd, ndl, o, c + 1, half);
      }
      s2 = mfma32(aq, kop[c], s2);
      dp2 = mfma32(ad, vop[c], dp2);
#pragma unroll
      for (int i = 16 * c / P::KCH; i < 16 * (c + 1) / P::KCH; ++i) {
        const int j = i >> 2, e = i & 3;
        const float lv = e == 0 ? l4[j].x : e == 1 ? l4[j].y : e == 2 ? l4[j].z : l4[j].w;
        const float dd = e == 0 ? d4[j].x : e == 1 ? d4[j].y : e == 2 ? d4[j].z : d4[j].w;
        const float ev = fast_exp2(__builtin_fmaf(s[i], p.scale_log2, -lv));
        float pv = mb + 8 * j + e >= 0 ? ev : 0.f;
        float sv = pv * (dp[i] - dd);
        asm volatile("" : "+v"(pv), "+v"(sv));
        pp[i >> 3][i & 7] = (__bf16)pv;
        ps[i >> 3][i & 7] = (__bf16)sv;
      }
      __builtin_amdgcn_sched_barrier(0);
      aq = aq1;
      ad = ad1;
    }
    // [dV_h | dZ^V_h] += P^T dOaug, [dK_h | dZ^K_h] / scale += dS^T Qaug,
    // block f's four MFMAs with block f + 1's operands read one step ahead
    bf16x8_t od[2], oq[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      od[c] = tr_col_chunk(drows, dlats, o, 0, c);
      oq[c] = tr_col_chunk(qrows, qlats, o, 0, c);
    }
#pragma unroll
    for (int f = 0; f < P::VBLK; ++f) {
      bf16x8_t od1[2] = {od[0], od[1]}, oq1[2] = {oq[0], oq[1]};
      if (f + 1 < P::VBLK) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          od1[c] = tr_col_chunk(drows, dlats, o, f + 1, c);
          oq1[c] = tr_col_chunk(qrows, qlats, o, f + 1, c);
        }
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        dv[f] = mfma32(pp[c], od[c], dv[f]);
        dk[f] = mfma32(ps[c], oq[c], dk[f]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        od[c] = od1[c];
        oq[c] = oq1[c];
      }
    }
    // buffer nn held tile qb - 1, read before the previous barrier
    if (qb + 2 < nqb) tile_store(nn);
    __syncthreads();
    s = s2;
    dp = dp2;
    cur = nxt;
  }
#pragma unroll
  for (int f = 0; f < P::VBLK; ++f) dk[f] *= p.scale;

  // ---- this head's dK_h, dV_h: one partial of dK_s, dV_s ----
  const size_t part = (size_t(h) * p.batch + b) * size_t(L) * DH;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int key = k0 + 8 * (i >> 2) + 4 * half + (i & 3);
    if (key < L) {
#pragma unroll
      for (int f = 0; f < DH / 32; ++f) {
        p.dks_part[part + size_t(key) * DH + 32 * f + n] = dk[f][i];
        p.dvs_part[part + size_t(key) * DH + 32 * f + n] = dv[f][i];
      }
    }
  }

  if constexpr (R > 0) {
    // ---- dZ^K_h, dZ^V_h (columns n < R) ----
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
    // ---- dB^K_h, dB^V_h over the block: C[d][j] = sum_key dK_h[key][d] Z^K[key][h][j] ----
    // A = dK_h^T (lane = feature row, k-slots = keys in accumulator order),
    // B = Z^K (lane = latent column n, the same keys).  The four waves'
    // partials are added in wave order through LDS.
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
    const size_t dbo = ((size_t(b) * p.n_kb + kb) * H + h) * DH * R;
#pragma unroll
    for (int f = 0; f < DH / 32; ++f) {
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        f32x16_t cb = {};
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          bf16x8_t a;
#pragma unroll
          for (int s8 = 0; s8 < 8; ++s8) a[s8] = (__bf16)(pass ? dv[f][8 * c + s8] : dk[f][8 * c + s8]);
          cb = mfma32(a, pass ? zv[c] : zk[c], cb);
        }
        float* dst = (pass ? p.dbv_part : p.dbk_part) + dbo;
#pragma unroll 1
        for (int w = 0; w < kTrKeyWaves; ++w) {
          if (wave == w && n < R) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int dl = 8 * (i >> 2) + 4 * half + (i & 3);
              const float v = w == 0 ? cb[i] : bx[dl * R + n] + cb[i];
              if (w + 1 < kTrKeyWaves) bx[dl * R + n] = v;
              else dst[size_t(32 * f + dl) * R + n] = v;
            }
          }
          __syncthreads();                                   // this turn's sums are visible (and read)
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Sums of the partials, each output element added in a fixed order:
// dK_s, dV_s over the heads; dB^K, dB^V over (sequence, key block).
// ---------------------------------------------------------------------------
// Eight running sums (partial k goes to sum k % 8), added pairwise at the
// end: a fixed order, with eight loads in flight per thread.
__global__ __launch_bounds__(256) void train_reduce_kernel(const float* part, float* out, long long n, int parts) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int k = 0;
  for (; k + 8 <= parts; k += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = part[(long long)(k + j) * n + e];
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] += v[j];
  }
  for (; k < parts; ++k) s[k & 7] += part[(long long)k * n + e];
  out[e] = ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
}

size_t train_backward_ws_bytes(int batch, int heads, int head_dim, int rank, int seq_len) {
  const size_t B = size_t(batch), H = size_t(heads), D = size_t(head_dim), R = size_t(rank), L = size_t(seq_len);
  const size_t nb = (L + kTrTile - 1) / kTrTile, lp = nb * kTrTile;
  const size_t nkb = (L + kTrKeyBlock - 1) / kTrKeyBlock;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  return 2 * al(B * L * H * R * 2) + 2 * al(B * H * lp * 4) + 2 * al(H * B * L * D * 4) +
         2 * al(B * nkb * H * D * R * 4);
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
  kp.n_kb = int((L + kTrKeyBlock - 1) / kTrKeyBlock);
  kp.scale = a.scale;
  kp.scale_log2 = a.scale * 1.4426950408889634f;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  unsigned char* w = static_cast<unsigned char*>(a.ws);
  kp.qb = reinterpret_cast<uint16_t*>(w); w += al(B * L * H * R * 2);
  kp.dob = reinterpret_cast<uint16_t*>(w); w += al(B * L * H * R * 2);
  kp.lse2 = reinterpret_cast<float*>(w); w += al(B * H * size_t(kp.seq_pad) * 4);
  kp.dd = reinterpret_cast<float*>(w); w += al(B * H * size_t(kp.seq_pad) * 4);
  kp.dks_part = reinterpret_cast<float*>(w); w += al(H * B * L * DH * 4);
  kp.dvs_part = reinterpret_cast<float*>(w); w += al(H * B * L * DH * 4);
  kp.dbk_part = reinterpret_cast<float*>(w); w += al(B * size_t(kp.n_kb) * H * DH * R * 4);
  kp.dbv_part = reinterpret_cast<float*>(w);

  const dim3 grid_prep(unsigned((B * L + kPrepBlocks * kTrTile - 1) / (kPrepBlocks * kTrTile)), unsigned(H / kTrWaves));
  hipLaunchKernelGGL((train_prep_kernel<DH, R>), grid_prep, dim3(kTrThreads), 0, st, kp);
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
  const unsigned grid_kv = unsigned(size_t(kp.n_kb) * H * B);
  hipLaunchKernelGGL((train_dkv_kernel<DH, R>), dim3(grid_kv), dim3(kTrThreads), size_t(lds_kv), st, kp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long nrow = (long long)(B * L * DH);
  hipLaunchKernelGGL(train_reduce_kernel, dim3(unsigned((nrow + 255) / 256)), dim3(256), 0, st, kp.dks_part, a.dk_s,
                     nrow, int(H));
  hipLaunchKernelGGL(train_reduce_kernel, dim3(unsigned((nrow + 255) / 256)), dim3(256), 0, st, kp.dvs_part, a.dv_s,
                     nrow, int(H));
  if constexpr (R > 0) {
    const long long nb = (long long)(H * DH * R);
    const int parts = int(B) * kp.n_kb;
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
