// LRKV causal prefill on bf16 MFMA at the ranks the rank-0/8/16/32 kernel
// does not take, up to 128: the trained ranks of the pages' models (slide
// "The rank directly sets the theoretical cache budget", Table 7: 46, 51,
// 54, 55; "Backup: the complete rank sweep clarifies the trade-off", Table
// 8: up to 128).  Same method, arguments and pipeline as prefill_kernel
// (slides "Compute logits without expanding historical keys", Eq. (6) with
// the causal mask, and "Aggregate values before the residual
// up-projection", Eq. (7)); what differs:
//   - a token's latent row in LDS is the run of the workgroup's 4 heads as
//     in HBM (4r elements, 4-byte aligned when heads * r is even), padded
//     to 4 RP elements (RP = 64 or 128) with the data that follows it (or
//     zeros past the array);
//   - wave w reads its head through an RP-element window that starts at
//     the 8-aligned element at or below w r: its first o_w = (w r) mod 8
//     rows and those past o_w + r belong to other heads, and the absorbed
//     query and B^V are zero there, so they add nothing to the logits and
//     the output;
//   - the value latents are RP/32 MFMA blocks of 32 rows; the softmax sum
//     is added up on the vector ALUs;
//   - a side is 24 KB (RP = 64) or 40 KB (RP = 128) with d_h = 128, so one
//     workgroup (one wave per SIMD) runs per compute unit, with up to 512
//     registers per lane.
#include "lrkv_device.h"
#include "lrkv_internal.h"

#include <algorithm>

namespace lrkv {

constexpr int kPwWaves = 4;                 // heads per workgroup
constexpr int kPwThreads = 64 * kPwWaves;
constexpr int kPwTile = 32;                 // key tokens per tile, query rows per wave
constexpr float kPwStale = 8.f;             // running-max refresh threshold (log2 units)
constexpr int kPwVmcntZero = 0x0F70;          // s_waitcnt immediate: vmcnt(0), expcnt and lgkmcnt not waited on
constexpr int kPwMaxPad = 128;              // window of latent rows per head in LDS: 64 or 128

// LDS tiles keep rows unpadded, with 16-byte chunk ch of row r at position
// ch ^ lds_swz(r, chunks per row); with it every read this kernel makes is
// free of bank conflicts: the 16-byte key and key-latent reads (16 rows, one
// chunk) and the transpose reads of values and value latents (4 rows x 2-4
// adjacent chunks), for rows of 64, 128 and 256 bytes.

template <int DH, int RP>
struct WideShape {
  static constexpr int KCH = DH / 16 + RP / 16;           // 16-wide chunks of the augmented key
  static constexpr int ZCH = RP / 16;                     // latent chunks
  static constexpr int LB = RP / 32;                      // 32-row blocks of the value latents
  static constexpr int VBLK = DH / 32 + LB;               // 32-row blocks of the augmented value
  // A side (the key side or the value side of one tile) in LDS: 32 shared
  // rows of RB bytes, then 32 token rows of ZB bytes holding the latents of
  // the workgroup's 4 heads, each padded to RP dims.
  static constexpr int RB = DH * 2, CR = RB / 16;
  static constexpr int ZB = kPwWaves * RP * 2, CZ = ZB / 16;
  static constexpr int SIDE = kPwTile * (RB + ZB);
  static constexpr int LDS = 4 * SIDE;                     // key side and value side, two of each
  static constexpr int NR = kPwTile * CR / 64;             // 1 KB DMA transfers per side: shared rows
  static constexpr int NZ = kPwTile * CZ / 64;             // and latents
  static constexpr int NRW = (NR + kPwWaves - 1) / kPwWaves;          // per wave
  static constexpr int NZW = (NZ + kPwWaves - 1) / kPwWaves;
  static_assert(DH % 32 == 0 && RP % 32 == 0 && RP <= kPwMaxPad, "wide prefill envelope");
  static_assert(CR >= 4 && CZ >= 4, "swizzle needs 4 chunks per row");
};

struct WideKernelParams {
  const uint16_t* q; const uint16_t* k_s; const uint16_t* v_s; const uint16_t* z_k; const uint16_t* z_v;
  const uint16_t* b_k; const uint16_t* b_v;
  uint16_t* out;
  int heads, seq_len, n_qblocks, n_hgroups, batch;
  // Keys and values: rows kv_stride tokens apart per sequence.  Without
  // history (start == NULL) they are the fresh tokens (kv_stride = seq_len);
  // with history they are the cache, where new token i of sequence b sits at
  // slot start[b] + i (start clamped to [0, max_start]).
  int kv_stride;
  const int32_t* start;
  int max_start;
  float scale_log2;
  int rank;                        // r: latent row length in HBM (every window fits in RP)
};

// Source byte offset (from the tile's first token) of latent chunk ch of
// token tok: with WIN, elements 8ch .. 8ch+7 of the run of the 4 heads'
// latents (4r of the row's 4 RP elements; past the run: the next token's
// data, or zeros past the array); without, dims 8(ch % (RP/8)) .. +7 of
// head ch / (RP/8) from that head's own row (past its r dims: the next
// row's data).
template <int RP, bool WIN>
__device__ __forceinline__ uint32_t pw_lat_src(int tok, int H, int r, int hg, int ch) {
  if constexpr (WIN) {
    return uint32_t(((tok * H + hg * kPwWaves) * r + 8 * ch) * 2);
  } else {
    const int hh = min(hg * kPwWaves + ch / (RP / 8), H - 1);
    return uint32_t(((tok * H + hh) * r + (ch % (RP / 8)) * 8) * 2);
  }
}

// This lane's source offsets (bytes from the first row of a tile) for the
// wave's share of one side's 1 KB transfers; the same for every tile, and for
// the key side and the value side.  Transfer j carries LDS bytes
// [1024j, 1024j+1024) of the side: lane i the chunk at position i of its row,
// i.e. source chunk (position ^ swizzle).
template <class P>
struct PwDmaOffsets {
  uint32_t row[P::NRW], lat[P::NZW];
};

template <int DH, int RP, bool WIN>
__device__ __forceinline__ PwDmaOffsets<WideShape<DH, RP>> pw_dma_offsets(int H, int r, int hg, int wave, int lane) {
  using P = WideShape<DH, RP>;
  PwDmaOffsets<P> d;
#pragma unroll
  for (int i = 0; i < P::NRW; ++i) {
    const int q = (wave + i * kPwWaves) * 64 + lane, row = q / P::CR, pos = q % P::CR;
    d.row[i] = uint32_t(row * P::RB + (pos ^ lds_swz(row, P::CR)) * 16);
  }
#pragma unroll
  for (int i = 0; i < P::NZW; ++i) {
    const int q = (wave + i * kPwWaves) * 64 + lane, tok = q / P::CZ, pos = q % P::CZ;
    const int ch = pos ^ lds_swz(tok, P::CZ);
    d.lat[i] = pw_lat_src<RP, WIN>(tok, H, r, hg, ch);
  }
  return d;
}

// Buffer resources over sequence b's part of one side's source arrays.
struct PwSources {
  __amdgpu_buffer_rsrc_t rows, lat;
};

template <int DH, int RP>
__device__ __forceinline__ PwSources pw_sources(const uint16_t* rows, const uint16_t* lat, const WideKernelParams& p,
                                                int b, int nkeys) {
  const size_t stride = size_t(p.kv_stride), n = size_t(nkeys);
  PwSources s;
  s.rows = buffer_resource(rows + size_t(b) * stride * DH, uint32_t(n * DH * 2));
  s.lat = buffer_resource(lat + size_t(b) * stride * p.heads * p.rank, uint32_t(n * p.heads * p.rank * 2));
  return s;
}

// Start the transfer of one side of key tile `kt` (tokens 32kt..32kt+31) into
// `side`: shared rows and the workgroup's heads' latents.  A whole tile adds
// a uniform tile offset to each lane's fixed offset; a tile reaching past the
// last token clamps its rows to token L-1 (their values are masked out of the
// softmax).  Each wave issues its share of the 1 KB transfers.
template <int DH, int RP, bool WIN>
__device__ __forceinline__ void pw_dma(unsigned char* side, const PwSources& src, const PwDmaOffsets<WideShape<DH, RP>>& d,
                                       const WideKernelParams& p, int hg, int kt, int wave, int lane, int L) {
  using P = WideShape<DH, RP>;
  const int H = p.heads, r = p.rank;
  if (kt * kPwTile + kPwTile <= L) {
#pragma unroll
    for (int i = 0; i < P::NRW; ++i) {
      const int j = wave + i * kPwWaves;
      // every wave has a transfer at i when the count divides evenly: no branch
      if (P::NR % kPwWaves == 0 || j < P::NR) dma16(src.rows, d.row[i], uint32_t(kt * kPwTile * P::RB), side + j * 1024);
    }
#pragma unroll
    for (int i = 0; i < P::NZW; ++i) {
      const int j = wave + i * kPwWaves;
      if (P::NZ % kPwWaves == 0 || j < P::NZ)
        dma16(src.lat, d.lat[i], uint32_t(kt * kPwTile * H * r * 2), side + kPwTile * P::RB + j * 1024);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < P::NRW; ++i) {
    const int j = wave + i * kPwWaves;
    if (j < P::NR) {
      const int q = j * 64 + lane, row = q / P::CR, pos = q % P::CR;
      const int t = min(kt * kPwTile + row, L - 1);
      dma16(src.rows, uint32_t(t * P::RB + (pos ^ lds_swz(row, P::CR)) * 16), 0u, side + j * 1024);
    }
  }
#pragma unroll
  for (int i = 0; i < P::NZW; ++i) {
    const int j = wave + i * kPwWaves;
    if (j < P::NZ) {
      const int q = j * 64 + lane, tok = q / P::CZ, pos = q % P::CZ;
      const int ch = pos ^ lds_swz(tok, P::CZ);
      const int t = min(kt * kPwTile + tok, L - 1);
      dma16(src.lat, pw_lat_src<RP, WIN>(t, H, r, hg, ch), 0u, side + kPwTile * P::RB + j * 1024);
    }
  }
}

// S^T tile (32 tokens x 32 queries) of one head from a key side: Kaug .
// Qaug^T; lane (query n, half) gets tokens 8(r/4)+4half+r%4.  The lane's
// A-operand k-slots of chunk c are dims 16c+8half..16c+8half+7, one 16-byte
// chunk of token row n (koff[c] / zoff[c] hold its swizzled offsets).  The
// operand reads run kPwAhead chunks ahead of the MFMA chain (scheduling
// barriers keep that order), so each MFMA waits for a read issued several
// MFMAs earlier instead of a full LDS round trip.
constexpr int kPwAhead = 3;

template <int DH, int RP>
__device__ __forceinline__ f32x16_t pw_scores(const unsigned char* side, const bf16x8_t (&qop)[WideShape<DH, RP>::KCH],
                                              const int (&koff)[DH / 16], const int (&zoff)[WideShape<DH, RP>::ZCH],
                                              int half) {
  using P = WideShape<DH, RP>;
  u32x4 ka[P::KCH];
  auto rd = [&](int c) __attribute__((always_inline)) {
    if (c < DH / 16) {
      ka[c] = *reinterpret_cast<const u32x4*>(side + koff[c]);
    } else {
      ka[c] = *reinterpret_cast<const u32x4*>(side + zoff[c - DH / 16]);
    }
  };
#pragma unroll
  for (int c = 0; c < kPwAhead && c < P::KCH; ++c) rd(c);
  f32x16_t s = {};
#pragma unroll
  for (int c = 0; c < P::KCH; ++c) {
    if (c + kPwAhead < P::KCH) rd(c + kPwAhead);
    __builtin_amdgcn_sched_barrier(0);
    s = mfma32(as_bf16x8(ka[c]), qop[c], s);
    __builtin_amdgcn_sched_barrier(0);
  }
  return s;
}

template <int DH, int RP, bool WIN>
__global__ __attribute__((amdgpu_flat_work_group_size(kPwThreads, kPwThreads), amdgpu_waves_per_eu(1)))
void prefill_wide_kernel(WideKernelParams p) {
  using P = WideShape<DH, RP>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, half = lane >> 5;
  // 1-D grid, heaviest query blocks first over the whole launch (block qb
  // scans qb+1 key tiles), batch fastest so that consecutive blocks, which
  // the dispatcher spreads round-robin over the XCDs, keep one sequence per
  // XCD when the batch divides 8.
  const int per_level = p.n_hgroups * p.batch;
  const int qb = p.n_qblocks - 1 - int(blockIdx.x) / per_level;
  const int rem = int(blockIdx.x) % per_level;
  const int b = rem % p.batch, hg = rem / p.batch;
  const int H = p.heads, L = p.seq_len, rk = p.rank;
  const int h = hg * kPwWaves + wave;
  const bool head_ok = h < H;
  const int hh = head_ok ? h : H - 1;
  const int q0 = qb * kPwTile;
  const int qrow = min(q0 + n, L - 1);
  // History: the block's queries sit at positions start + q0 .. and see the
  // keys up to their own position; nkeys keys in all.
  int start = p.start ? p.start[b] : 0;
  start = start < 0 ? 0 : (start > p.max_start ? p.max_start : start);
  const int qpos0 = start + q0;
  const int nkeys = start + L;
  const int kt_last = min(qpos0 + kPwTile - 1, nkeys - 1) / kPwTile;   // last key tile of this block

  // Per-lane LDS offsets inside a side (loop-invariant).
  int koff[DH / 16], zoff[P::ZCH];
#pragma unroll
  for (int c = 0; c < DH / 16; ++c) koff[c] = n * P::RB + ((2 * c + half) ^ lds_swz(n, P::CR)) * 16;
  // With WIN this wave's head sits at elements [wave r, wave r + r) of the
  // run; it reads the RP-element window from the 8-aligned element at or
  // below, whose first o_w elements belong to the previous head (o_w < 8,
  // and r + o_w <= RP: the host picks RP so).  Without, its padded row.
  const int wstart = WIN ? (wave * rk) & ~7 : wave * RP, o_w = WIN ? wave * rk - wstart : 0;
#pragma unroll
  for (int c = 0; c < P::ZCH; ++c) {
    const int ch = wstart / 8 + 2 * c + half;
    zoff[c] = kPwTile * P::RB + n * P::ZB + (ch ^ lds_swz(n, P::CZ)) * 16;
  }
  // Transpose reads of a 16-token value chunk: this lane addresses token
  // 4*half + k (k = lane bits 2-3) at features 16*(lane bit 4) + 4*(lane
  // bits 0-1) of each 32-feature block (first read), and token + 8 (second
  // read; its swizzle differs).  Rows +16 share the swizzle.
  const int tr_tok = 4 * half + ((lane >> 2) & 3);
  int voff[DH / 32][2];
#pragma unroll
  for (int f = 0; f < DH / 32; ++f) {
    const int ch = 4 * f + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = tr_tok + 8 * j;
      voff[f][j] = row * P::RB + (ch ^ lds_swz(row, P::CR)) * 16 + 8 * (lane & 1);
    }
  }
  // Value latents, block v (padded dims 32v .. 32v+31), token rows as the
  // shared values.
  int zvoff[P::LB][2][2];
#pragma unroll
  for (int v = 0; v < P::LB; ++v) {
    const int feat = 32 * v + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int byte = (wstart + feat) * 2;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = 16 * c + tr_tok + 8 * j;
        zvoff[v][c][j] = kPwTile * P::RB + row * P::ZB + ((byte / 16) ^ lds_swz(row, P::CZ)) * 16 + byte % 16;
      }
  }
  const PwDmaOffsets<P> dma = pw_dma_offsets<DH, RP, WIN>(H, rk, hg, wave, lane);

  // ---- query rows (B operands, K-dim = features): lane (query n, half) ----
  bf16x8_t qop[P::KCH];
  {
    const uint16_t* qr = p.q + ((size_t(b) * L + qrow) * H + hh) * DH;
#pragma unroll
    for (int c = 0; c < DH / 16; ++c) qop[c] = as_bf16x8(*reinterpret_cast<const u32x4*>(qr + 16 * c + 8 * half));
  }
  {
    // absorbed query, transposed, per block v of 32 padded latent dims:
    // (latent j x query n) = (B^K_h)^T (j x d) . Q^T (d x n), rows j >= r zero
    f32x16_t qt[P::LB];
    const uint16_t* bk = p.b_k + size_t(hh) * DH * rk;
#pragma unroll
    for (int v = 0; v < P::LB; ++v) {
      qt[v] = f32x16_t{};
      const int j = 32 * v + n - o_w;                   // window row -> latent dim
#pragma unroll
      for (int c = 0; c < DH / 16; ++c) {
        bf16x8_t a;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const bool ok = j >= 0 && j < rk;
          const uint16_t x = bk[size_t(16 * c + 8 * half + i) * rk + (ok ? j : 0)];
          a[i] = __builtin_bit_cast(__bf16, ok ? x : uint16_t(0));
        }
        qt[v] = mfma32(a, qop[c], qt[v]);
      }
    }
    // The accumulator gives lane half the latent dims 16c + {4half..4half+3,
    // 8+4half..8+4half+3}; the key latents are read as dims 16c+8half..+7, so
    // the halves trade dims 8-11 (half 0) for 4-7 (half 1).
#pragma unroll
    for (int c = 0; c < P::ZCH; ++c) {
      const f32x16_t& q2 = qt[c / 2];
      const int c2 = c % 2;
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(q2[8 * c2 + 2 * i], q2[8 * c2 + 2 * i + 1]);
      const uint32_t s0 = half ? w[0] : w[2], s1 = half ? w[1] : w[3];
      const uint32_t r0 = uint32_t(__shfl_xor(int(s0), 32)), r1 = uint32_t(__shfl_xor(int(s1), 32));
      if (half) { w[0] = r0; w[1] = r1; } else { w[2] = r0; w[3] = r1; }
      qop[DH / 16 + c] = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
    }
  }

  f32x16_t oacc[P::VBLK];
#pragma unroll
  for (int f = 0; f < P::VBLK; ++f) oacc[f] = f32x16_t{};
  float m = -INFINITY, lsum = 0.f;

  // Software pipeline over key tiles: the key side runs one tile ahead of the
  // value side, so that the score MFMAs of tile kt+1 are issued before the
  // softmax of tile kt and overlap it.  Key side of tile t in kside(t & 1),
  // value side in vside(t & 1).  Step kt reads kside((kt+1)&1) and
  // vside(kt&1) and refills kside(kt&1) (tile kt+2) and vside((kt+1)&1)
  // (tile kt+1), both last read in step kt-1: one barrier per tile.
  unsigned char* const kside0 = smem;
  unsigned char* const vside0 = smem + 2 * P::SIDE;
  const PwSources ksrc = pw_sources<DH, RP>(p.k_s, p.z_k, p, b, nkeys);
  const PwSources vsrc = pw_sources<DH, RP>(p.v_s, p.z_v, p, b, nkeys);
  pw_dma<DH, RP, WIN>(kside0, ksrc, dma, p, hg, 0, wave, lane, nkeys);
  pw_dma<DH, RP, WIN>(vside0, vsrc, dma, p, hg, 0, wave, lane, nkeys);
  if (kt_last >= 1) pw_dma<DH, RP, WIN>(kside0 + P::SIDE, ksrc, dma, p, hg, 1, wave, lane, nkeys);
  __builtin_amdgcn_s_waitcnt(kPwVmcntZero);
  __syncthreads();
  f32x16_t s0 = pw_scores<DH, RP>(kside0, qop, koff, zoff, half);
  __syncthreads();                                         // kside(0) is refilled in step 0

  // One pipeline step; the two score tiles swap roles every step (the loop
  // is unrolled by two so that no accumulator is copied).
  auto step = [&](const int kt, f32x16_t& s_cur, f32x16_t& s_nxt) __attribute__((always_inline)) {
    const bool next_k = kt + 2 <= kt_last, next_v = kt + 1 <= kt_last;
    if (next_v) s_nxt = pw_scores<DH, RP>(kside0 + ((kt + 1) & 1) * P::SIDE, qop, koff, zoff, half);

    // value operands of tile kt: lane (feature n, half) gets tokens
    // {4half..4half+3, 8+4half..8+4half+3} of each 16-token chunk, the k-slot
    // order of P^T below
    const unsigned char* vs = vside0 + (kt & 1) * P::SIDE;
    u32x4 va[P::VBLK][2];
#pragma unroll
    for (int f = 0; f < DH / 32; ++f)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint2 lo = lds_read_tr16(vs + 16 * c * P::RB + voff[f][0]);
        const uint2 hi = lds_read_tr16(vs + 16 * c * P::RB + voff[f][1]);
        va[f][c] = u32x4{lo.x, lo.y, hi.x, hi.y};
      }
#pragma unroll
    for (int v = 0; v < P::LB; ++v)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint2 lo = lds_read_tr16(vs + zvoff[v][c][0]), hi = lds_read_tr16(vs + zvoff[v][c][1]);
        va[DH / 32 + v][c] = u32x4{lo.x, lo.y, hi.x, hi.y};
      }
    // Refill the buffers read in the previous step.  Issued after this step's
    // LDS reads, which therefore never wait on the transfers; they overlap
    // the softmax and the value MFMAs.
    if (next_k) pw_dma<DH, RP, WIN>(kside0 + (kt & 1) * P::SIDE, ksrc, dma, p, hg, kt + 2, wave, lane, nkeys);
    if (next_v) pw_dma<DH, RP, WIN>(vside0 + ((kt + 1) & 1) * P::SIDE, vsrc, dma, p, hg, kt + 1, wave, lane, nkeys);

    // online softmax (log2 domain) for the query at position qpos0 + n.
    // Only tiles reaching past the block's first query position (the
    // diagonal) or past the last key need the mask, applied in place to the
    // score registers (dead after this step), so both paths leave the scores
    // where the common code expects them.  The running max is refreshed only
    // when a score exceeds it by more than kPwStale (log2 units): weights
    // then stay <= 2^kPwStale, and since the sum and the output use the same
    // reference the result is unchanged.
    if (kt * kPwTile + kPwTile - 1 > qpos0 || kt * kPwTile + kPwTile > nkeys) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = kt * kPwTile + 8 * (r >> 2) + 4 * half + (r & 3);
        if (!(tok <= qpos0 + n && tok < nkeys)) s_cur[r] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s_cur[r]);
    // Lanes n and n+32 share query n and must share m, so the refresh is
    // decided for the whole wave; the common case exchanges nothing.
    if (__builtin_amdgcn_ballot_w64(mx * p.scale_log2 > m + kPwStale)) {
      const float mn = fmaxf(m, fmaxf(mx, __shfl_xor(mx, 32)) * p.scale_log2);  // finite: key 0 <= qpos0 + n
      const float alpha = fast_exp2(m - mn);               // 0 on the first tile (m = -inf)
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int f = 0; f < P::VBLK; ++f) oacc[f] *= alpha;
    }
    float sv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sv[r] = fast_exp2(__builtin_fmaf(s_cur[r], p.scale_log2, -m));
      lsum += sv[r];                                        // this lane's 16 tokens; halves combined at the end
    }
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

    __builtin_amdgcn_s_waitcnt(kPwVmcntZero);                // this wave's transfers have landed
    __syncthreads();
  };
  f32x16_t s1 = {};
  for (int kt = 0;; kt += 2) {
    step(kt, s0, s1);
    if (kt + 1 > kt_last) break;
    step(kt + 1, s1, s0);
    if (kt + 2 > kt_last) break;
  }

  if (!head_ok) return;
  // softmax sum of query n: the two halves' partial sums
  lsum += __shfl_xor(lsum, 32);
  // ---- epilogue: O_s += B^V_h . O_z^T, then divide by the softmax sum ----
  // B^V_h is zero outside the head's dims (window rows o_w .. o_w + r - 1;
  // O_z holds finite values in the others).
#pragma unroll
  for (int c = 0; c < P::ZCH; ++c) {
    bf16x8_t bz;                                          // O_z^T k-slots, accumulator order
#pragma unroll
    for (int i = 0; i < 8; ++i) bz[i] = (__bf16)oacc[DH / 32 + c / 2][8 * (c % 2) + i];
#pragma unroll
    for (int f = 0; f < DH / 32; ++f) {
      const uint16_t* bv = p.b_v + (size_t(hh) * DH + 32 * f + n) * rk;
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // window rows e, e + 1 -> latent dims e - o_w, e + 1 - o_w (without
        // WIN: o_w = 0 and r even, so the pair is whole on one side of r)
        const int j = 16 * c + 8 * (k >> 1) + 4 * half + 2 * (k & 1) - o_w;
        if constexpr (WIN) {
          const uint32_t lo = (j >= 0 && j < rk) ? bv[j] : 0u, hi = (j + 1 >= 0 && j + 1 < rk) ? bv[j + 1] : 0u;
          w[k] = lo | (hi << 16);
        } else {
          w[k] = j < rk ? *reinterpret_cast<const uint32_t*>(bv + j) : 0u;
        }
      }
      oacc[f] = mfma32(as_bf16x8(u32x4{w[0], w[1], w[2], w[3]}), bz, oacc[f]);
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

template <int DH, int RP, bool WIN>
static hipError_t launch_wide_t(const PrefillArgs& a, hipStream_t st) {
  using P = WideShape<DH, RP>;
  WideKernelParams kp;
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
  kp.n_qblocks = (a.seq_len + kPwTile - 1) / kPwTile;
  kp.n_hgroups = (a.heads + kPwWaves - 1) / kPwWaves;
  kp.batch = a.batch;
  kp.scale_log2 = a.scale_log2;
  kp.kv_stride = a.kv_stride;
  kp.start = a.start;
  kp.max_start = a.max_start;
  kp.rank = a.rank;
  const long long blocks = (long long)kp.n_qblocks * kp.n_hgroups * a.batch;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid{static_cast<unsigned>(blocks)};
  const size_t lds = size_t(P::LDS);
  const hipError_t attr = allow_dynamic_lds<&prefill_wide_kernel<DH, RP, WIN>>(int(lds));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((prefill_wide_kernel<DH, RP, WIN>), grid, dim3(kPwThreads), lds, st, kp);
  return hipGetLastError();
}

// Latent rows per head in LDS for rank r: the smallest of 64 and 128 that
// holds the head's rows: r for an even rank (each head's own row, padded),
// r plus the window offset o_w = (w r) mod 8, w < 4, for an odd one; 0 if
// neither does.
static int wide_pad(int r) {
  int need = r;
  if (r % 2)
    for (int w = 1; w < kPwWaves; ++w) need = std::max(need, r + ((w * r) & 7));
  return need <= 64 ? 64 : need <= kPwMaxPad ? kPwMaxPad : 0;
}

// Ranks 1-128 with the transfers' sources 4-byte aligned in HBM: an even
// rank (every head's row), or an odd one with an even number of heads
// (every 4-head run starts at an even element), whose windows fit.
bool prefill_wide_supported(int dtype, int head_dim, int rank, int heads) {
  return dtype == 1 && (head_dim == 64 || head_dim == 128) && rank >= 1 && rank <= kPwMaxPad && heads >= 1 &&
         (heads % 2 == 0 || rank % 2 == 0) && wide_pad(rank) > 0;
}

hipError_t launch_prefill_wide(const PrefillArgs& a, hipStream_t st) {
  // the training forward's log-sum-exp output is the rank 0-32 kernel's only
  if (!prefill_wide_supported(1, a.head_dim, a.rank, a.heads) || a.lse) return hipErrorInvalidValue;
  const bool odd = a.rank % 2, d64 = a.head_dim == 64;
  if (wide_pad(a.rank) == 64) {
    if (odd) return d64 ? launch_wide_t<64, 64, true>(a, st) : launch_wide_t<128, 64, true>(a, st);
    return d64 ? launch_wide_t<64, 64, false>(a, st) : launch_wide_t<128, 64, false>(a, st);
  }
  if (odd) return d64 ? launch_wide_t<64, 128, true>(a, st) : launch_wide_t<128, 128, true>(a, st);
  return d64 ? launch_wide_t<64, 128, false>(a, st) : launch_wide_t<128, 128, false>(a, st);
}

hipError_t prefill_wide_prepare() {
  hipError_t e = hipSuccess;
#define LRKV_PW(DHV, RPV, W) \
  if (e == hipSuccess) e = allow_dynamic_lds<&prefill_wide_kernel<DHV, RPV, W>>(WideShape<DHV, RPV>::LDS);
  LRKV_PW(64, 64, false) LRKV_PW(128, 64, false) LRKV_PW(64, 128, false) LRKV_PW(128, 128, false)
  LRKV_PW(64, 64, true) LRKV_PW(128, 64, true) LRKV_PW(64, 128, true) LRKV_PW(128, 128, true)
#undef LRKV_PW
  return e;
}

}  // namespace lrkv
