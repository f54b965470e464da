// LRKV causal prefill on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16).
//
// Method (Low-Rank Key Value Attention, slide discussion of arXiv:2601.11471v3):
// with L new tokens, every query row i of head h attends to keys j <= i
// (slide "Compute logits without expanding historical keys", Eq. (6), causal
// mask); with start tokens of history already cached, new token i sits at
// position start + i and attends to the cached keys j <= start + i.  Both go
// through the absorbed forms
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
//   are taken in the order the accumulator layout provides).  Value rows sit
//   in LDS row-major like the keys; the transposed A operand comes from LDS
//   transpose reads (ds_read_b64_tr_b16), whose per-lane row addresses put
//   the tokens in that same order.
// The absorbed query Q B^K_h and the residual up-projection O_z (B^V_h)^T are
// MFMA products too.  Softmax runs in fp32 in the log2 domain; P, the absorbed
// query and O_z enter MFMAs rounded to bf16.
#include "lrkv_device.h"
#include "lrkv_internal.h"

namespace lrkv {

constexpr int kPfWaves = 4;                 // heads per workgroup
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfTile = 32;                 // key tokens per tile, query rows per wave
constexpr float kPfStale = 8.f;             // running-max refresh threshold (log2 units)
constexpr int kVmcntZero = 0x0F70;          // s_waitcnt immediate: vmcnt(0), expcnt and lgkmcnt not waited on

// LDS tiles keep rows unpadded, with 16-byte chunk ch of row r at position
// ch ^ lds_swz(r, chunks per row); with it every read this kernel makes is
// free of bank conflicts: the 16-byte key and key-latent reads (16 rows, one
// chunk) and the transpose reads of values and value latents (4 rows x 2-4
// adjacent chunks), for rows of 64, 128 and 256 bytes.

template <int DH, int R>
struct PrefillShape {
  static constexpr int RK = (R + 15) / 16 * 16;          // latent dims padded for the K-dim chunks
  static constexpr int KCH = DH / 16 + RK / 16;           // 16-wide chunks of the augmented key
  static constexpr int ZCH = RK / 16 > 0 ? RK / 16 : 1;   // latent chunks (array extent)
  static constexpr int VBLK = DH / 32 + (R > 0 ? 1 : 0);  // 32-row blocks of the augmented value
  // With 0 < R < 32 row R of the latent value block is padding; a row of ones
  // there makes the value MFMAs accumulate the softmax sum as well.
  static constexpr bool SUM_ROW = R > 0 && R < 32;
  static constexpr int SUM_REG = R / 2;                    // accumulator register of row R in lanes 0-31
  // A side (the key side or the value side of one tile) in LDS: 32 shared
  // rows of RB bytes, then 32 token rows of ZB bytes holding the latents of
  // the workgroup's 4 heads, [token][head][rank] as in HBM, then 16 constant
  // bytes (bf16 1, 0, 0, 0) that feed the ones row of the value latents.
  static constexpr int RB = DH * 2, CR = RB / 16;
  static constexpr int ZB = kPfWaves * R * 2, CZ = ZB / 16;
  static constexpr int ONES = kPfTile * (RB + ZB);         // offset of the constant inside a side
  static constexpr int SIDE = ONES + 16;
  static constexpr int LDS = 4 * SIDE;                     // key side and value side, two of each
  static constexpr int NR = kPfTile * CR / 64;             // 1 KB DMA transfers per side: shared rows
  static constexpr int NZ = kPfTile * CZ / 64;             // and latents
  static constexpr int NRW = (NR + kPfWaves - 1) / kPfWaves;          // per wave
  static constexpr int NZW = NZ > 0 ? (NZ + kPfWaves - 1) / kPfWaves : 1;
  static_assert(DH % 32 == 0 && R <= 32 && R % 8 == 0, "prefill envelope");
  static_assert(CR >= 4 && (R == 0 || CZ >= 4), "swizzle needs 4 chunks per row");
};

struct PrefillKernelParams {
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
  // Optional: the natural log-sum-exp of each query row's scaled logits,
  // [batch][seq_len][heads] fp32 (NULL: not written).
  float* lse;
};

// This lane's source offsets (bytes from the first row of a tile) for the
// wave's share of one side's 1 KB transfers; the same for every tile, and for
// the key side and the value side.  Transfer j carries LDS bytes
// [1024j, 1024j+1024) of the side: lane i the chunk at position i of its row,
// i.e. source chunk (position ^ swizzle).
template <class P>
struct PfDmaOffsets {
  uint32_t row[P::NRW], lat[P::NZW];
};

template <int DH, int R>
__device__ __forceinline__ PfDmaOffsets<PrefillShape<DH, R>> pf_dma_offsets(int H, int hg, int wave, int lane) {
  using P = PrefillShape<DH, R>;
  PfDmaOffsets<P> d;
#pragma unroll
  for (int i = 0; i < P::NRW; ++i) {
    const int q = (wave + i * kPfWaves) * 64 + lane, row = q / P::CR, pos = q % P::CR;
    d.row[i] = uint32_t(row * P::RB + (pos ^ lds_swz(row, P::CR)) * 16);
  }
#pragma unroll
  for (int i = 0; i < P::NZW; ++i) {
    d.lat[i] = 0;
    if constexpr (R > 0) {
      const int q = (wave + i * kPfWaves) * 64 + lane, tok = q / P::CZ, pos = q % P::CZ;
      const int ch = pos ^ lds_swz(tok, P::CZ);              // chunk of the 4 heads' latents of token tok
      const int hh = min(hg * kPfWaves + ch / (R / 8), H - 1);
      d.lat[i] = uint32_t(((tok * H + hh) * R + (ch % (R / 8)) * 8) * 2);
    }
  }
  return d;
}

// Buffer resources over sequence b's part of one side's source arrays.
struct PfSources {
  __amdgpu_buffer_rsrc_t rows, lat;
};

template <int DH, int R>
__device__ __forceinline__ PfSources pf_sources(const uint16_t* rows, const uint16_t* lat, const PrefillKernelParams& p,
                                                int b, int nkeys) {
  const size_t stride = size_t(p.kv_stride), n = size_t(nkeys);
  PfSources s;
  s.rows = buffer_resource(rows + size_t(b) * stride * DH, uint32_t(n * DH * 2));
  s.lat = buffer_resource(lat + size_t(b) * stride * p.heads * R, uint32_t(n * p.heads * (R > 0 ? R : 1) * 2));
  return s;
}

// Start the transfer of one side of key tile `kt` (tokens 32kt..32kt+31) into
// `side`: shared rows and the workgroup's heads' latents.  A whole tile adds
// a uniform tile offset to each lane's fixed offset; a tile reaching past the
// last token clamps its rows to token L-1 (their values are masked out of the
// softmax).  Each wave issues its share of the 1 KB transfers.
template <int DH, int R>
__device__ __forceinline__ void pf_dma(unsigned char* side, const PfSources& src, const PfDmaOffsets<PrefillShape<DH, R>>& d,
                                       const PrefillKernelParams& p, int hg, int kt, int wave, int lane, int L) {
  using P = PrefillShape<DH, R>;
  const int H = p.heads;
  if (kt * kPfTile + kPfTile <= L) {
#pragma unroll
    for (int i = 0; i < P::NRW; ++i) {
      const int j = wave + i * kPfWaves;
      // every wave has a transfer at i when the count divides evenly: no branch
      if (P::NR % kPfWaves == 0 || j < P::NR) dma16(src.rows, d.row[i], uint32_t(kt * kPfTile * P::RB), side + j * 1024);
    }
    if constexpr (R > 0) {
#pragma unroll
      for (int i = 0; i < P::NZW; ++i) {
        const int j = wave + i * kPfWaves;
        if (P::NZ % kPfWaves == 0 || j < P::NZ)
          dma16(src.lat, d.lat[i], uint32_t(kt * kPfTile * H * R * 2), side + kPfTile * P::RB + j * 1024);
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < P::NRW; ++i) {
    const int j = wave + i * kPfWaves;
    if (j < P::NR) {
      const int q = j * 64 + lane, row = q / P::CR, pos = q % P::CR;
      const int t = min(kt * kPfTile + row, L - 1);
      dma16(src.rows, uint32_t(t * P::RB + (pos ^ lds_swz(row, P::CR)) * 16), 0u, side + j * 1024);
    }
  }
  if constexpr (R > 0) {
#pragma unroll
    for (int i = 0; i < P::NZW; ++i) {
      const int j = wave + i * kPfWaves;
      if (j < P::NZ) {
        const int q = j * 64 + lane, tok = q / P::CZ, pos = q % P::CZ;
        const int ch = pos ^ lds_swz(tok, P::CZ);            // chunk of the 4 heads' latents of token tok
        const int t = min(kt * kPfTile + tok, L - 1);
        const int hh = min(hg * kPfWaves + ch / (R / 8), H - 1);
        dma16(src.lat, uint32_t(((t * H + hh) * R + (ch % (R / 8)) * 8) * 2), 0u, side + kPfTile * P::RB + j * 1024);
      }
    }
  }
}

// S^T tile (32 tokens x 32 queries) of one head from a key side: Kaug .
// Qaug^T; lane (query n, half) gets tokens 8(r/4)+4half+r%4.  The lane's
// A-operand k-slots of chunk c are dims 16c+8half..16c+8half+7, one 16-byte
// chunk of token row n (koff[c] / zoff[c] hold its swizzled offsets).  The
// operand reads run kPfAhead chunks ahead of the MFMA chain (scheduling
// barriers keep that order), so each MFMA waits for a read issued several
// MFMAs earlier instead of a full LDS round trip.
constexpr int kPfAhead = 3;

template <int DH, int R>
__device__ __forceinline__ f32x16_t pf_scores(const unsigned char* side, const bf16x8_t (&qop)[PrefillShape<DH, R>::KCH],
                                              const int (&koff)[DH / 16], const int (&zoff)[PrefillShape<DH, R>::ZCH],
                                              int half) {
  using P = PrefillShape<DH, R>;
  u32x4 ka[P::KCH];
  auto rd = [&](int c) __attribute__((always_inline)) {
    if (c < DH / 16) {
      ka[c] = *reinterpret_cast<const u32x4*>(side + koff[c]);
    } else if constexpr (R > 0) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(side + zoff[c - DH / 16]);
      ka[c] = (R == 8 && half) ? u32x4{0u, 0u, 0u, 0u} : v;   // R = 8: dims 8..15 are padding
    }
  };
#pragma unroll
  for (int c = 0; c < kPfAhead && c < P::KCH; ++c) rd(c);
  f32x16_t s = {};
#pragma unroll
  for (int c = 0; c < P::KCH; ++c) {
    if (c + kPfAhead < P::KCH) rd(c + kPfAhead);
    __builtin_amdgcn_sched_barrier(0);
    s = mfma32(as_bf16x8(ka[c]), qop[c], s);
    __builtin_amdgcn_sched_barrier(0);
  }
  return s;
}

template <int DH, int R>
__global__ __attribute__((amdgpu_flat_work_group_size(kPfThreads, kPfThreads), amdgpu_waves_per_eu(2)))
void prefill_kernel(PrefillKernelParams p) {
  using P = PrefillShape<DH, R>;
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
  const int H = p.heads, L = p.seq_len;
  const int h = hg * kPfWaves + wave;
  const bool head_ok = h < H;
  const int hh = head_ok ? h : H - 1;
  const int q0 = qb * kPfTile;
  const int qrow = min(q0 + n, L - 1);
  // History: the block's queries sit at positions start + q0 .. and see the
  // keys up to their own position; nkeys keys in all.
  int start = p.start ? p.start[b] : 0;
  start = start < 0 ? 0 : (start > p.max_start ? p.max_start : start);
  const int qpos0 = start + q0;
  const int nkeys = start + L;
  const int kt_last = min(qpos0 + kPfTile - 1, nkeys - 1) / kPfTile;   // last key tile of this block

  // Per-lane LDS offsets inside a side (loop-invariant).
  int koff[DH / 16], zoff[P::ZCH];
#pragma unroll
  for (int c = 0; c < DH / 16; ++c) koff[c] = n * P::RB + ((2 * c + half) ^ lds_swz(n, P::CR)) * 16;
  if constexpr (R > 0) {
#pragma unroll
    for (int c = 0; c < P::RK / 16; ++c) {
      const int ch = wave * (R / 8) + (R == 8 ? 0 : 2 * c + half);
      zoff[c] = kPfTile * P::RB + n * P::ZB + (ch ^ lds_swz(n, P::CZ)) * 16;
    }
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
  // Value latents: lanes addressing dims < R read them; the lanes whose 4
  // dims start at R read the constant (1, 0, 0, 0), which turns latent row R
  // into a row of ones (the softmax sum); rows above R are never used, so
  // their lanes just read some valid latent row.
  int zvoff[2][2] = {{0, 0}, {0, 0}};
  if constexpr (R > 0) {
    const int feat = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int byte = wave * R * 2 + (feat < R ? feat : 0) * 2;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = 16 * c + tr_tok + 8 * j;
        zvoff[c][j] = (P::SUM_ROW && feat == R)
                          ? P::ONES
                          : kPfTile * P::RB + row * P::ZB + ((byte / 16) ^ lds_swz(row, P::CZ)) * 16 + byte % 16;
      }
  }
  const PfDmaOffsets<P> dma = pf_dma_offsets<DH, R>(H, hg, wave, lane);

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
        const uint16_t v = bk[size_t(16 * c + 8 * half + i) * R + (n < R ? n : 0)];
        a[i] = __builtin_bit_cast(__bf16, n < R ? v : uint16_t(0));
      }
      qt = mfma32(a, qop[c], qt);
    }
    // The accumulator gives lane half the latent dims 16c + {4half..4half+3,
    // 8+4half..8+4half+3}; the key latents are read as dims 16c+8half..+7, so
    // the halves trade dims 8-11 (half 0) for 4-7 (half 1).
#pragma unroll
    for (int c = 0; c < P::RK / 16; ++c) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(qt[8 * c + 2 * i], qt[8 * c + 2 * i + 1]);
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
  if (tid < 2) *reinterpret_cast<uint4*>(vside0 + tid * P::SIDE + P::ONES) = make_uint4(0x3F80u, 0u, 0u, 0u);
  const PfSources ksrc = pf_sources<DH, R>(p.k_s, p.z_k, p, b, nkeys);
  const PfSources vsrc = pf_sources<DH, R>(p.v_s, p.z_v, p, b, nkeys);
  pf_dma<DH, R>(kside0, ksrc, dma, p, hg, 0, wave, lane, nkeys);
  pf_dma<DH, R>(vside0, vsrc, dma, p, hg, 0, wave, lane, nkeys);
  if (kt_last >= 1) pf_dma<DH, R>(kside0 + P::SIDE, ksrc, dma, p, hg, 1, wave, lane, nkeys);
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  __syncthreads();
  f32x16_t s0 = pf_scores<DH, R>(kside0, qop, koff, zoff, half);
  __syncthreads();                                         // kside(0) is refilled in step 0

  // One pipeline step; the two score tiles swap roles every step (the loop
  // is unrolled by two so that no accumulator is copied).
  auto step = [&](const int kt, f32x16_t& s_cur, f32x16_t& s_nxt) __attribute__((always_inline)) {
    const bool next_k = kt + 2 <= kt_last, next_v = kt + 1 <= kt_last;
    if (next_v) s_nxt = pf_scores<DH, R>(kside0 + ((kt + 1) & 1) * P::SIDE, qop, koff, zoff, half);

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
    if constexpr (R > 0) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint2 lo = lds_read_tr16(vs + zvoff[c][0]), hi = lds_read_tr16(vs + zvoff[c][1]);
        va[DH / 32][c] = u32x4{lo.x, lo.y, hi.x, hi.y};
      }
    }
    // Refill the buffers read in the previous step.  Issued after this step's
    // LDS reads, which therefore never wait on the transfers; they overlap
    // the softmax and the value MFMAs.
    if (next_k) pf_dma<DH, R>(kside0 + (kt & 1) * P::SIDE, ksrc, dma, p, hg, kt + 2, wave, lane, nkeys);
    if (next_v) pf_dma<DH, R>(vside0 + ((kt + 1) & 1) * P::SIDE, vsrc, dma, p, hg, kt + 1, wave, lane, nkeys);

    // online softmax (log2 domain) for the query at position qpos0 + n.
    // Only tiles reaching past the block's first query position (the
    // diagonal) or past the last key need the mask, applied in place to the
    // score registers (dead after this step), so both paths leave the scores
    // where the common code expects them.  The running max is refreshed only
    // when a score exceeds it by more than kPfStale (log2 units): weights
    // then stay <= 2^kPfStale, and since the sum and the output use the same
    // reference the result is unchanged.
    if (kt * kPfTile + kPfTile - 1 > qpos0 || kt * kPfTile + kPfTile > nkeys) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = kt * kPfTile + 8 * (r >> 2) + 4 * half + (r & 3);
        if (!(tok <= qpos0 + n && tok < nkeys)) s_cur[r] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s_cur[r]);
    // Lanes n and n+32 share query n and must share m, so the refresh is
    // decided for the whole wave; the common case exchanges nothing.
    if (__builtin_amdgcn_ballot_w64(mx * p.scale_log2 > m + kPfStale)) {
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
      if constexpr (!P::SUM_ROW) lsum += sv[r];            // this lane's 16 tokens; halves combined at the end
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

    __builtin_amdgcn_s_waitcnt(kVmcntZero);                // this wave's transfers have landed
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
  // softmax sum of query n: from the ones row (lanes 0-31 hold it), else the two halves' partial sums
  if constexpr (P::SUM_ROW) {
    const float part = oacc[DH / 32][P::SUM_REG];
    const float other = __shfl_xor(part, 32);
    lsum = half ? other : part;
  } else {
    lsum += __shfl_xor(lsum, 32);
  }
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
  // log-sum-exp of this row: ln(2^m * lsum), m the running max in log2 units
  if (p.lse && half == 0) p.lse[(size_t(b) * L + q0 + n) * H + h] = (m + __builtin_amdgcn_logf(lsum)) * 0.6931471805599453f;
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
  kp.n_hgroups = (a.heads + kPfWaves - 1) / kPfWaves;
  kp.batch = a.batch;
  kp.scale_log2 = a.scale_log2;
  kp.kv_stride = a.kv_stride;
  kp.start = a.start;
  kp.max_start = a.max_start;
  kp.lse = a.lse;
  const long long blocks = (long long)kp.n_qblocks * kp.n_hgroups * a.batch;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid{static_cast<unsigned>(blocks)};
  const size_t lds = size_t(P::LDS);
  const hipError_t attr = allow_dynamic_lds<&prefill_kernel<DH, R>>(int(lds));
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

hipError_t prefill_prepare() {
  hipError_t e = hipSuccess;
#define LRKV_PF(DHV, RV) \
  if (e == hipSuccess) e = allow_dynamic_lds<&prefill_kernel<DHV, RV>>(PrefillShape<DHV, RV>::LDS);
  LRKV_PF(64, 0) LRKV_PF(64, 8) LRKV_PF(64, 16) LRKV_PF(64, 32)
  LRKV_PF(128, 0) LRKV_PF(128, 8) LRKV_PF(128, 16) LRKV_PF(128, 32)
#undef LRKV_PF
  return e;
}

}  // namespace lrkv
