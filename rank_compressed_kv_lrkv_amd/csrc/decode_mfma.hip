// LRKV decode over the compressed cache with the shared term on bf16 MFMA.
//
// Method (Low-Rank Key Value Attention, slide discussion of arXiv:2601.11471v3):
//   logits  s_t = ( q_h.k_{s,t} + (B^K_h^T q_h).z^K_{t,h} ) / sqrt(d_h)     slide
//           "Compute logits without expanding historical keys", Eq. (6);
//   output  o_h = sum_t a_t v_{s,t} + B^V_h ( sum_t a_t z^V_{t,h} )           slide
//           "Aggregate values before the residual up-projection", Eq. (7).
//
// The shared term is a dense contraction across the heads that share one key
// and value row per token: for 32 heads h and 32 cached tokens t,
//   S^T[t][h] = K_s[t][:] . Q[h][:]            (32 x d_h by d_h x 32)
//   O_s^T[d][h] += V_s[t][d]^T . P^T[t][h]     (d_h x 32 by 32 x 32)
// and runs on v_mfma_f32_32x32x16_bf16.  The latent terms are per-head dot
// products (a different z per head), not a contraction, and stay on the
// vector ALUs: q~_h.z^K_{t,h} with q~_h = B^K_h^T q_h (2-wide bf16 dots along
// the rank), and sum_t p_t z^V_{t,h} (2-wide dots over token pairs).  Per-head
// keys and values are never formed, and B^V_h is applied once per head after
// the split-K merge.
//
// Work decomposition.  A workgroup is 4 wave64 over one sequence, one group
// of 32 heads and one split of the context; the split's 32-token tiles are
// dealt to the four waves round-robin, and at the end the four waves' states are
// folded in LDS into the workgroup's partial state (m, l, sum p v_s,
// sum p z^V) for the split-K merge.  Lane l owns head l%32 of the group and,
// in every tile, the 16 tokens 8(i/4) + 4(l/32) + i%4 (i = 0..15) of the
// MFMA accumulator layout.
//
// Data movement.  Per token the wave reads the shared key row, the shared
// value row and the 32 heads' key and value latents, each exactly once, and
// every load instruction reads whole contiguous runs of the cache:
//   - key and value rows are copied global -> LDS (buffer loads into LDS,
//     one tile ahead, swizzled so that the operand reads are free of bank
//     conflicts); the key operand is read back row-wise, the value operand
//     with LDS transpose reads;
//   - latents stream to registers through a ring of D groups of rows,
//     issued D groups ahead of use in the order (key latents of tile t,
//     value latents of tile t, key latents of tile t+1, ...).  For each
//     accumulator row the two lane halves load the two halves of the same
//     token's latent rows (so one instruction covers a contiguous run of all
//     heads), and a cross-half swap (v_permlane32_swap) puts the partial
//     dots, and the softmax weights, where they are needed;
//   - all cache loads carry the non-temporal (streaming) cache policy.
// All global loads go through buffer resources that end at the wave's last
// token, so loads past it return zero (those logits are masked); the tile
// transfers clamp their rows to the last token instead.
//
// Numerics: fp32 accumulation throughout; the absorbed query is rounded once
// to bf16 for the latent dots, the weights p enter the value MFMA and the
// latent value dots rounded to bf16 (relative error <= 2^-9 each), and the
// running sum l adds the fp32 weights.  Softmax runs in the log2 domain with
// a lazily refreshed running max.
#include "decode_balance.h"
#include "lrkv_device.h"
#include "lrkv_internal.h"

#include <utility>

namespace lrkv {

constexpr int kMfWaves = 4;
constexpr int kMfThreads = 64 * kMfWaves;
constexpr int kMfHeads = 32;      // heads per wave: the N dimension of the MFMA
constexpr int kMfTile = 32;       // cache tokens per tile: the M dimension
constexpr float kMfStale = 8.f;   // running-max refresh threshold (log2 units)

template <int DH, int R>
struct MfShape {
  static constexpr int KC = DH / 16;           // k-chunks of the score MFMA
  static constexpr int VB = DH / 32;           // 32-feature blocks of the value MFMA
  static constexpr int RB = DH * 2;            // bytes per shared row
  static constexpr int CR = RB / 16;           // 16-byte chunks per shared row
  static constexpr int VT = kMfTile * RB;      // bytes of one shared-row tile in LDS
  static constexpr int NT = VT / 1024;         // 1 KB global -> LDS transfers per tile
  static constexpr int ZB = R * 2;             // bytes of one head's latent row
  static constexpr int HB = ZB / 2;            // bytes of half a latent row (one lane's share)
  static constexpr int HW = HB / 4;            // 32-bit words of half a latent row
  static constexpr int LPT = HB >= 16 ? HB / 16 : 1;   // loads per half row
  static constexpr int KG = R <= 16 ? 4 : 2;   // accumulator rows per latent group
  static constexpr int NG = 16 / KG;           // latent groups per tile and side
  static constexpr int GL = KG * 2 * LPT;      // loads per latent group
  static constexpr int D = 4;                  // latent groups in flight
  static constexpr int TILES = kMfWaves * 2 * VT + kMfHeads * (R > 0 ? R : 1) * 4;   // tiles, absorbed query
  static constexpr int FOLD = (kMfWaves * 64 * (16 * VB + (R > 0 ? R / 2 : 0) + 4) + kMfWaves * kMfHeads) * 4;
  static constexpr int LDS = TILES > FOLD ? TILES : FOLD;
  static_assert(DH % 32 == 0 && VT % 1024 == 0, "tiles made of 1 KB transfers");
  static_assert(R % 8 == 0 && R <= 32, "latent rows of whole 16-byte units");
  static_assert((2 * NG) % D == 0, "ring slots repeat every tile");
};

struct MfParams {
  const void* k_s; const void* v_s; const void* z_k; const void* z_v;
  const int32_t* seq_lens;
  const void* q; const void* b_k;
  float scale_log2;
  int heads, partials, max_len, split_tokens;
  int batch, balanced, bal_cap;     // balanced: length-balanced items (grid.x = item), else fixed splits
  int64_t capacity;
  float* ws_ml; float* ws_acc;
  int* ws_meta;
};

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8): wait until at most n (< 64) vector-memory loads are
// outstanding, or until every LDS access has completed.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kLgkmZero = 0xC07F;

// Token (row of the 32-token tile) held in accumulator element i by lane half hf.
__device__ __forceinline__ constexpr int acc_row(int i, int hf) { return 8 * (i / 4) + 4 * hf + (i % 4); }

// v_permlane32_swap with both operands given: returns (x0 with its upper
// half replaced by the lower half of x1, x1 with its lower half replaced by
// the upper half of x0).  For x0 = x1 = x the two results hold, in every
// lane, the lower half's and the upper half's x; for (x0, x1) the sum of the
// results in lane l is x0[l] + x0[l ^ 32] for l < 32 and x1[l ^ 32] + x1[l]
// above (the lower half gets x0 summed over both halves, the upper half x1).
__device__ __forceinline__ void swap_halves(uint32_t& x0, uint32_t& x1) {
  const auto r = __builtin_amdgcn_permlane32_swap(x0, x1, false, false);
  x0 = r[0];
  x1 = r[1];
}
__device__ __forceinline__ float sum_halves(float a, float b) {
  uint32_t x0 = __float_as_uint(a), x1 = __float_as_uint(b);
  swap_halves(x0, x1);
  return __uint_as_float(x0) + __uint_as_float(x1);
}

template <int DH, int R>
__global__ __attribute__((amdgpu_flat_work_group_size(kMfThreads, kMfThreads), amdgpu_waves_per_eu(1)))
void decode_mfma_kernel(MfParams p) {
  using S = MfShape<DH, R>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  float* const s_qt = reinterpret_cast<float*>(smem + kMfWaves * 2 * S::VT);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, hf = lane >> 5;
  const int hg = blockIdx.y;
  const int H = p.heads;
  const int h = hg * kMfHeads + j;

  // This workgroup's work item: a sequence b and its tokens [lo, hi).
  // Every exit below is uniform over the workgroup.
  int b, lo, hi, item;
  if (p.balanced) {
    item = blockIdx.x;
    const BalLens L = bal_load(p.seq_lens, p.batch, p.max_len, lane);
    int u;
    bool valid;
    if (!bal_uniform(L, p.batch, p.bal_cap, item, lane, &u, &b, &lo, &hi, &valid)) {
      u = bal_item_size(L, p.max_len, p.bal_cap, lane);
      valid = u != 0 && bal_item(L, u, item, lane, &b, &lo, &hi);
    }
    if (!valid) return;
    // the first item of each sequence records where its items start, and
    // the item size, for the merge
    if (lo == 0 && tid == 0) {
      p.ws_meta[b] = item;
      p.ws_meta[p.batch] = u;
    }
  } else {
    b = blockIdx.z;
    item = b * p.partials + int(blockIdx.x);
    int len = p.seq_lens[b];
    len = len < 0 ? 0 : (len > p.max_len ? p.max_len : len);
    lo = int(blockIdx.x) * p.split_tokens;
    if (lo >= len) return;
    hi = min(lo + p.split_tokens, len);
  }
  b = __builtin_amdgcn_readfirstlane(b);
  lo = __builtin_amdgcn_readfirstlane(lo);
  hi = __builtin_amdgcn_readfirstlane(hi);
  item = __builtin_amdgcn_readfirstlane(item);
  // The item's 32-token tiles are dealt to the four waves round-robin (wave
  // w takes tiles w, w+4, ...), so that the workgroup streams one contiguous
  // run of the cache.
  const int nwg = hi - lo;                                  // the item's tokens [lo, hi)
  const int ntile_wg = (nwg + kMfTile - 1) / kMfTile;
  const int ntiles = ntile_wg > wave ? (ntile_wg - wave + kMfWaves - 1) / kMfWaves : 0;   // this wave's
  auto gtile = [&](int kt) { return wave + kMfWaves * kt; };   // item tile of this wave's kt-th tile

  // Resources over the item's tokens (the host keeps them below 4 GiB).
  const size_t row0 = size_t(b) * size_t(p.capacity) + size_t(lo);
  const uint32_t ztok = uint32_t(H) * S::ZB;                // latent bytes per token
  const __amdgpu_buffer_rsrc_t kres =
      buffer_resource(static_cast<const unsigned char*>(p.k_s) + row0 * S::RB, uint32_t(nwg) * S::RB);
  const __amdgpu_buffer_rsrc_t vres =
      buffer_resource(static_cast<const unsigned char*>(p.v_s) + row0 * S::RB, uint32_t(nwg) * S::RB);
  const __amdgpu_buffer_rsrc_t zkres =
      buffer_resource(static_cast<const unsigned char*>(p.z_k) + row0 * ztok, uint32_t(nwg) * ztok);
  const __amdgpu_buffer_rsrc_t zvres =
      buffer_resource(static_cast<const unsigned char*>(p.z_v) + row0 * ztok, uint32_t(nwg) * ztok);

  unsigned char* const ktile = smem + wave * 2 * S::VT;    // this wave's key tile
  unsigned char* const vtile = ktile + S::VT;               // and value tile

  // Shared-row tile transfer (tile = item tile index): transfer x carries
  // LDS bytes [1024x, 1024x + 1024) of a tile, lane i the chunk at position
  // pos of row rw, i.e. source chunk pos ^ lds_swz(rw).  Rows at or past the
  // item's last token clamp to it (a partial last tile; a tile past the end,
  // transferred but never read, re-reads that row).
  auto row_dma = [&](__amdgpu_buffer_rsrc_t res, int tile, unsigned char* dst) {
    const int last = nwg - 1 - tile * kMfTile;
    const int base = tile * kMfTile;
#pragma unroll
    for (int x = 0; x < S::NT; ++x) {
      const int q = x * 64 + lane, rw = q / S::CR, pos = q % S::CR;
      const int src = base + min(rw, last);
      dma16<kStream>(res, uint32_t(src * S::RB + ((pos ^ lds_swz(rw, S::CR)) * 16)), 0u, dst + x * 1024);
    }
  };

  // Latent ring.  Ring position pos in [0, 2NG) of a tile is key-latent group
  // pos (pos < NG) or value-latent group pos - NG; group a covers accumulator
  // rows a*KG .. a*KG+KG-1.  For row i the lane loads half hf of head h's
  // latent row of token A = acc_row(i, 0) and of token B = acc_row(i, 1):
  // one load instruction covers both halves of every head of one token, a
  // contiguous run of the cache.  Slot pos % D.
  uint32_t ring[S::D][S::KG][2][S::HW > 0 ? S::HW : 1];
  auto z_load = [&](auto slot_c, int pos, int tile) {
    constexpr int slot = decltype(slot_c)::value;
    if constexpr (R > 0) {
      const __amdgpu_buffer_rsrc_t res = pos < S::NG ? zkres : zvres;
      const int a = pos % S::NG;
      const uint32_t lane_off = uint32_t(h) * S::ZB + uint32_t(hf) * S::HB;
#pragma unroll
      for (int t = 0; t < S::KG; ++t) {
        const int i = a * S::KG + t;
#pragma unroll
        for (int sd = 0; sd < 2; ++sd) {
          const uint32_t tok = uint32_t(tile) * kMfTile + uint32_t(acc_row(i, sd));
          // r = 32: a half row is two 16-byte loads, and each load instruction
          // covers every other 16 bytes of its 2 KB; with the cached policy the
          // second half of each line is then served by the L1, where the
          // streaming policy fetched it again
          buffer_words<S::HB, (R == 32 ? kCached : kStream)>(ring[slot][t][sd], res, tok * ztok + lane_off, 0u);
        }
      }
    }
  };

  // ---- prologue.  Loads are issued in three ordered batches so that waiting
  // for an earlier batch never drains a later one: (1) the query operand and
  // the inputs of the absorbed query; (2) the first transfers (key tile 0,
  // value tile 0, latent groups 0..D-1), unconditional like every load here
  // (a wave without tiles reads zeros, or the item's last row); (3) the
  // absorbed query q~_h = B^K_h^T q_h for the group's 32 heads (Eq. (6)),
  // 8 lanes per head, formed while (2) is in flight and shared through LDS. ----
  bf16x8_t qop[S::KC];                                       // B operand: q_h dims 16c + 8hf .. +7
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + (size_t(b) * H + h) * DH + 8 * hf;
#pragma unroll
    for (int c = 0; c < S::KC; ++c) qop[c] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 16 * c));
  }
  // Absorbed-query inputs, 8 lanes per head (hq = tid / 8, g = tid % 8).
  // B^K_h is DH rows of CPR 16-byte chunks (4 KB at DH = 128, R = 16); load k
  // of lane g takes chunk 8k + g, so the 8 lanes of a head read 128
  // contiguous bytes per instruction (one cache line, 8 lines per wave
  // instruction).  Chunk 8k + g holds B^K_h[d][i0 .. i0 + 7] with
  // d = (8k + g) / CPR and i0 = 8 ((8k + g) % CPR) = 8 (g % CPR).  The
  // lane also holds the whole row q_h (QW chunks, the same addresses for the
  // 8 lanes of a head) and picks q_h[d] out of chunk k / CPR.
  constexpr int CPR = R >= 8 ? R / 8 : 1;                   // 16-byte chunks per row of B^K_h
  constexpr int NBK = R > 0 ? DH * CPR / 8 : 1;             // B^K chunks per lane
  constexpr int QW = DH / 8;                                 // 16-byte chunks of a query row
  const int hq = tid / 8, g = tid % 8;
  u32x4 qrow[R > 0 ? QW : 1];
  u32x4 bkv[NBK];
  if constexpr (R > 0) {
    const u32x4* qsl = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.q) +
                                                        (size_t(b) * H + hg * kMfHeads + hq) * DH);
    const u32x4* bk = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.b_k) +
                                                       size_t(hg * kMfHeads + hq) * DH * R);
#pragma unroll
    for (int c = 0; c < QW; ++c) qrow[c] = qsl[c];
#pragma unroll
    for (int k = 0; k < NBK; ++k) bkv[k] = bk[8 * k + g];
  }
  __builtin_amdgcn_sched_barrier(0);
  row_dma(kres, gtile(0), ktile);
  row_dma(vres, gtile(0), vtile);
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (z_load(std::integral_constant<int, I>{}, I, gtile(0)), ...);
  }(std::make_integer_sequence<int, S::D>{});
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (R > 0) {
    // part[e] = sum over this lane's d of q_h[d] B^K_h[d][i0 + e]; q_h[d] is
    // element ek + gq of chunk k / CPR, with ek = 8 (k % CPR) / CPR from the
    // load index and gq = g / CPR from the lane (selected, not indexed);
    // NBK is even (DH >= 64), so loads pair up for dot2
    const int gq = g / CPR;
    float part[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) part[e] = 0.f;
    auto q_bits = [&](int k) -> uint32_t {                   // bf16 bits of q_h[d] for load k
      const u32x4 qc = qrow[k / CPR];
      const int el = 8 * (k % CPR) / CPR + gq;               // element of the chunk, 0..7
      const uint32_t w01 = (el & 2) ? qc.y : qc.x, w23 = (el & 2) ? qc.w : qc.z;
      const uint32_t w = (el & 4) ? w23 : w01;
      return (el & 1) ? (w >> 16) : (w & 0xffffu);
    };
    // loads k and k + 1 in one bf16 dot2 per output: (q[d_k], q[d_k+1]) . (B_k[e], B_k+1[e])
#pragma unroll
    for (int k = 0; k < NBK; k += 2) {
      const uint32_t qp = q_bits(k) | (q_bits(k + 1) << 16);
      const uint32_t b0[4] = {bkv[k].x, bkv[k].y, bkv[k].z, bkv[k].w};
      const uint32_t b1[4] = {bkv[k + 1].x, bkv[k + 1].y, bkv[k + 1].z, bkv[k + 1].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t bp = __builtin_amdgcn_perm(b1[e / 2], b0[e / 2], (e & 1) ? 0x07060302u : 0x05040100u);
        part[e] = BF16::dot2(part[e], qp, bp);
      }
    }
    // sum over the lanes of the head with the same g % CPR (xor of the bits above CPR)
    auto xor_add = [&]<int M>(std::integral_constant<int, M>) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        part[e] += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(part[e]), 0x1F | (M << 10)));
    };
    if constexpr (CPR <= 1) xor_add(std::integral_constant<int, 1>{});
    if constexpr (CPR <= 2) xor_add(std::integral_constant<int, 2>{});
    if constexpr (CPR <= 4) xor_add(std::integral_constant<int, 4>{});
    if (gq == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_qt[hq * R + 8 * (g % CPR) + e] = part[e];
    }
  }
  __syncthreads();
  uint32_t qh[S::HW > 0 ? S::HW : 1];                      // half hf of q~_h as bf16 pairs
  if constexpr (R > 0) {
#pragma unroll
    for (int w = 0; w < S::HW; ++w)
      qh[w] = pack_bf16x2(s_qt[j * R + hf * (R / 2) + 2 * w], s_qt[j * R + hf * (R / 2) + 2 * w + 1]);
  }

  // LDS offsets (loop-invariant).  Key operand: lane (token row j, half hf)
  // reads chunk 2c + hf of row j.  Value operand (as in the prefill kernel):
  // transpose reads where this lane addresses token 4*hf + (lane bits 2-3) at
  // features 16*(lane bit 4) + 4*(lane bits 0-1) of each 32-feature block
  // (first read) and token + 8 (second read); rows +16 share the swizzle.
  int koff[S::KC];
#pragma unroll
  for (int c = 0; c < S::KC; ++c) koff[c] = j * S::RB + ((2 * c + hf) ^ lds_swz(j, S::CR)) * 16;
  const int tr_tok = 4 * hf + ((lane >> 2) & 3);
  int voff[S::VB][2];
#pragma unroll
  for (int f = 0; f < S::VB; ++f) {
    const int ch = 4 * f + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int row = tr_tok + 8 * x;
      voff[f][x] = row * S::RB + (ch ^ lds_swz(row, S::CR)) * 16 + 8 * (lane & 1);
    }
  }

  f32x16_t oacc[S::VB];
#pragma unroll
  for (int f = 0; f < S::VB; ++f) oacc[f] = f32x16_t{};
  float acc_z[R > 0 ? R / 2 : 1];                           // dims hf*R/2 .. of sum_t p_t z^V_{t,h}
#pragma unroll
  for (int i = 0; i < (R > 0 ? R / 2 : 1); ++i) acc_z[i] = 0.f;
  float m = -INFINITY, lsum = 0.f;

  // Issue order (every load unconditional; loads past the wave's last token
  // return zero, the tile transfers clamp): step kt issues K(kt+1) after its
  // key reads, latent groups D..D+NG-1 of the ring, V(kt+1) after its value
  // reads, then NG more latent groups.  Scheduling barriers keep that order,
  // and ring registers are overwritten only after their last use.  The key
  // and value reads wait for their transfers with explicit counts of the
  // loads issued after them (in the first step: after the prologue's).
  constexpr int NK = S::NT, NV = S::NT;
  constexpr int kKAfter = NV + (S::D < 2 * S::NG ? S::D : 2 * S::NG) * S::GL;
  constexpr int kVAfter = NK + (S::D + S::NG < 2 * S::NG ? S::D + S::NG : 2 * S::NG) * S::GL;
  constexpr int kKWait = kKAfter < 63 ? kKAfter : 63;
  constexpr int kVWait = kVAfter < 63 ? kVAfter : 63;
  for (int kt = 0; kt < ntiles; ++kt) {
    // -- shared scores S^T = K_s . Q^T; then the key tile is refilled --
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kKWait));             // K(kt) has landed in LDS
    f32x16_t s = {};
    {
      u32x4 ka[S::KC];
#pragma unroll
      for (int c = 0; c < S::KC; ++c) ka[c] = *reinterpret_cast<const u32x4*>(ktile + koff[c]);
#pragma unroll
      for (int c = 0; c < S::KC; ++c) s = mfma32(as_bf16x8(ka[c]), qop[c], s);
    }
    __builtin_amdgcn_s_waitcnt(kLgkmZero);                    // key reads done before the refill
    __builtin_amdgcn_sched_barrier(0);
    row_dma(kres, gtile(kt + 1), ktile);
    __builtin_amdgcn_sched_barrier(0);

    // -- latent scores: s += q~_h . z^K_{t,h}; ring positions 0..NG-1.  Each
    //    lane dots its half of q~_h with half rows of tokens A and B; one
    //    swap gives each lane its own token's full dot. --
    if constexpr (R > 0) {
      [&]<int... A>(std::integer_sequence<int, A...>) {
        ([&] {
          constexpr int a = A, slot = a % S::D;
#pragma unroll
          for (int t = 0; t < S::KG; ++t) {
            float pa = 0.f, pb = 0.f;
#pragma unroll
            for (int w = 0; w < S::HW; ++w) {
              pa = BF16::dot2(pa, qh[w], ring[slot][t][0][w]);
              pb = BF16::dot2(pb, qh[w], ring[slot][t][1][w]);
            }
            s[a * S::KG + t] += sum_halves(pa, pb);
          }
          __builtin_amdgcn_sched_barrier(0);
          z_load(std::integral_constant<int, slot>{}, a + S::D, gtile(kt));   // a + D < 2NG: same tile
          __builtin_amdgcn_sched_barrier(0);
        }(), ...);
      }(std::make_integer_sequence<int, S::NG>{});
    }

    // -- online softmax (log2 domain).  Only a partial last tile is masked.
    //    Lanes l and l^32 hold the same head and must share m, so the refresh
    //    is decided for the whole wave; the common case exchanges nothing. --
    if ((gtile(kt) + 1) * kMfTile > nwg) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (gtile(kt) * kMfTile + acc_row(i, hf) >= nwg) s[i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
    if (__builtin_amdgcn_ballot_w64(mx * p.scale_log2 > m + kMfStale)) {
      uint32_t x0 = __float_as_uint(mx), x1 = x0;
      swap_halves(x0, x1);                                    // this head's maxima of both halves
      const float mn = fmaxf(m, fmaxf(__uint_as_float(x0), __uint_as_float(x1)) * p.scale_log2);
      const float alpha = fast_exp2(m - mn);                  // 0 on the first tile (m = -inf)
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int f = 0; f < S::VB; ++f) oacc[f] *= alpha;
#pragma unroll
      for (int i = 0; i < (R > 0 ? R / 2 : 1); ++i) acc_z[i] *= alpha;
    }
    float pv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      pv[i] = fast_exp2(__builtin_fmaf(s[i], p.scale_log2, -m));   // masked rows: exp2(-inf) = 0
      lsum += pv[i];
    }
    uint32_t pw[8];                                           // bf16 pairs (p_{2w}, p_{2w+1})
#pragma unroll
    for (int w = 0; w < 8; ++w) pw[w] = pack_bf16x2(pv[2 * w], pv[2 * w + 1]);

    // -- shared values O_s^T += V_s^T . P^T; then the value tile is refilled --
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kVWait));             // V(kt) has landed in LDS
#pragma unroll
    for (int f = 0; f < S::VB; ++f) {
      u32x4 va[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint2 lo = lds_read_tr16(vtile + 16 * c * S::RB + voff[f][0]);
        const uint2 hi = lds_read_tr16(vtile + 16 * c * S::RB + voff[f][1]);
        va[c] = u32x4{lo.x, lo.y, hi.x, hi.y};
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
        oacc[f] = mfma32(as_bf16x8(va[c]), as_bf16x8(u32x4{pw[4 * c], pw[4 * c + 1], pw[4 * c + 2], pw[4 * c + 3]}),
                         oacc[f]);
    }
    __builtin_amdgcn_s_waitcnt(kLgkmZero);                    // value reads done before the refill
    __builtin_amdgcn_sched_barrier(0);
    row_dma(vres, gtile(kt + 1), vtile);
    __builtin_amdgcn_sched_barrier(0);

    // -- latent values: acc_z += sum_t p_t z^V_{t,h} over all 32 tokens of the
    //    tile; ring positions NG..2NG-1.  One swap gives every lane the
    //    weights of tokens A (lower half's) and B (upper half's). --
    if constexpr (R > 0) {
      uint32_t pa_w[8], pb_w[8];
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        pa_w[w] = pw[w];
        pb_w[w] = pw[w];
        swap_halves(pa_w[w], pb_w[w]);
      }
      [&]<int... A>(std::integer_sequence<int, A...>) {
        ([&] {
          constexpr int a = A, pos = S::NG + a, slot = pos % S::D;
#pragma unroll
          for (int t = 0; t < S::KG; t += 2) {
            const int i = a * S::KG + t;                      // rows i, i+1: consecutive tokens
#pragma unroll
            for (int sd = 0; sd < 2; ++sd) {
              const uint32_t pp = sd == 0 ? pa_w[i / 2] : pb_w[i / 2];
#pragma unroll
              for (int w = 0; w < S::HW; ++w) {
                const uint32_t z0 = ring[slot][t][sd][w], z1 = ring[slot][t + 1][sd][w];
                acc_z[2 * w] = BF16::dot2(acc_z[2 * w], pp, __builtin_amdgcn_perm(z1, z0, 0x05040100u));
                acc_z[2 * w + 1] = BF16::dot2(acc_z[2 * w + 1], pp, __builtin_amdgcn_perm(z1, z0, 0x07060302u));
              }
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          constexpr int nxt = pos + S::D;                      // next position for this slot
          if constexpr (nxt < 2 * S::NG) {
            z_load(std::integral_constant<int, slot>{}, nxt, gtile(kt));
          } else {
            z_load(std::integral_constant<int, slot>{}, nxt - 2 * S::NG, gtile(kt + 1));
          }
          __builtin_amdgcn_sched_barrier(0);
        }(), ...);
      }(std::make_integer_sequence<int, S::NG>{});
    }
  }

  // ---- fold the four waves' states into the workgroup's partial state:
  //      with M the largest of their running maxima, each wave's sums are
  //      scaled by 2^(m - M) and added (Eq. (7) is linear in the weights).
  //      The tile memory is reused once every transfer into it has landed. ----
  constexpr int P = 16 * S::VB + (R > 0 ? R / 2 : 0) + 4;   // floats per lane (stride conflict-free for 16-byte access)
  float* const s_red = reinterpret_cast<float*>(smem);      // [wave][lane][P]
  float* const s_m = s_red + kMfWaves * 64 * P;             // [wave][head]
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  if (hf == 0) s_m[wave * kMfHeads + j] = m;
  __syncthreads();
  float M = s_m[j];
#pragma unroll
  for (int w = 1; w < kMfWaves; ++w) M = fmaxf(M, s_m[w * kMfHeads + j]);   // finite: wave 0 has tokens
  const float sc = m == -INFINITY ? 0.f : fast_exp2(m - M);
  {
    float* dst = s_red + (wave * 64 + lane) * P;
#pragma unroll
    for (int f = 0; f < S::VB; ++f)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<float4*>(dst + 16 * f + 4 * r4) = make_float4(
            oacc[f][4 * r4] * sc, oacc[f][4 * r4 + 1] * sc, oacc[f][4 * r4 + 2] * sc, oacc[f][4 * r4 + 3] * sc);
    if constexpr (R > 0) {
#pragma unroll
      for (int i = 0; i < R / 2; i += 4)
        *reinterpret_cast<float4*>(dst + 16 * S::VB + i) =
            make_float4(acc_z[i] * sc, acc_z[i + 1] * sc, acc_z[i + 2] * sc, acc_z[i + 3] * sc);
    }
    dst[P - 4] = lsum * sc;
  }
  __syncthreads();
  // Block x of the state (value block f = x for x < VB; the latent sums and
  // the softmax sum for x = VB) is added up over the waves and written by
  // wave x % 4, so the four waves share the final reads and stores.
  const size_t pidx = size_t(item) * H + h;
  float* const out_acc = p.ws_acc + pidx * (DH + R);
  const float* const src0 = s_red + lane * P;               // this lane's slot of wave 0
#pragma unroll
  for (int f = 0; f < S::VB; ++f) {
    if (f % kMfWaves != wave) continue;                     // uniform
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float4 a = *reinterpret_cast<const float4*>(src0 + 16 * f + 4 * r4);
#pragma unroll
      for (int w = 1; w < kMfWaves; ++w) {
        const float4 v = *reinterpret_cast<const float4*>(src0 + w * 64 * P + 16 * f + 4 * r4);
        a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
      }
      *reinterpret_cast<float4*>(out_acc + 32 * f + 8 * r4 + 4 * hf) = a;
    }
  }
  if (S::VB % kMfWaves == wave) {
    if constexpr (R > 0) {
#pragma unroll
      for (int i = 0; i < R / 2; i += 4) {
        float4 a = *reinterpret_cast<const float4*>(src0 + 16 * S::VB + i);
#pragma unroll
        for (int w = 1; w < kMfWaves; ++w) {
          const float4 v = *reinterpret_cast<const float4*>(src0 + w * 64 * P + 16 * S::VB + i);
          a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
        }
        *reinterpret_cast<float4*>(out_acc + DH + hf * (R / 2) + i) = a;
      }
    }
    float ls = src0[P - 4];
#pragma unroll
    for (int w = 1; w < kMfWaves; ++w) ls += src0[w * 64 * P + P - 4];
    uint32_t x0 = __float_as_uint(ls), x1 = x0;
    swap_halves(x0, x1);                                     // the two halves' sums of this head
    ls = __uint_as_float(x0) + __uint_as_float(x1);
    if (hf == 0) *reinterpret_cast<float2*>(p.ws_ml + 2 * pidx) = make_float2(M, ls);
  }
}

template <int DH, int R>
static hipError_t launch_mfma_t(const DecodePlan& pl, const DecodeArgs& a, hipStream_t st) {
  using S = MfShape<DH, R>;
  MfParams kp;
  kp.k_s = a.k_s; kp.v_s = a.v_s; kp.z_k = a.z_k; kp.z_v = a.z_v;
  kp.seq_lens = a.seq_lens; kp.q = a.q; kp.b_k = a.b_k;
  kp.scale_log2 = a.scale_log2;
  kp.heads = pl.heads; kp.partials = pl.partials;
  kp.max_len = pl.max_len; kp.split_tokens = pl.split_tokens;
  kp.batch = pl.batch; kp.balanced = pl.balanced; kp.bal_cap = pl.bal_cap;
  kp.capacity = pl.capacity;
  kp.ws_ml = a.ws_ml; kp.ws_acc = a.ws_acc; kp.ws_meta = a.ws_meta;
  const hipError_t attr = allow_dynamic_lds<&decode_mfma_kernel<DH, R>>(S::LDS);
  if (attr != hipSuccess) return attr;
  const dim3 grid(pl.n_splits, pl.heads / kMfHeads, pl.balanced ? 1 : pl.batch);
  hipLaunchKernelGGL((decode_mfma_kernel<DH, R>), grid, dim3(kMfThreads), size_t(S::LDS), st, kp);
  return hipGetLastError();
}

bool decode_mfma_supported(int dtype, int head_dim, int rank, int heads) {
  return dtype == 1 && (head_dim == 64 || head_dim == 128) &&
         (rank == 0 || rank == 8 || rank == 16 || rank == 32) && heads >= kMfHeads && heads % kMfHeads == 0 &&
         heads <= 64;
}

hipError_t launch_decode_mfma_scan(const DecodePlan& pl, const DecodeArgs& a, hipStream_t st) {
  if (pl.n_splits == 0) return hipSuccess;
#define LRKV_MF(DHV, RV) \
  if (pl.head_dim == DHV && pl.rank == RV) return launch_mfma_t<DHV, RV>(pl, a, st);
  LRKV_MF(64, 0) LRKV_MF(64, 8) LRKV_MF(64, 16) LRKV_MF(64, 32)
  LRKV_MF(128, 0) LRKV_MF(128, 8) LRKV_MF(128, 16) LRKV_MF(128, 32)
#undef LRKV_MF
  return hipErrorInvalidValue;
}

hipError_t decode_mfma_prepare() {
  hipError_t e = hipSuccess;
#define LRKV_MF(DHV, RV) \
  if (e == hipSuccess) e = allow_dynamic_lds<&decode_mfma_kernel<DHV, RV>>(MfShape<DHV, RV>::LDS);
  LRKV_MF(64, 0) LRKV_MF(64, 8) LRKV_MF(64, 16) LRKV_MF(64, 32)
  LRKV_MF(128, 0) LRKV_MF(128, 8) LRKV_MF(128, 16) LRKV_MF(128, 32)
#undef LRKV_MF
  return e;
}

}  // namespace lrkv
