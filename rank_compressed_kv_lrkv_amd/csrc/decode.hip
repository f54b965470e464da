// LRKV decode over the compressed cache: split-K scan + log-sum-exp merge.
//
// Method (Low-Rank Key Value Attention, slide discussion of arXiv:2601.11471v3):
//   logits  s_t = ( q_h.k_{s,t} + (B^K_h^T q_h).z^K_{t,h} ) / sqrt(d_h)     slide
//           "Compute logits without expanding historical keys", Eq. (6);
//   output  o_h = sum_t a_t v_{s,t} + B^V_h ( sum_t a_t z^V_{t,h} )           slide
//           "Aggregate values before the residual up-projection", Eq. (7).
// Per-head keys and values are never formed.  The shared rows k_s/v_s of a
// token are staged once in LDS and serve all H heads of the workgroup; the
// per-head latents stream from HBM straight into the lanes that own the head.
//
// Work decomposition (one workgroup = 256 lanes = 4 wave64):
//   grid.x = split index (a run of split_tokens tokens), grid.y = sequence.
//   Lane -> (slot, head h, g) with g in [0, G).  The G lanes of a head form an
//   aligned group inside one wave.  Tokens are processed in batches of G: in a
//   batch, lane g scores token g of the batch (the full d_h + r dot product,
//   no cross-lane reduction), then every lane of the group folds all G tokens
//   into its slice of the accumulators (d_h/G shared dims, r/G latent dims).
//   When H*G < 256 the workgroup runs several independent token streams
//   ("slots"), each producing its own partial state.
// Numerics: bf16 products accumulate in fp32 via v_dot2_f32_bf16; the
// absorbed query B^K_h^T q_h is formed in fp32 and rounded once to bf16 for
// the dot products with the bf16 latents (relative error <= 2^-9 per
// element, the same as the stored q, k and z themselves); softmax runs in
// the log2 domain with running max m and sum l (fp32 weights); the weights
// enter the value sums rounded to bf16 (relative error <= 2^-9 each,
// unbiased).  fp32 storage runs all-fp32 FMAs.
//
// Addressing.  Every global load goes through a buffer resource that starts
// at the split's first token: a lane adds its fixed byte offset to a uniform
// offset that advances per tile or per batch, so the loop does no 64-bit
// address arithmetic.
#include "lrkv_device.h"
#include "lrkv_internal.h"

#include <utility>

namespace lrkv {

template <class E, int DH, int R, int G>
struct DecodeShape {
  using T = typename E::T;
  using Pair = typename E::Pair;
  static constexpr int ES = E::kBytes;
  static constexpr int PB = 2 * ES;                    // bytes per pair
  static constexpr int ROW_BYTES = DH * ES;            // one k_s / v_s row
  static constexpr int ROW_CH = ROW_BYTES / 16;        // 16-byte chunks per row
  static constexpr int KS_STRIDE = ROW_BYTES + 16;     // padded LDS row (bank spread)
  static constexpr int VP_STRIDE = DH * PB;            // two tokens interleaved per LDS row
  static constexpr int DPL = DH / G;                   // head dims owned per lane
  static constexpr int SLICE_BYTES = DPL * ES;         // a lane's slice of a k_s row
  static constexpr int VSLICE_BYTES = DPL * PB;        // a lane's slice of an interleaved v row
  static constexpr int CPS = VSLICE_BYTES / 16;        // 16-byte chunks per v slice (0 if < 16 B)
  static constexpr int RPL = R / G;                    // latent-value dims per lane
  static constexpr int RP = R / 2;                     // latent pairs
  static constexpr int ZK_BYTES = R * ES;              // one head's key latent row
  static constexpr int ZV_BYTES = RPL * ES;            // one lane's slice of a value latent row
  static constexpr int NBT = kDecodeTile / G;          // batches per tile
  static constexpr int KV_CH = kDecodeTile * ROW_CH;   // 16-byte chunks of one K (or V) tile
  static constexpr int K_PER_LANE = (KV_CH + kDecodeThreads - 1) / kDecodeThreads;
  static constexpr int VPAIR_ITEMS = (kDecodeTile / 2) * ROW_CH;  // (pair row, chunk) items
  static constexpr int V_PER_LANE = (VPAIR_ITEMS + kDecodeThreads - 1) / kDecodeThreads;
  static_assert(DH % G == 0 && (R == 0 || R % G == 0), "dims per lane");
  static_assert(ROW_BYTES % 16 == 0 && ZK_BYTES % 16 == 0, "16-byte rows");
  static_assert(G % 2 == 0 && DPL % 2 == 0, "pairs");
  // Physical 16-byte chunk of logical chunk L of an interleaved v row: the
  // chunks of each lane's slice are rotated so that the G lanes of a group,
  // reading chunk c of their slices together, hit distinct LDS banks.
  __device__ static __forceinline__ int vchunk(int L) {
    if constexpr (CPS >= 2) {
      const int j = L / CPS;
      const int rot = ((j * CPS) / 8) & (CPS - 1);
      return (L & ~(CPS - 1)) | (((L & (CPS - 1)) + rot) & (CPS - 1));
    } else {
      return L;
    }
  }
};

// Batches of latents in flight ahead of the one being computed.
constexpr int kZDepth = 1;
// The running max is refreshed only when a logit exceeds it by more than
// this (log2 units): weights stay <= 2^kDecStale, and the sum, the value
// sums and the merge all use the same reference, so the result is unchanged.
constexpr float kDecStale = 8.f;

struct DecodeKernelParams {
  const void* k_s; const void* v_s; const void* z_k; const void* z_v;
  const int32_t* seq_lens;
  const void* q; const void* b_k;
  float scale_log2;
  int heads, heads_pow2, slots, partials;
  int64_t capacity;
  int max_len, split_tokens;
  float* ws_ml; float* ws_acc;
};

// One tile of shared rows in registers: 64 K rows, and V rows taken two at a
// time so they can be interleaved token-wise.  Rows at or beyond `nvalid`
// are zero (never read from memory).
template <class S>
struct TileRegs {
  u32x4 k[S::K_PER_LANE];
  u32x4 va[S::V_PER_LANE];
  u32x4 vb[S::V_PER_LANE];
};

// Stage the 64-token tile starting `rel` tokens after the split's first
// token into registers (kres/vres start at that token).  Rows past the
// split's last token (`lim` rows after the tile start) re-read that token's
// row (valid, finite data whose logit is masked and whose weight is zero),
// so every load is unconditional.
template <class S>
__device__ __forceinline__ void tile_load(TileRegs<S>& tr, __amdgpu_buffer_rsrc_t kres, __amdgpu_buffer_rsrc_t vres,
                                          int rel, int lim, int tid) {
  const uint32_t soff = uint32_t(rel) * S::ROW_BYTES;
#pragma unroll
  for (int i = 0; i < S::K_PER_LANE; ++i) {
    const int c = tid + i * kDecodeThreads;
    if (c < S::KV_CH) {
      const int row = min(c / S::ROW_CH, lim), ch = c % S::ROW_CH;
      tr.k[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              kres, row * S::ROW_BYTES + ch * 16, int(soff), kStream));
    }
  }
#pragma unroll
  for (int i = 0; i < S::V_PER_LANE; ++i) {
    const int it = tid + i * kDecodeThreads;
    if (it < S::VPAIR_ITEMS) {
      const int pr = it / S::ROW_CH, ch = it % S::ROW_CH;
      const int r0 = min(2 * pr, lim), r1 = min(2 * pr + 1, lim);
      tr.va[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               vres, r0 * S::ROW_BYTES + ch * 16, int(soff), kStream));
      tr.vb[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               vres, r1 * S::ROW_BYTES + ch * 16, int(soff), kStream));
    }
  }
}

// Interleave two 16-byte row chunks element-wise into 32 bytes of pairs.
template <class E>
__device__ __forceinline__ void zip16(const u32x4& a, const u32x4& b, u32x4& o0, u32x4& o1) {
  if constexpr (E::kBytes == 2) {
    auto lo = [](uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x05040100u); };  // (x.lo, y.lo)
    auto hi = [](uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x07060302u); };  // (x.hi, y.hi)
    o0 = u32x4{lo(a.x, b.x), hi(a.x, b.x), lo(a.y, b.y), hi(a.y, b.y)};
    o1 = u32x4{lo(a.z, b.z), hi(a.z, b.z), lo(a.w, b.w), hi(a.w, b.w)};
  } else {
    o0 = u32x4{a.x, b.x, a.y, b.y};
    o1 = u32x4{a.z, b.z, a.w, b.w};
  }
}

template <class S, class E>
__device__ __forceinline__ void tile_store(const TileRegs<S>& tr, unsigned char* ks, unsigned char* vp, int tid) {
#pragma unroll
  for (int i = 0; i < S::K_PER_LANE; ++i) {
    const int c = tid + i * kDecodeThreads;
    if (c < S::KV_CH) {
      const int row = c / S::ROW_CH, ch = c % S::ROW_CH;
      *reinterpret_cast<u32x4*>(ks + row * S::KS_STRIDE + ch * 16) = tr.k[i];
    }
  }
#pragma unroll
  for (int i = 0; i < S::V_PER_LANE; ++i) {
    const int it = tid + i * kDecodeThreads;
    if (it < S::VPAIR_ITEMS) {
      const int pr = it / S::ROW_CH, ch = it % S::ROW_CH;
      u32x4 o0, o1;
      zip16<E>(tr.va[i], tr.vb[i], o0, o1);
      unsigned char* row = vp + pr * S::VP_STRIDE;
      *reinterpret_cast<u32x4*>(row + S::vchunk(2 * ch) * 16) = o0;
      *reinterpret_cast<u32x4*>(row + S::vchunk(2 * ch + 1) * 16) = o1;
    }
  }
}

// Latents of one batch for one lane: its own token's key latent row (all r
// dims, for the logit) and, for each of the G tokens, its r/G-dim slice of
// that token's value latent row (for the aggregation), as 32-bit words.
template <class S>
struct ZRegs {
  static constexpr int ZKW = S::ZK_BYTES / 4 > 0 ? S::ZK_BYTES / 4 : 1;
  static constexpr int ZVW = S::ZV_BYTES >= 4 ? S::ZV_BYTES / 4 : 1;
  uint32_t zk[ZKW];
  uint32_t zv[8][ZVW];   // [token of the batch][words]  (G <= 8)
};

// Load the latents of the batch of tokens [tb, tb+G), tb = tb0 + slot*G,
// through resources that start at the split's first token t0 (rel0 = tb0 -
// t0 is uniform).  A full batch (all G tokens before the split end) adds the
// uniform offset to the lane's fixed offsets (zk_lane: token g of the batch,
// head h; zv_lane: head h, slice g; both include the slot's first token); the
// split's last, partial batch (CLAMP) clamps token indices to the last valid
// token (rel_last), whose data is finite and whose weight is zero there.
template <class S, int G, bool CLAMP>
__device__ __forceinline__ void z_load(ZRegs<S>& zr, __amdgpu_buffer_rsrc_t zkres, __amdgpu_buffer_rsrc_t zvres,
                                       int rel0, int rel_tb, uint32_t zk_lane, uint32_t zv_lane, uint32_t zk_head,
                                       uint32_t zv_head, uint32_t ztok, int rel_last, int g) {
  if constexpr (S::ZK_BYTES > 0) {
    if constexpr (!CLAMP) {
      const uint32_t soff = uint32_t(rel0) * ztok;
      buffer_words<S::ZK_BYTES, kStream>(zr.zk, zkres, zk_lane, soff);
#pragma unroll
      for (int j = 0; j < G; ++j) buffer_words<S::ZV_BYTES, kStream>(zr.zv[j], zvres, zv_lane, soff + uint32_t(j) * ztok);
    } else {
      const int tok = min(rel_tb + g, rel_last);
      buffer_words<S::ZK_BYTES, kStream>(zr.zk, zkres, uint32_t(tok) * ztok + zk_head, 0u);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const int tj = min(rel_tb + j, rel_last);
        buffer_words<S::ZV_BYTES, kStream>(zr.zv[j], zvres, uint32_t(tj) * ztok + zv_head, 0u);
      }
    }
  }
}

// XOR-ordered reduce-scatter of per-lane partial sums within an aligned
// group of G lanes.  On entry part[i] of lane g is the partial sum of item
// (i ^ g) over lane g's slice; on exit part[0] of lane g is the complete sum
// of item g.  Stage masks (G=8: 7, 2, 1; G=4: 3, 1; G=2: 1) keep the register
// index exchanged the same in every lane, so each stage is a DPP add.
template <int G>
__device__ __forceinline__ void xor_reduce_scatter(float* part) {
  if constexpr (G == 8) {
#pragma unroll
    for (int k = 0; k < 4; ++k) part[k] += dpp_mov<kDppHalfMirror>(part[k ^ 7]);
#pragma unroll
    for (int k = 0; k < 2; ++k) part[k] += dpp_mov<kDppSwap2>(part[k ^ 2]);
    part[0] += dpp_mov<kDppSwap1>(part[1]);
  } else if constexpr (G == 4) {
#pragma unroll
    for (int k = 0; k < 2; ++k) part[k] += dpp_mov<kDppRev4>(part[k ^ 3]);
    part[0] += dpp_mov<kDppSwap1>(part[1]);
  } else {
    static_assert(G == 2, "group size");
    part[0] += dpp_mov<kDppSwap1>(part[1]);
  }
}

// Per-lane running state of one (slot, head) and the loop over a split.
//
// Placement.  Rounds n = 0, 1, ... cover tokens [t0 + n*step, t0 + (n+1)*step)
// (step = min(slots*G, 64)); slot s takes the G tokens starting at
// tb = t0 + n*step + s*G (even, so token pairs line up with the interleaved
// value rows).  64-token tiles are staged in LDS at 64-token boundaries.  Rows
// and latents past the split end are clamped to its last token, so no load
// is predicated; those tokens' logits are masked.
template <class E, int DH, int R, int G>
__device__ __forceinline__ void decode_split_body(
    const DecodeKernelParams& p, unsigned char* s_k, unsigned char* s_v, int tid, int b, int split,
    int t0, int t1, int g, int h, int slot, bool active, float& m, float& l, float* acc_s, float* acc_z) {
  using S = DecodeShape<E, DH, R, G>;
  using T = typename S::T;
  using Pair = typename S::Pair;
  const int H = p.heads;
  const uint32_t ztok = uint32_t(H) * S::ZK_BYTES;           // latent bytes per token
  // resources over the split's tokens [t0, t1) (the host keeps them < 4 GiB)
  const size_t row0 = size_t(b) * p.capacity + size_t(t0);
  const uint32_t ntok = uint32_t(t1 - t0);
  const __amdgpu_buffer_rsrc_t kres =
      buffer_resource(static_cast<const unsigned char*>(p.k_s) + row0 * S::ROW_BYTES, ntok * S::ROW_BYTES);
  const __amdgpu_buffer_rsrc_t vres =
      buffer_resource(static_cast<const unsigned char*>(p.v_s) + row0 * S::ROW_BYTES, ntok * S::ROW_BYTES);
  const __amdgpu_buffer_rsrc_t zkres = buffer_resource(static_cast<const unsigned char*>(p.z_k) + row0 * ztok, ntok * ztok);
  const __amdgpu_buffer_rsrc_t zvres = buffer_resource(static_cast<const unsigned char*>(p.z_v) + row0 * ztok, ntok * ztok);

  const int step = min(p.slots * G, kDecodeTile);
  const int nb = (t1 - t0 + step - 1) / step;                 // rounds
  const bool slot_in_round = slot * G < step;
  const int last = t1 - 1;
  const int ntiles = (t1 - t0 + kDecodeTile - 1) / kDecodeTile;
  const uint32_t zk_head = uint32_t(h) * S::ZK_BYTES;
  const uint32_t zv_head = uint32_t(h) * S::ZK_BYTES + uint32_t(g) * S::ZV_BYTES;
  const uint32_t zk_lane = uint32_t(slot * G + g) * ztok + zk_head;
  const uint32_t zv_lane = uint32_t(slot * G) * ztok + zv_head;

  // ---- prologue: this lane's slice of q_h, and the absorbed query B^K_h^T q_h ----
  const int hq = active ? h : 0;
  const T* qrow = static_cast<const T*>(p.q) + (size_t(b) * H + hq) * DH;
  Pair qs[S::DPL / 2];
  {
    uint32_t qw[S::SLICE_BYTES / 4];
    load_words<S::SLICE_BYTES>(qw, qrow + g * S::DPL);
#pragma unroll
    for (int i = 0; i < S::DPL / 2; ++i) qs[i] = pair_at<E>(qw, i);
  }
  Pair qt[S::RP > 0 ? S::RP : 1];
  if constexpr (R > 0) {
    // lane g sums rows d in its slice of B^K_h, then the group adds up.
    float part[R];
#pragma unroll
    for (int i = 0; i < R; ++i) part[i] = 0.f;
    const T* bk = static_cast<const T*>(p.b_k) + size_t(hq) * DH * R;
#pragma unroll
    for (int dd = 0; dd < S::DPL; ++dd) {
      const int d = g * S::DPL + dd;
      const float qd = (dd & 1) ? E::hi(qs[dd / 2]) : E::lo(qs[dd / 2]);
      uint32_t rw[S::ZK_BYTES / 4];
      load_words<S::ZK_BYTES>(rw, bk + size_t(d) * R);
#pragma unroll
      for (int i = 0; i < R; ++i) part[i] = __builtin_fmaf(qd, E::to_f32(elem_at<E>(rw, i)), part[i]);
    }
#pragma unroll
    for (int i = 0; i < S::RP; ++i) {
      const float a = group_sum<G>(part[2 * i]);
      const float c = group_sum<G>(part[2 * i + 1]);
      qt[i] = E::make_pair(a, c);
    }
  }

  TileRegs<S> tr;
  tile_load<S>(tr, kres, vres, 0, last - t0, tid);

  auto fetch = [&](ZRegs<S>& zr, int n) {
    const int tb = t0 + n * step + slot * G;
    if (!(active && slot_in_round && tb < t1)) return;
    if (tb + G <= t1)
      z_load<S, G, false>(zr, zkres, zvres, n * step, tb - t0, zk_lane, zv_lane, zk_head, zv_head, ztok, last - t0, g);
    else
      z_load<S, G, true>(zr, zkres, zvres, n * step, tb - t0, zk_lane, zv_lane, zk_head, zv_head, ztok, last - t0, g);
  };

  // One batch: logits of tokens [tb, tb+G), online softmax, aggregation.
  auto process = [&](const ZRegs<S>& zc, int n) {
    const int off = n * step;
    const int tile = off / kDecodeTile;
    if ((off & (kDecodeTile - 1)) == 0) {                    // first round of a tile: stage it
      __syncthreads();                                       // previous tile fully consumed
      tile_store<S, E>(tr, s_k, s_v, tid);
      __syncthreads();
      if (tile + 1 < ntiles) tile_load<S>(tr, kres, vres, (tile + 1) * kDecodeTile, last - t0 - (tile + 1) * kDecodeTile, tid);
    }
    const int tb = t0 + n * step + slot * G;
    if (!(active && slot_in_round && tb < t1)) return;
    const int brow = (off & (kDecodeTile - 1)) + slot * G;   // first tile row of this batch (even)

    // -- logits (Eq. (6)): shared path by slices + reduce-scatter, then the latent path --
    float part[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      uint32_t kw[S::SLICE_BYTES / 4];
      load_words<S::SLICE_BYTES>(kw, s_k + (brow + (i ^ g)) * S::KS_STRIDE + g * S::SLICE_BYTES);
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < S::DPL / 2; ++j) a = E::dot2(a, qs[j], pair_at<E>(kw, j));
      part[i] = a;
    }
    xor_reduce_scatter<G>(part);
    float sc = part[0];
    if constexpr (R > 0) {
#pragma unroll
      for (int i = 0; i < S::RP; ++i) {
        sc = E::dot2(sc, qt[i], pair_at<E>(zc.zk, i));
      }
    }
    const float s = (tb + g < t1) ? sc * p.scale_log2 : -INFINITY;

    // -- online softmax over the batch; the running max is refreshed only when
    //    a logit exceeds it by more than kDecStale --
    const float gmax = group_max<G>(s);                      // finite: token tb is valid
    if (gmax > m + kDecStale) {
      const float m_new = gmax;
      const float alpha = fast_exp2(m - m_new);               // 0 on the first batch (m = -inf)
      l *= alpha;
#pragma unroll
      for (int i = 0; i < S::DPL; ++i) acc_s[i] *= alpha;
#pragma unroll
      for (int i = 0; i < S::RPL; ++i) acc_z[i] *= alpha;
      m = m_new;
    }
    const float pe = fast_exp2(s - m);
    l += pe;
    // weights of tokens (2k, 2k+1) as one pair, held by both lanes of the pair
    const Pair pp = E::make_pair(dpp_mov<kDppEven>(pe), dpp_mov<kDppOdd>(pe));

    // -- aggregation (Eq. (7)): shared values and value latents --
    auto fold = [&](auto kc) {
      constexpr int k = decltype(kc)::value;
      Pair pk;
      if constexpr (S::PB == 4) {
        pk = __builtin_bit_cast(Pair, group_bcast<G, 2 * k>(__builtin_bit_cast(uint32_t, pp)));
      } else {
        const float2 f = __builtin_bit_cast(float2, pp);
        pk = make_float2(__uint_as_float(group_bcast<G, 2 * k>(__float_as_uint(f.x))),
                         __uint_as_float(group_bcast<G, 2 * k>(__float_as_uint(f.y))));
      }
      const unsigned char* vrow = s_v + ((brow >> 1) + k) * S::VP_STRIDE;
      uint32_t vw[S::VSLICE_BYTES / 4];
      if constexpr (S::CPS >= 1) {
#pragma unroll
        for (int c = 0; c < S::CPS; ++c)
          load_words<16>(vw + 4 * c, vrow + S::vchunk(g * S::CPS + c) * 16);
      } else {
        load_words<S::VSLICE_BYTES>(vw, vrow + g * S::VSLICE_BYTES);
      }
#pragma unroll
      for (int i = 0; i < S::DPL; ++i) acc_s[i] = E::dot2(acc_s[i], pk, pair_at<E>(vw, i));
      if constexpr (R > 0) {
#pragma unroll
        for (int i = 0; i < S::RPL; ++i)
          acc_z[i] = E::dot2(acc_z[i], pk, zip_at<E>(zc.zv[2 * k], zc.zv[2 * k + 1], i));
      }
    };
    [&]<int... K>(std::integer_sequence<int, K...>) {
      (fold(std::integral_constant<int, K>{}), ...);
    }(std::make_integer_sequence<int, G / 2>{});
  };

  // Latents prefetched kZDepth rounds ahead through kZDepth+1 register
  // buffers used round-robin (the loop is unrolled so each index is static).
  constexpr int NBUF = kZDepth + 1;
  ZRegs<S> zbuf[NBUF];
#pragma unroll
  for (int i = 0; i < kZDepth; ++i)
    if (i < nb) fetch(zbuf[i], i);
  for (int n = 0; n < nb; n += NBUF) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      if (n + u + kZDepth < nb) fetch(zbuf[(u + kZDepth) % NBUF], n + u + kZDepth);
      if (n + u < nb) process(zbuf[u], n + u);
    }
  }
}

template <class E, int DH, int R, int G>
__global__ __attribute__((amdgpu_flat_work_group_size(kDecodeThreads, kDecodeThreads), amdgpu_waves_per_eu(2)))
void decode_split_kernel(DecodeKernelParams p) {
  using S = DecodeShape<E, DH, R, G>;
  __shared__ __attribute__((aligned(16))) unsigned char s_k[kDecodeTile * S::KS_STRIDE];
  __shared__ __attribute__((aligned(16))) unsigned char s_v[(kDecodeTile / 2) * S::VP_STRIDE];

  const int tid = threadIdx.x;
  const int split = blockIdx.x;
  const int b = blockIdx.y;
  const int H = p.heads;
  const int g = tid % G;
  const int h = (tid / G) % p.heads_pow2;
  const int slot = tid / (G * p.heads_pow2);
  const bool active = (h < H) && (slot < p.slots);

  int len = p.seq_lens[b];
  len = len < 0 ? 0 : (len > p.max_len ? p.max_len : len);
  const int t0 = split * p.split_tokens;
  if (t0 >= len) return;                                   // whole workgroup: uniform exit
  const int t1 = min(t0 + p.split_tokens, len);

  float m = -INFINITY, l = 0.f;
  float acc_s[S::DPL];
  float acc_z[S::RPL > 0 ? S::RPL : 1];
#pragma unroll
  for (int i = 0; i < S::DPL; ++i) acc_s[i] = 0.f;
#pragma unroll
  for (int i = 0; i < (S::RPL > 0 ? S::RPL : 1); ++i) acc_z[i] = 0.f;

  decode_split_body<E, DH, R, G>(p, s_k, s_v, tid, b, split, t0, t1, g, h, slot, active, m, l, acc_s, acc_z);

  if (!active) return;
  // ---- partial state of this (split, slot, head) ----
  const float l_tot = group_sum<G>(l);
  const size_t pidx = (size_t(b) * p.partials + size_t(split) * p.slots + slot) * H + h;
  if (g == 0) {
    p.ws_ml[2 * pidx] = m;
    p.ws_ml[2 * pidx + 1] = l_tot;
  }
  float* dst = p.ws_acc + pidx * (DH + R);
#pragma unroll
  for (int i = 0; i < S::DPL; ++i) dst[g * S::DPL + i] = acc_s[i];
#pragma unroll
  for (int i = 0; i < S::RPL; ++i) dst[DH + g * S::RPL + i] = acc_z[i];
}

// Merge the partial states of one (sequence, head) and apply the residual
// up-projection once: o = (sum_j w_j acc_s_j + B^V_h sum_j w_j acc_z_j) / L,
// w_j = 2^(m_j - M), L = sum_j w_j l_j (Eq. (7): the latent sums are linear in
// the weights, so B^V is applied after the merge).  Thread t < DH + R owns
// merged dimension t; every thread folds all partial states itself (the
// (m, l) pairs are the same for every thread and come from cache), eight at
// a time with all of their loads issued together and an online rescale, so
// the kernel costs two dependent memory round trips (the length, then
// everything else) plus one LDS exchange of the latent sums.
constexpr int kMergeThreads = 256;
constexpr int kMergeBatch = 8;        // partial states whose loads are in flight together

template <class E, int DH, int R>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(
    const float* __restrict__ ws_ml, const float* __restrict__ ws_acc, const int32_t* __restrict__ seq_lens,
    const void* b_v, void* out, int heads, int partials, int slots, int split_tokens, int max_len, int batch,
    const int* __restrict__ ws_meta) {
  static_assert(DH + R <= kMergeThreads, "one thread per merged dimension");
  using T = typename E::T;
  __shared__ float s_z[R > 0 ? R : 1];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int col = tid < DH + R ? tid : DH + R - 1;           // threads past the last dimension shadow it
  int len = seq_lens[b];
  len = len < 0 ? 0 : (len > max_len ? max_len : len);
  T* o = static_cast<T*>(out) + (size_t(b) * heads + h) * DH;
  if (len == 0) {
    if (tid < DH) o[tid] = E::from_f32(0.f);
    return;
  }
  // B^V_h row of this output dimension, loaded alongside the partial states
  uint32_t bw[R > 0 ? (R * E::kBytes) / 4 : 1];
  if constexpr (R > 0) {
    if (tid < DH) load_words<R * E::kBytes>(bw, static_cast<const T*>(b_v) + (size_t(h) * DH + tid) * R);
  }
  // the partial states of this sequence: items j0 .. j0 + n - 1
  int j0, n;
  if (ws_meta) {                                             // balanced partition, recorded by the scan
    // clamped to the workspace, so that a workspace the scan did not fill
    // (a contract violation) gives wrong values, never an access outside it
    j0 = min(max(ws_meta[b], 0), partials - 1);
    const int u = max(ws_meta[batch], 1);
    n = min((len + u - 1) / u, partials - j0);
  } else {
    j0 = b * partials;
    n = ((len + split_tokens - 1) / split_tokens) * slots;
  }
  const float2* ml = reinterpret_cast<const float2*>(ws_ml) + size_t(j0) * heads + h;
  const float* acc = ws_acc + (size_t(j0) * heads + h) * (DH + R) + col;
  const size_t as = size_t(heads) * (DH + R);

  float M = -INFINITY, L = 0.f, a = 0.f;
  for (int j0 = 0; j0 < n; j0 += kMergeBatch) {
    float2 v[kMergeBatch];
    float x[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const bool ok = j0 + u < n;
      v[u] = ok ? ml[size_t(j0 + u) * heads] : make_float2(-INFINITY, 0.f);
      x[u] = ok ? acc[size_t(j0 + u) * as] : 0.f;
    }
    float mb = M;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) mb = fmaxf(mb, v[u].x);
    if (mb == -INFINITY) continue;                          // only empty states so far
    const float r = fast_exp2(M - mb);                      // 0 while M = -inf
    L *= r;
    a *= r;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const float w = fast_exp2(v[u].x - mb);              // empty state: m = -inf -> 0
      L = __builtin_fmaf(w, v[u].y, L);
      a = __builtin_fmaf(w, x[u], a);
    }
    M = mb;
  }
  if constexpr (R > 0) {
    if (tid >= DH && tid < DH + R) s_z[tid - DH] = a;
    __syncthreads();
  }
  if (tid < DH) {
    if constexpr (R > 0) {
#pragma unroll
      for (int i = 0; i < R; ++i) a = __builtin_fmaf(E::to_f32(elem_at<E>(bw, i)), s_z[i], a);
    }
    o[tid] = E::from_f32(a / L);
  }
}

// ---------------------------------------------------------------------------
// Host-side dispatch over the compiled envelope.
// ---------------------------------------------------------------------------
template <class E, int DH, int R, int G>
static hipError_t launch_decode_t(const DecodePlan& pl, const DecodeArgs& a, int phase, hipStream_t st) {
  DecodeKernelParams kp;
  kp.k_s = a.k_s; kp.v_s = a.v_s; kp.z_k = a.z_k; kp.z_v = a.z_v;
  kp.seq_lens = a.seq_lens; kp.q = a.q; kp.b_k = a.b_k;
  kp.scale_log2 = a.scale_log2;
  kp.heads = pl.heads; kp.heads_pow2 = pl.heads_pow2; kp.slots = pl.slots; kp.partials = pl.partials;
  kp.capacity = pl.capacity; kp.max_len = pl.max_len; kp.split_tokens = pl.split_tokens;
  kp.ws_ml = a.ws_ml; kp.ws_acc = a.ws_acc;
  if ((phase & 1) && pl.mfma) {
    const hipError_t e = launch_decode_mfma_scan(pl, a, st);
    if (e != hipSuccess) return e;
  } else if ((phase & 1) && pl.n_splits > 0) {
    hipLaunchKernelGGL((decode_split_kernel<E, DH, R, G>), dim3(pl.n_splits, pl.batch), dim3(kDecodeThreads), 0, st, kp);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!(phase & 2)) return hipSuccess;
  hipLaunchKernelGGL((decode_merge_kernel<E, DH, R>), dim3(pl.heads, pl.batch), dim3(kMergeThreads), 0, st,
                     a.ws_ml, a.ws_acc, a.seq_lens, a.b_v, a.out, pl.heads, pl.partials, pl.slots,
                     pl.split_tokens, pl.max_len, pl.batch, pl.balanced ? a.ws_meta : nullptr);
  return hipGetLastError();
}

template <class E, int DH, int R, int G>
static hipError_t launch_if_valid(const DecodePlan& pl, const DecodeArgs& a, int phase, hipStream_t st) {
  if constexpr ((R * E::kBytes) % 16 == 0 && DH % G == 0 && (R == 0 || R % G == 0)) {
    return launch_decode_t<E, DH, R, G>(pl, a, phase, st);
  } else {
    return hipErrorInvalidValue;
  }
}

template <class E, int DH>
static hipError_t dispatch_rank(const DecodePlan& pl, const DecodeArgs& a, int phase, hipStream_t st) {
  const bool g4 = pl.group == 4;
  switch (pl.rank) {
#define LRKV_RANK_CASE(RV)                                                                          \
    case RV: return g4 ? launch_if_valid<E, DH, RV, 4>(pl, a, phase, st) : launch_if_valid<E, DH, RV, 8>(pl, a, phase, st);
    LRKV_RANK_CASE(0) LRKV_RANK_CASE(4) LRKV_RANK_CASE(8) LRKV_RANK_CASE(16) LRKV_RANK_CASE(32) LRKV_RANK_CASE(64)
#undef LRKV_RANK_CASE
    default: return hipErrorInvalidValue;
  }
}

template <class E>
static hipError_t dispatch_dim(const DecodePlan& pl, const DecodeArgs& a, int phase, hipStream_t st) {
  switch (pl.head_dim) {
    case 16: return dispatch_rank<E, 16>(pl, a, phase, st);
    case 32: return dispatch_rank<E, 32>(pl, a, phase, st);
    case 64: return dispatch_rank<E, 64>(pl, a, phase, st);
    case 128: return dispatch_rank<E, 128>(pl, a, phase, st);
    default: return hipErrorInvalidValue;
  }
}

bool decode_supported(int dtype, int head_dim, int rank, int heads) {
  if (dtype != 0 && dtype != 1) return false;
  if (!(head_dim == 16 || head_dim == 32 || head_dim == 64 || head_dim == 128)) return false;
  if (!(rank == 0 || rank == 4 || rank == 8 || rank == 16 || rank == 32 || rank == 64)) return false;
  if (dtype == 1 && rank % 8 != 0) return false;           // 16-byte latent rows in bf16
  if (heads < 1 || heads > 64) return false;
  if (heads > 32 && rank == 0) return true;                 // G = 4
  if (heads > 32 && rank % 4 != 0) return false;
  return true;
}

hipError_t launch_decode(const DecodePlan& pl, const DecodeArgs& a, int phase, hipStream_t st) {
  if (pl.generic) return launch_decode_generic(pl, a, phase, st);
  return pl.dtype == 1 ? dispatch_dim<BF16>(pl, a, phase, st) : dispatch_dim<F32>(pl, a, phase, st);
}

hipError_t launch_plain_merge(int dtype, int head_dim, const float* ws_ml, const float* ws_acc,
                              const int32_t* seq_lens, void* out, int heads, int partials, int split_tokens,
                              int max_len, int batch, hipStream_t st) {
  const dim3 grid(heads, batch);
  if (dtype == 1 && head_dim == 64)
    hipLaunchKernelGGL((decode_merge_kernel<BF16, 64, 0>), grid, dim3(kMergeThreads), 0, st, ws_ml, ws_acc, seq_lens,
                       nullptr, out, heads, partials, 1, split_tokens, max_len, batch, nullptr);
  else if (dtype == 1 && head_dim == 128)
    hipLaunchKernelGGL((decode_merge_kernel<BF16, 128, 0>), grid, dim3(kMergeThreads), 0, st, ws_ml, ws_acc,
                       seq_lens, nullptr, out, heads, partials, 1, split_tokens, max_len, batch, nullptr);
  else if (dtype == 0 && head_dim == 64)
    hipLaunchKernelGGL((decode_merge_kernel<F32, 64, 0>), grid, dim3(kMergeThreads), 0, st, ws_ml, ws_acc, seq_lens,
                       nullptr, out, heads, partials, 1, split_tokens, max_len, batch, nullptr);
  else if (dtype == 0 && head_dim == 128)
    hipLaunchKernelGGL((decode_merge_kernel<F32, 128, 0>), grid, dim3(kMergeThreads), 0, st, ws_ml, ws_acc,
                       seq_lens, nullptr, out, heads, partials, 1, split_tokens, max_len, batch, nullptr);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lrkv
