// LRKV decode at any rank, with the shared term on bf16 MFMA.
//
// Method (Low-Rank Key Value Attention, slide discussion of arXiv:2601.11471v3):
//   logits  s_t = ( q_h.k_{s,t} + (B^K_h^T q_h).z^K_{t,h} ) / sqrt(d_h)     slide
//           "Compute logits without expanding historical keys", Eq. (6);
//   output  o_h = sum_t a_t v_{s,t} + B^V_h ( sum_t a_t z^V_{t,h} )           slide
//           "Aggregate values before the residual up-projection", Eq. (7);
// at the ranks the pages' trained models use (slide "The rank directly sets
// the theoretical cache budget", Table 7, ranks 46 to 55; slide "Backup: the
// complete rank sweep clarifies the trade-off", Table 8, up to 128), where a
// head's latent row of r bf16 need not fill whole 16-byte chunks, nor start
// on a 4-byte boundary when r is odd.
//
// Work decomposition and the shared term follow decode_mfma_kernel: a
// workgroup is 4 wave64 over one split of one sequence and one group of
// 32/F heads (F below; lanes of heads past the last one idle); the split's
// 32-token tiles are dealt to the waves round-robin, and per tile
//   S^T[t][c] = K_s[t][:] . Q[c][:]          (32 x d_h by d_h x 32 columns)
//   O_s^T[d][c] += V_s[t][d]^T . P^T[t][c]   (d_h x 32 by 32 x 32)
// run on v_mfma_f32_32x32x16_bf16, the shared rows copied global -> LDS one
// tile ahead.  Lane l owns MFMA column l%32 and, in every tile, the 16
// tokens 8(i/4) + 4(l/32) + i%4 of the accumulator layout.
//
// Latent terms.  With fewer heads than MFMA columns each head fills F = 1, 2
// or 4 columns (column j holds head j % (32/F); the shared term is simply
// computed F times), so a head owns 2F lanes: (column, half).  Lane slice k
// = 2 (j / (32/F)) + hf covers a window of 2*NAB consecutive elements of the
// head's latent row: slices 0..2F-2 start at k * 2*NAB, the last one ends at
// the row's end.  All windows lie inside the row; where the last overlaps its
// neighbour it skips its copy (zero absorbed query there, and those sums are
// not written).  For each accumulator row the lane loads its window of the
// two tokens the row holds in the two lane halves: NAB words from the 4-byte
// boundary at or below the window, plus one word when the rank is odd (the
// window then starts mid-word in some heads, and v_alignbyte shifts each
// word pair back onto bf16 pairs).  So no load reaches past the end of the
// row it serves, and none is partly outside the split's buffer range; rows
// past the split's end fall outside the split's buffer range (zeros).  Per
// token the lane forms a 2-wide bf16 dot over its window; xor-lane swizzles
// add the F column copies, and one cross-half swap (v_permlane32_swap) adds
// the two halves' dots of each token into the lanes that hold it; the
// weights go the other way for sum_t p_t z^V_{t,h}, with 2-wide dots over
// token pairs.  Latents are loaded with the cached policy: a wave's loads
// for one token cover its contiguous run of all heads in overlapping
// pieces, which the L1 then serves.
//
// The absorbed query q~_h = B^K_h^T q_h comes from decode_absorb_kernel (fp32
// in the workspace), rounded once to bf16 here.  Partial states use the
// layout of the any-rank merge: [sequence][split][head] x (m, l) and
// [..][d_h + r] sums, with B^V_h applied once per head in the merge.
//
// Numerics: fp32 accumulation; q~, the weights p in the value MFMA and the
// latent value dots are rounded to bf16 (relative error <= 2^-9 each).
#include "lrkv_device.h"
#include "lrkv_internal.h"

#include <utility>

namespace lrkv {

namespace {

constexpr int kMaWaves = 4;
constexpr int kMaThreads = 64 * kMaWaves;
constexpr int kMaHeads = 32;            // MFMA columns per wave (heads times their copies): the N dimension
constexpr int kMaTile = 32;             // cache tokens per tile: the M dimension
constexpr int kMaDH = 128;              // head dimension
constexpr float kMaStale = 8.f;         // running-max refresh threshold (log2 units)

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8): wait until at most n (< 64) vector-memory loads are
// outstanding, or until every LDS access has completed.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kLgkmZero = 0xC07F;

// Token (row of the 32-token tile) held in accumulator element i by lane half hf.
__device__ __forceinline__ constexpr int acc_row(int i, int hf) { return 8 * (i / 4) + 4 * hf + (i % 4); }

// v_permlane32_swap: swaps the upper half of x0 with the lower half of x1, so
// x0 becomes (x0 lower, x1 lower) and x1 becomes (x0 upper, x1 upper) across
// the two 32-lane halves.  For x0 = x1 = x every lane then holds the lower
// half's and the upper half's x.
__device__ __forceinline__ void swap_halves(uint32_t& x0, uint32_t& x1) {
  const auto r = __builtin_amdgcn_permlane32_swap(x0, x1, false, false);
  x0 = r[0];
  x1 = r[1];
}
// Lane l < 32 gets a[l] + a[l + 32], lane l >= 32 gets b[l - 32] + b[l]: the
// lower half the two halves' sum of a, the upper half that of b.
__device__ __forceinline__ float sum_halves(float a, float b) {
  uint32_t x0 = __float_as_uint(a), x1 = __float_as_uint(b);
  swap_halves(x0, x1);
  return __uint_as_float(x0) + __uint_as_float(x1);
}

// Words per lane window with F column copies per head: a 2F-th of a row's
// ceil(r/2) bf16 pairs, rounded up to whole 16-byte loads.
constexpr int window_words(int rank, int f) { return ((((rank + 1) / 2 + 2 * f - 1) / (2 * f)) + 3) / 4 * 4; }

// The 2F windows of 2*NAB elements fit a row as laid out (slices 0..2F-2 end
// inside it, with the extra word of an odd rank) and cover it.
constexpr bool windows_fit(int rank, int f) {
  const int nab = window_words(rank, f);
  return (2 * f - 1) * 2 * nab <= rank - (rank & 1) && 2 * f * 2 * nab >= rank;
}

// Column copies per head: as many as the head count allows (32 / F heads per
// workgroup) and the windows fit.
constexpr int column_copies(int rank, int heads) {
  if (heads <= 8 && windows_fit(rank, 4)) return 4;
  if (heads <= 16 && windows_fit(rank, 2)) return 2;
  return 1;
}

template <int NAB, bool ODD, int F>
struct MaShape {
  static constexpr int DH = kMaDH;
  static constexpr int HP = kMaHeads / F;      // heads per workgroup
  static constexpr int KC = DH / 16;           // k-chunks of the score MFMA
  static constexpr int VB = DH / 32;           // 32-feature blocks of the value MFMA
  static constexpr int RB = DH * 2;            // bytes per shared row
  static constexpr int CR = RB / 16;           // 16-byte chunks per shared row
  static constexpr int VT = kMaTile * RB;      // bytes of one shared-row tile in LDS
  static constexpr int NT = VT / 1024;         // 1 KB global -> LDS transfers per tile
  static constexpr int WL = NAB + (ODD ? 1 : 0);           // words loaded per token window
  static constexpr int LPW = NAB / 4 + (ODD ? 1 : 0);      // load instructions per token window
  // accumulator rows per latent group: two (consecutive tokens, paired in
  // the value dots) for windows up to 20 words, else one (its tokens A and B
  // paired), which halves the registers one group holds
  static constexpr int KG = NAB <= 20 ? 2 : 1;
  static constexpr int NG = 16 / KG;           // latent groups per tile and side
  static constexpr int GL = KG * 2 * LPW;      // loads per latent group
  // latent groups in flight, by the registers a group holds (one at 16-word
  // windows: deeper rings measured no faster there)
  static constexpr int D = KG * WL <= 8 ? 4 : KG * WL <= 17 ? 2 : 1;
  static constexpr int TILES = kMaWaves * 2 * VT;
  static constexpr int P = 16 * VB + 2 * NAB + 4;          // floats per lane in the fold
  static constexpr int FOLD = (kMaWaves * 64 * P + kMaWaves * kMaHeads) * 4;
  static constexpr int LDS = TILES > FOLD ? TILES : FOLD;
  static_assert(NAB % 4 == 0 && NAB >= 4 && NAB <= 32, "window of whole 16-byte loads");
  static_assert(F == 1 || F == 2 || F == 4, "column copies");
  static_assert((2 * NG) % D == 0, "ring slots repeat every tile");
};

struct MaParams {
  const void* k_s; const void* v_s; const void* z_k; const void* z_v;
  const int32_t* seq_lens;
  const void* q;
  const float* qt;                  // absorbed query [batch][heads][rank], fp32
  float scale_log2;
  int heads, rank, partials, max_len, split_tokens;
  int64_t capacity;
  float* ws_ml; float* ws_acc;
};

// q~[b][h][e] = sum_d q[b][h][d] B^K_h[d][e] (the absorbed query of Eq. (6)),
// fp32.  Grid (heads, ceil(batch / 8)), 256 threads: thread (e, g) takes
// elements e, e + 64, ... below the rank and the 32 dims d = 32g .. 32g + 31
// for 8 sequences (all 32 loads of a column slice in flight at once); the
// four dim slices are added in LDS.
constexpr int kAbSeq = 8;
__global__ __launch_bounds__(256) void decode_absorb_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ b_k, float* __restrict__ qt,
                                                            int batch, int heads, int rank) {
  constexpr int DH = kMaDH, DS = DH / 4;
  __shared__ float s_q[kAbSeq][DH];
  __shared__ float s_part[4][kAbSeq][64];
  const int h = blockIdx.x, b0 = blockIdx.y * kAbSeq, tid = threadIdx.x;
  const int el = tid & 63, g = tid >> 6;
  // column slice of B^K_h for elements e0 + el (every load unconditional)
  float w[DS];
  auto load_w = [&](int e0) {
    const int e = e0 + el < rank ? e0 + el : rank - 1;
#pragma unroll
    for (int k = 0; k < DS; ++k) w[k] = bf16_to_f32(b_k[(size_t(h) * DH + DS * g + k) * rank + e]);
  };
  load_w(0);                                                 // in flight while the queries are staged
  float qv[kAbSeq * DH / 256];
#pragma unroll
  for (int k = 0; k < kAbSeq * DH / 256; ++k) {          // all loads issued before any store
    const int i = tid + 256 * k, s = i / DH, d = i % DH, bb = b0 + s < batch ? b0 + s : batch - 1;
    qv[k] = bf16_to_f32(q[(size_t(bb) * heads + h) * DH + d]);
  }
#pragma unroll
  for (int k = 0; k < kAbSeq * DH / 256; ++k) {
    const int i = tid + 256 * k;
    s_q[i / DH][i % DH] = qv[k];                             // rows past the batch: never written out
  }
  __syncthreads();
  for (int e0 = 0; e0 < rank; e0 += 64) {                  // uniform
    if (e0 > 0) load_w(e0);
#pragma unroll
    for (int s = 0; s < kAbSeq; ++s) {
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < DS; ++k) acc = __builtin_fmaf(s_q[s][DS * g + k], w[k], acc);
      s_part[g][s][el] = acc;
    }
    __syncthreads();
    // thread (el, g) adds the four slices for sequences 2g and 2g + 1
    const int e = e0 + el;
#pragma unroll
    for (int s = 2 * g; s < 2 * g + 2; ++s) {
      const float v = (s_part[0][s][el] + s_part[1][s][el]) + (s_part[2][s][el] + s_part[3][s][el]);
      if (e < rank && b0 + s < batch) qt[(size_t(b0 + s) * heads + h) * rank + e] = v;
    }
    __syncthreads();
  }
}

template <int NAB, bool ODD, int F>
__global__ __attribute__((amdgpu_flat_work_group_size(kMaThreads, kMaThreads), amdgpu_waves_per_eu(1)))
void decode_mfma_any_kernel(MaParams p) {
  using S = MaShape<NAB, ODD, F>;
  constexpr int DH = S::DH;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, hf = lane >> 5;
  const int H = p.heads, R = p.rank;
  const int copy = j / S::HP;                                // column copy of this lane's head
  const int h = int(blockIdx.y) * S::HP + j % S::HP;
  const bool hv = h < H;                                     // lanes past the last head compute nothing kept
  const int slice = 2 * copy + hf;                           // this lane's window of the head's latent row
  const int b = blockIdx.z;

  // This workgroup's split: tokens [lo, hi) of sequence b (uniform exits).
  int len = p.seq_lens[b];
  len = len < 0 ? 0 : (len > p.max_len ? p.max_len : len);
  const int lo = int(blockIdx.x) * p.split_tokens;
  if (lo >= len) return;
  const int hi = min(lo + p.split_tokens, len);
  const int item = b * p.partials + int(blockIdx.x);
  const int nwg = hi - lo;
  const int ntile_wg = (nwg + kMaTile - 1) / kMaTile;
  const int ntiles = ntile_wg > wave ? (ntile_wg - wave + kMaWaves - 1) / kMaWaves : 0;   // this wave's
  auto gtile = [&](int kt) { return wave + kMaWaves * kt; };   // split tile of this wave's kt-th tile

  // Resources over the split's tokens (the host keeps them below 4 GiB).  With
  // heads * rank even (a host condition) every token's latent run starts on a
  // 4-byte boundary.
  const size_t row0 = size_t(b) * size_t(p.capacity) + size_t(lo);
  const uint32_t ztok = uint32_t(H) * uint32_t(R) * 2;     // latent bytes per token
  const __amdgpu_buffer_rsrc_t kres =
      buffer_resource(static_cast<const unsigned char*>(p.k_s) + row0 * S::RB, uint32_t(nwg) * S::RB);
  const __amdgpu_buffer_rsrc_t vres =
      buffer_resource(static_cast<const unsigned char*>(p.v_s) + row0 * S::RB, uint32_t(nwg) * S::RB);
  const __amdgpu_buffer_rsrc_t zkres =
      buffer_resource(static_cast<const unsigned char*>(p.z_k) + row0 * ztok, uint32_t(nwg) * ztok);
  const __amdgpu_buffer_rsrc_t zvres =
      buffer_resource(static_cast<const unsigned char*>(p.z_v) + row0 * ztok, uint32_t(nwg) * ztok);

  // This lane's window: elements [wofs, wofs + 2 NAB) of head h's row.  Its
  // byte in token 0 is wbyte (2 mod 4 where h * r + wofs is odd); loads
  // start at the boundary below, and `sh` is the byte shift back onto the
  // window's pairs.
  const bool last = slice == 2 * F - 1;
  const int wofs = last ? R - 2 * NAB : slice * 2 * NAB;
  const int ov = last ? 2 * F * 2 * NAB - R : 0;             // leading elements the previous slice covers
  const uint32_t wbyte = (uint32_t(h) * uint32_t(R) + uint32_t(wofs)) * 2;
  const uint32_t wload = wbyte & ~3u;
  const uint32_t sh = wbyte & 3u;

  unsigned char* const ktile = smem + wave * 2 * S::VT;    // this wave's key tile
  unsigned char* const vtile = ktile + S::VT;               // and value tile

  // Shared-row tile transfer (tile = split tile index): transfer x carries
  // LDS bytes [1024x, 1024x + 1024) of a tile, lane i the chunk at position
  // pos of row rw, i.e. source chunk pos ^ lds_swz(rw).  Rows at or past the
  // split's last token clamp to it.
  auto row_dma = [&](__amdgpu_buffer_rsrc_t res, int tile, unsigned char* dst) {
    const int last = nwg - 1 - tile * kMaTile;
    const int base = tile * kMaTile;
#pragma unroll
    for (int x = 0; x < S::NT; ++x) {
      const int q = x * 64 + lane, rw = q / S::CR, pos = q % S::CR;
      const int src = base + min(rw, last);
      dma16<kStream>(res, uint32_t(src * S::RB + ((pos ^ lds_swz(rw, S::CR)) * 16)), 0u, dst + x * 1024);
    }
  };

  // Latent ring.  Ring position pos in [0, 2NG) of a tile is key-latent group
  // pos (pos < NG) or value-latent group pos - NG; group a covers accumulator
  // rows 2a and 2a+1.  For row i the lane loads its window of token A =
  // acc_row(i, 0) and of token B = acc_row(i, 1).  Slot pos % D.
  uint32_t ring[S::D][S::KG][2][S::WL];
  auto z_load = [&](auto slot_c, int pos, int tile) {
    constexpr int slot = decltype(slot_c)::value;
    const __amdgpu_buffer_rsrc_t res = pos < S::NG ? zkres : zvres;
    const int a = pos % S::NG;
#pragma unroll
    for (int t = 0; t < S::KG; ++t) {
      const int i = a * S::KG + t;
#pragma unroll
      for (int sd = 0; sd < 2; ++sd) {
        // tokens past the split fall outside the buffer range (zeros); lanes
        // of heads past the last one read other heads' latents, never used
        const uint32_t off = uint32_t(tile * kMaTile + acc_row(i, sd)) * ztok + wload;
        buffer_words<4 * NAB, kCached>(ring[slot][t][sd], res, off, 0u);
        if constexpr (ODD) ring[slot][t][sd][NAB] = __builtin_amdgcn_raw_buffer_load_b32(res, int(off + 4 * NAB), 0, kCached);
      }
    }
  };
  // Word w of a loaded window (a bf16 pair of the window).
  auto wword = [&](const uint32_t* raw, int w) -> uint32_t {
    if constexpr (ODD) return __builtin_amdgcn_alignbyte(raw[w + 1], raw[w], sh);
    else return raw[w];
  };

  // ---- prologue: the query operand and the lane's absorbed-query window,
  // then the first transfers (key tile 0, value tile 0, latent groups
  // 0..D-1).  Half 1 zeroes the window elements half 0 also covers. ----
  bf16x8_t qop[S::KC];                                       // B operand: q_h dims 16c + 8hf .. +7
  float qv[2 * NAB];
  {
    const int hh = hv ? h : 0;
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + (size_t(b) * H + hh) * DH + 8 * hf;
#pragma unroll
    for (int c = 0; c < S::KC; ++c) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 16 * c);
      qop[c] = as_bf16x8(hv ? v : u32x4{0u, 0u, 0u, 0u});
    }
    const float* qtr = p.qt + (size_t(b) * H + hh) * R + wofs;
#pragma unroll
    for (int e = 0; e < 2 * NAB; ++e) qv[e] = qtr[e];
  }
  __builtin_amdgcn_sched_barrier(0);
  row_dma(kres, gtile(0), ktile);
  row_dma(vres, gtile(0), vtile);
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (z_load(std::integral_constant<int, I>{}, I, gtile(0)), ...);
  }(std::make_integer_sequence<int, S::D>{});
  __builtin_amdgcn_sched_barrier(0);
  uint32_t qh[NAB];                                          // the window of q~_h as bf16 pairs
  {
#pragma unroll
    for (int w = 0; w < NAB; ++w) {
      const float x0 = (hv && 2 * w >= ov) ? qv[2 * w] : 0.f;
      const float x1 = (hv && 2 * w + 1 >= ov) ? qv[2 * w + 1] : 0.f;
      qh[w] = pack_bf16x2(x0, x1);
    }
  }

  // LDS offsets (loop-invariant), as in decode_mfma_kernel.
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
  float acc_z[2 * NAB];                                      // window of sum_t p_t z^V_{t,h}
#pragma unroll
  for (int i = 0; i < 2 * NAB; ++i) acc_z[i] = 0.f;
  float m = -INFINITY, lsum = 0.f;

  // Issue order as in decode_mfma_kernel (every load unconditional; loads
  // past the split return zero, the tile transfers clamp): step kt issues
  // K(kt+1) after its key reads, latent groups D..D+NG-1 of the ring, V(kt+1)
  // after its value reads, then NG more latent groups.  The key and value
  // reads wait for their transfers with explicit counts of the loads issued
  // after them.
  constexpr int NK = S::NT, NV = S::NT;
  constexpr int kKAfter = NV + S::D * S::GL;
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

    // -- latent scores: s += q~_h . z^K_{t,h}; ring positions 0..NG-1 --
    [&]<int... A>(std::integer_sequence<int, A...>) {
      ([&] {
        constexpr int a = A, slot = a % S::D;
#pragma unroll
        for (int t = 0; t < S::KG; ++t) {
          float pa = 0.f, pb = 0.f;
#pragma unroll
          for (int w = 0; w < NAB; ++w) {
            pa = BF16::dot2(pa, qh[w], wword(ring[slot][t][0], w));
            pb = BF16::dot2(pb, qh[w], wword(ring[slot][t][1], w));
          }
          if constexpr (F >= 4) {                             // copies j, j ^ 8 (within each half)
            pa += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(pa), 0x201F));
            pb += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(pb), 0x201F));
          }
          if constexpr (F >= 2) {                             // copies j, j ^ 16
            pa += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(pa), 0x401F));
            pb += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(pb), 0x401F));
          }
          s[a * S::KG + t] += sum_halves(pa, pb);
        }
        __builtin_amdgcn_sched_barrier(0);
        z_load(std::integral_constant<int, slot>{}, a + S::D, gtile(kt));   // a + D < 2NG: same tile
        __builtin_amdgcn_sched_barrier(0);
      }(), ...);
    }(std::make_integer_sequence<int, S::NG>{});

    // -- online softmax (log2 domain); only a partial last tile is masked --
    if ((gtile(kt) + 1) * kMaTile > nwg) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (gtile(kt) * kMaTile + acc_row(i, hf) >= nwg) s[i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
    if (__builtin_amdgcn_ballot_w64(mx * p.scale_log2 > m + kMaStale)) {
      uint32_t x0 = __float_as_uint(mx), x1 = x0;
      swap_halves(x0, x1);                                    // this head's maxima of both halves
      const float mn = fmaxf(m, fmaxf(__uint_as_float(x0), __uint_as_float(x1)) * p.scale_log2);
      const float alpha = fast_exp2(m - mn);                  // 0 on the first tile (m = -inf)
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int f = 0; f < S::VB; ++f) oacc[f] *= alpha;
#pragma unroll
      for (int i = 0; i < 2 * NAB; ++i) acc_z[i] *= alpha;
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
        const uint2 lo2 = lds_read_tr16(vtile + 16 * c * S::RB + voff[f][0]);
        const uint2 hi2 = lds_read_tr16(vtile + 16 * c * S::RB + voff[f][1]);
        va[c] = u32x4{lo2.x, lo2.y, hi2.x, hi2.y};
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

    // -- latent values: acc_z += sum_t p_t z^V_{t,h} over the tile's 32
    //    tokens; ring positions NG..2NG-1.  One swap gives every lane the
    //    weights of tokens A (lower half's) and B (upper half's). --
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
        if constexpr (S::KG == 2) {
          constexpr int i = a * S::KG;                        // rows i, i+1: consecutive tokens
#pragma unroll
          for (int sd = 0; sd < 2; ++sd) {
            const uint32_t pp = sd == 0 ? pa_w[i / 2] : pb_w[i / 2];
#pragma unroll
            for (int w = 0; w < NAB; ++w) {
              const uint32_t z0 = wword(ring[slot][0][sd], w), z1 = wword(ring[slot][1][sd], w);
              acc_z[2 * w] = BF16::dot2(acc_z[2 * w], pp, __builtin_amdgcn_perm(z1, z0, 0x05040100u));
              acc_z[2 * w + 1] = BF16::dot2(acc_z[2 * w + 1], pp, __builtin_amdgcn_perm(z1, z0, 0x07060302u));
            }
          }
        } else {
          // row a: tokens A and B with weights (p_A, p_B)
          const uint32_t pp = __builtin_amdgcn_perm(pb_w[a / 2], pa_w[a / 2], (a & 1) ? 0x07060302u : 0x05040100u);
#pragma unroll
          for (int w = 0; w < NAB; ++w) {
            const uint32_t z0 = wword(ring[slot][0][0], w), z1 = wword(ring[slot][0][1], w);
            acc_z[2 * w] = BF16::dot2(acc_z[2 * w], pp, __builtin_amdgcn_perm(z1, z0, 0x05040100u));
            acc_z[2 * w + 1] = BF16::dot2(acc_z[2 * w + 1], pp, __builtin_amdgcn_perm(z1, z0, 0x07060302u));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        constexpr int nxt = pos + S::D;                        // next position for this slot
        if constexpr (nxt < 2 * S::NG) {
          z_load(std::integral_constant<int, slot>{}, nxt, gtile(kt));
        } else {
          z_load(std::integral_constant<int, slot>{}, nxt - 2 * S::NG, gtile(kt + 1));
        }
        __builtin_amdgcn_sched_barrier(0);
      }(), ...);
    }(std::make_integer_sequence<int, S::NG>{});
  }

  // ---- fold the four waves' states into the split's partial state (each
  //      wave's sums scaled by 2^(m - M), M the largest running maximum).
  //      The tile memory is reused once every transfer into it has landed. ----
  constexpr int P = S::P;
  float* const s_red = reinterpret_cast<float*>(smem);      // [wave][lane][P]
  float* const s_m = s_red + kMaWaves * 64 * P;             // [wave][head]
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  if (hf == 0) s_m[wave * kMaHeads + j] = m;
  __syncthreads();
  float M = s_m[j];
#pragma unroll
  for (int w = 1; w < kMaWaves; ++w) M = fmaxf(M, s_m[w * kMaHeads + j]);   // finite: wave 0 has tokens
  const float sc = m == -INFINITY ? 0.f : fast_exp2(m - M);
  {
    float* dst = s_red + (wave * 64 + lane) * P;
#pragma unroll
    for (int f = 0; f < S::VB; ++f)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<float4*>(dst + 16 * f + 4 * r4) = make_float4(
            oacc[f][4 * r4] * sc, oacc[f][4 * r4 + 1] * sc, oacc[f][4 * r4 + 2] * sc, oacc[f][4 * r4 + 3] * sc);
#pragma unroll
    for (int i = 0; i < 2 * NAB; i += 4)
      *reinterpret_cast<float4*>(dst + 16 * S::VB + i) =
          make_float4(acc_z[i] * sc, acc_z[i + 1] * sc, acc_z[i + 2] * sc, acc_z[i + 3] * sc);
    dst[P - 4] = lsum * sc;
  }
  __syncthreads();
  // Value block f is added up over the waves and written by wave f % 4; the
  // latent window sums and the softmax sum by wave VB % 4.
  const size_t pidx = size_t(item) * H + (hv ? h : 0);
  float* const out_acc = p.ws_acc + pidx * (DH + R);
  const float* const src0 = s_red + lane * P;               // this lane's slot of wave 0
#pragma unroll
  for (int f = 0; f < S::VB; ++f) {
    if (f % kMaWaves != wave) continue;                     // uniform
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float4 a = *reinterpret_cast<const float4*>(src0 + 16 * f + 4 * r4);
#pragma unroll
      for (int w = 1; w < kMaWaves; ++w) {
        const float4 v = *reinterpret_cast<const float4*>(src0 + w * 64 * P + 16 * f + 4 * r4);
        a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
      }
      if (hv && copy == 0) *reinterpret_cast<float4*>(out_acc + 32 * f + 8 * r4 + 4 * hf) = a;
    }
  }
  if (S::VB % kMaWaves == wave) {
#pragma unroll
    for (int i = 0; i < 2 * NAB; ++i) {
      float a = src0[16 * S::VB + i];
#pragma unroll
      for (int w = 1; w < kMaWaves; ++w) a += src0[w * 64 * P + 16 * S::VB + i];
      if (hv && i >= ov) out_acc[DH + wofs + i] = a;
    }
    float ls = src0[P - 4];
#pragma unroll
    for (int w = 1; w < kMaWaves; ++w) ls += src0[w * 64 * P + P - 4];
    uint32_t x0 = __float_as_uint(ls), x1 = x0;
    swap_halves(x0, x1);                                     // the two halves' sums of this head
    ls = __uint_as_float(x0) + __uint_as_float(x1);
    if (hf == 0 && copy == 0 && hv) *reinterpret_cast<float2*>(p.ws_ml + 2 * pidx) = make_float2(M, ls);
  }
}

template <int NAB, bool ODD, int F>
static hipError_t launch_any_t(const DecodePlan& pl, const DecodeArgs& a, hipStream_t st) {
  using S = MaShape<NAB, ODD, F>;
  MaParams kp;
  kp.k_s = a.k_s; kp.v_s = a.v_s; kp.z_k = a.z_k; kp.z_v = a.z_v;
  kp.seq_lens = a.seq_lens; kp.q = a.q; kp.qt = a.ws_qt;
  kp.scale_log2 = a.scale_log2;
  kp.heads = pl.heads; kp.rank = pl.rank; kp.partials = pl.partials;
  kp.max_len = pl.max_len; kp.split_tokens = pl.split_tokens;
  kp.capacity = pl.capacity;
  kp.ws_ml = a.ws_ml; kp.ws_acc = a.ws_acc;
  const hipError_t attr = allow_dynamic_lds<&decode_mfma_any_kernel<NAB, ODD, F>>(S::LDS);
  if (attr != hipSuccess) return attr;
  const dim3 grid(pl.n_splits, (pl.heads + S::HP - 1) / S::HP, pl.batch);
  hipLaunchKernelGGL((decode_mfma_any_kernel<NAB, ODD, F>), grid, dim3(kMaThreads), size_t(S::LDS), st, kp);
  return hipGetLastError();
}

// Instances: window words NAB up to 32 / F (a 2F-th of a rank-128 row).
template <int F, int NAB>
static hipError_t launch_any_nab(const DecodePlan& pl, const DecodeArgs& a, hipStream_t st) {
  if constexpr (NAB * F <= 32) {
    return (pl.rank & 1) ? launch_any_t<NAB, true, F>(pl, a, st) : launch_any_t<NAB, false, F>(pl, a, st);
  } else {
    return hipErrorInvalidValue;
  }
}

template <int F>
static hipError_t launch_any_f(const DecodePlan& pl, const DecodeArgs& a, hipStream_t st) {
  switch (window_words(pl.rank, F)) {
    case 4: return launch_any_nab<F, 4>(pl, a, st);
    case 8: return launch_any_nab<F, 8>(pl, a, st);
    case 12: return launch_any_nab<F, 12>(pl, a, st);
    case 16: return launch_any_nab<F, 16>(pl, a, st);
    case 20: return launch_any_nab<F, 20>(pl, a, st);
    case 24: return launch_any_nab<F, 24>(pl, a, st);
    case 28: return launch_any_nab<F, 28>(pl, a, st);
    case 32: return launch_any_nab<F, 32>(pl, a, st);
    default: return hipErrorInvalidValue;
  }
}

template <int F, int... N>
static hipError_t prepare_f(std::integer_sequence<int, N...>) {
  hipError_t e = hipSuccess;
  auto one = [&](auto nab_c) {
    constexpr int NAB = 4 * (decltype(nab_c)::value + 1);
    if constexpr (NAB * F <= 32) {
      if (e == hipSuccess) e = allow_dynamic_lds<&decode_mfma_any_kernel<NAB, false, F>>(MaShape<NAB, false, F>::LDS);
      if (e == hipSuccess) e = allow_dynamic_lds<&decode_mfma_any_kernel<NAB, true, F>>(MaShape<NAB, true, F>::LDS);
    }
  };
  (one(std::integral_constant<int, N>{}), ...);
  return e;
}

}  // namespace

bool decode_mfma_any_supported(int dtype, int head_dim, int rank, int heads) {
  if (dtype != 1 || head_dim != kMaDH || rank < 8 || rank > kGenericMaxRank) return false;
  if (heads < 1 || heads > kGenericMaxHeads || (int64_t(heads) * rank) % 2 != 0) return false;
  return windows_fit(rank, 1);                              // one copy per head always fits
}

// The default scan for the shapes both any-rank scans take: this one, but for
// 32-word windows (ranks above 112 with one column per head) with fewer than
// 32 heads, where most lanes idle and each lane's chain is longest (B = 32,
// 8K context, 20 heads at rank 128: the vector scan is faster).
bool decode_mfma_any_preferred(int dtype, int head_dim, int rank, int heads) {
  if (!decode_mfma_any_supported(dtype, head_dim, rank, heads)) return false;
  return window_words(rank, column_copies(rank, heads)) < 32 || heads >= 32;
}

hipError_t launch_decode_mfma_any(const DecodePlan& pl, const DecodeArgs& a, int phase, hipStream_t st) {
  if ((phase & 1) && pl.n_splits > 0) {
    const dim3 agrid(pl.heads, (pl.batch + kAbSeq - 1) / kAbSeq);
    hipLaunchKernelGGL(decode_absorb_kernel, agrid, dim3(256), 0, st, static_cast<const uint16_t*>(a.q),
                       static_cast<const uint16_t*>(a.b_k), a.ws_qt, pl.batch, pl.heads, pl.rank);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (column_copies(pl.rank, pl.heads)) {
      case 4: e = launch_any_f<4>(pl, a, st); break;
      case 2: e = launch_any_f<2>(pl, a, st); break;
      default: e = launch_any_f<1>(pl, a, st); break;
    }
    if (e != hipSuccess) return e;
  }
  if (!(phase & 2)) return hipSuccess;
  return launch_decode_generic(pl, a, 2, st);               // the any-rank merge
}

hipError_t decode_mfma_any_prepare() {
  hipError_t e = prepare_f<1>(std::make_integer_sequence<int, 8>{});
  if (e == hipSuccess) e = prepare_f<2>(std::make_integer_sequence<int, 8>{});
  if (e == hipSuccess) e = prepare_f<4>(std::make_integer_sequence<int, 8>{});
  return e;
}

}  // namespace lrkv
