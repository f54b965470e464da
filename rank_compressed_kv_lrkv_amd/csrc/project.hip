// Fused projection + append: the cache rows of new tokens computed from their
// hidden states and written straight into the cache.
//
// Method (Low-Rank Key Value Attention, slide discussion of arXiv:2601.11471v3):
// a token's hidden state x (width d) is projected to the shared features
// k_s = x W^K_shared, v_s = x W^V_shared (width d_h) and to the per-head
// latents z^K_h = x U^K_h, z^V_h = x U^V_h (width r), which is all the cache
// keeps (slide "Cache shared features and compact per-head latents",
// Eqs. (4)-(5)).  Concatenated, that is one product
//   y = x . [W^K_shared | W^V_shared | U^K_1 .. U^K_H | U^V_1 .. U^V_H]
// from d to 2(d_h + H r) outputs per token, a dense GEMM over the batch's
// tokens: C[M x N] = X[M x d] . W^T with M = batch * n_new, N = 2(d_h + H r),
// and the weight given output-major (W[N][d], each output's d weights
// contiguous), so both operands are contiguous along the contraction.
//
// Tiling: a workgroup (4 wave64) computes a 128 x 128 block of C; each wave a
// 64 x 64 quarter as 2 x 2 tiles of v_mfma_f32_32x32x16_bf16.  The contraction
// advances 32 at a time; the X and W slices of a step (128 rows x 64 bytes
// each) are copied global -> LDS (buffer loads into LDS), double-buffered,
// rows swizzled so the operand reads are free of bank conflicts.  Rows past
// M or N clamp to the last row (their results are not stored).
//
// Epilogue: each output is rounded once to bf16 and stored at cache slot
// pos[b] + i of token (b, i) in the array its column belongs to; the array
// boundaries (d_h, 2 d_h, 2 d_h + H r) are multiples of 32, so every 32-column
// MFMA tile belongs to one array.  Slots outside [0, capacity) are dropped,
// as for the append.
#include "lrkv_device.h"
#include "lrkv_internal.h"

namespace lrkv {

constexpr int kPjThreads = 256;
constexpr int kPjBM = 128, kPjBN = 128, kPjBK = 32;     // block tile and contraction step
constexpr int kPjRowBytes = kPjBK * 2;                   // one row of a step slice: 64 bytes
constexpr int kPjSlice = kPjBM * kPjRowBytes;            // 8 KB per operand and step
constexpr int kPjChunks = kPjRowBytes / 16;              // 16-byte chunks per slice row

// s_waitcnt immediate (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8): wait until at most n (< 64) vector-memory loads are outstanding.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

struct ProjectParams {
  const uint16_t* x; const uint16_t* w;
  uint16_t* k_s; uint16_t* v_s; uint16_t* z_k; uint16_t* z_v;
  const int32_t* pos;
  int M, N, K, n_new, head_dim, hr;   // hr = H * r
  int64_t capacity;
};

__global__ __launch_bounds__(kPjThreads) void project_append_kernel(ProjectParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char s_a[2][kPjSlice];
  __shared__ __attribute__((aligned(1024))) unsigned char s_b[2][kPjSlice];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;                 // the wave's 64 x 64 quarter
  const int n_lane = lane & 31, hf = lane >> 5;
  const int m0 = blockIdx.y * kPjBM, nb0 = blockIdx.x * kPjBN;

  // operand sources: rows m0.. of X and nb0.. of W, the whole contraction
  const __amdgpu_buffer_rsrc_t xres = buffer_resource(p.x + size_t(m0) * p.K, uint32_t(min(kPjBM, p.M - m0)) * p.K * 2);
  const __amdgpu_buffer_rsrc_t wres = buffer_resource(p.w + size_t(nb0) * p.K, uint32_t(min(kPjBN, p.N - nb0)) * p.K * 2);
  const int last_m = min(kPjBM, p.M - m0) - 1, last_n = min(kPjBN, p.N - nb0) - 1;

  // Transfer x of a slice carries LDS bytes [1024x, 1024x + 1024): 16 rows of
  // 64 bytes; lane i the chunk at position i % 4 of row 16x + i / 4, i.e.
  // source chunk pos ^ lds_swz(row, 4).  Each wave moves 2 of the 8.
  uint32_t a_off[2], b_off[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int xfer = wave * 2 + t, row = xfer * 16 + lane / 4, pos = lane % 4;
    const int ch = pos ^ lds_swz(row, kPjChunks);
    a_off[t] = uint32_t(min(row, last_m)) * p.K * 2 + ch * 16;
    b_off[t] = uint32_t(min(row, last_n)) * p.K * 2 + ch * 16;
  }
  auto load_step = [&](int ks, int buf) {
    const uint32_t k_off = uint32_t(ks) * kPjRowBytes;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int xfer = wave * 2 + t;
      dma16(xres, a_off[t] + k_off, 0u, &s_a[buf][xfer * 1024]);
      dma16(wres, b_off[t] + k_off, 0u, &s_b[buf][xfer * 1024]);
    }
  };

  // operand reads: lane (row n_lane of a 32-row tile, half hf) takes 16-byte
  // chunk 2c + hf of its row for contraction chunk c (k = 16c + 8hf ..)
  int a_rd[2][2], b_rd[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int ra = wm * 64 + t * 32 + n_lane, rb = wn * 64 + t * 32 + n_lane;
      a_rd[t][c] = ra * kPjRowBytes + ((2 * c + hf) ^ lds_swz(ra, kPjChunks)) * 16;
      b_rd[t][c] = rb * kPjRowBytes + ((2 * c + hf) ^ lds_swz(rb, kPjChunks)) * 16;
    }

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

  const int nsteps = p.K / kPjBK;
  load_step(0, 0);
  for (int ks = 0; ks < nsteps; ++ks) {
    const int buf = ks & 1;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));               // this wave's transfers of step ks have landed
    __syncthreads();                                        // everyone's have; buffer buf^1 is free
    if (ks + 1 < nsteps) load_step(ks + 1, buf ^ 1);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4 av[2], bv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        av[t] = *reinterpret_cast<const u32x4*>(&s_a[buf][a_rd[t][c]]);
        bv[t] = *reinterpret_cast<const u32x4*>(&s_b[buf][b_rd[t][c]]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(as_bf16x8(av[i]), as_bf16x8(bv[j]), acc[i][j]);
    }
  }

  // ---- epilogue: element e of tile (i, j) is row 8(e/4) + 4hf + e%4, column n_lane ----
  uint16_t* base[2];
  int col0[2], width[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n0 = nb0 + wn * 64 + j * 32;                 // first column of this 32-column tile
    if (n0 < p.head_dim) { base[j] = p.k_s; col0[j] = n0; width[j] = p.head_dim; }
    else if (n0 < 2 * p.head_dim) { base[j] = p.v_s; col0[j] = n0 - p.head_dim; width[j] = p.head_dim; }
    else if (n0 < 2 * p.head_dim + p.hr) { base[j] = p.z_k; col0[j] = n0 - 2 * p.head_dim; width[j] = p.hr; }
    else { base[j] = p.z_v; col0[j] = n0 - 2 * p.head_dim - p.hr; width[j] = p.hr; }
  }
  const bool col_ok[2] = {nb0 + wn * 64 < p.N, nb0 + wn * 64 + 32 < p.N};
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m0 + wm * 64 + i * 32 + 8 * (e / 4) + 4 * hf + (e % 4);
      if (m >= p.M) continue;
      const int b = m / p.n_new, tok = m - b * p.n_new;
      const long slot = long(p.pos ? p.pos[b] : 0) + tok;
      if (slot < 0 || slot >= p.capacity) continue;        // outside the cache: dropped
      const size_t row = size_t(b) * p.capacity + slot;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (col_ok[j]) base[j][row * width[j] + col0[j] + n_lane] = f32_to_bf16(acc[i][j][e]);
    }
}

// ---------------------------------------------------------------------------
// Large-tile projection for many tokens: a workgroup of 8 waves computes a
// 256 x (64 TJ) block of C, each wave a 64 x (32 TJ) part (2 x TJ tiles of
// v_mfma_f32_32x32x16_bf16: 2 + TJ operand reads from LDS per 2 TJ MFMAs).
// The contraction runs kPgBK at a time (one 128-byte line of every row)
// through a ring of kPgStages LDS stages; waves 0-3 copy the X slice of a
// stage, waves 4-7 the W slice, one stage ahead of the MFMAs.  One
// workgroup per compute unit (144 KB of LDS for TJ = 5), two waves per SIMD.
//
// Tile order is XCD-aware: workgroups are dispatched round-robin over the 8
// XCDs (L2 domains), so workgroup L runs on XCD L % 8; it takes tile
// (L % 8) * T/8 + L / 8 of the T tiles numbered row block by row block, so
// the column blocks of one row block run on one XCD at the same time and
// read its X rows (the large operand: 2 MB per row block at d = 4096) from
// that XCD's L2 once, while every XCD reads all of W (10.5 MB).
// ---------------------------------------------------------------------------
constexpr int kPgStages = 2;
constexpr int kPgThreads = 512;
constexpr int kPgBK = 64;                                  // contraction per stage
constexpr int kPgRowBytes = kPgBK * 2;                     // bytes of one row in a stage
constexpr int kPgChunks = kPgRowBytes / 16;                // 16-byte chunks per stage row
constexpr int kPgXferRows = 1024 / kPgRowBytes;            // rows one 1 KB transfer carries

template <int TJ>
struct PgShape {
  static constexpr int BM = 256, BN = 64 * TJ;
  static constexpr int A_BYTES = BM * kPgRowBytes, B_BYTES = BN * kPgRowBytes;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS = kPgStages * STAGE;
  static constexpr int A_XF = BM / kPgXferRows / 4;   // 1 KB transfers per stage of each X-copying wave
  static constexpr int B_XF = BN / kPgXferRows / 4;   // ... of each W-copying wave
  static constexpr int XF = A_XF > B_XF ? A_XF : B_XF;
};

// Store one 32 x 32 accumulator tile's bf16 results at their cache slots:
// element e of lane (n_lane, hf) is row rows[e] (cache row index, or -1 when
// dropped), column col0 + n_lane of the array at base with row width `width`.
__device__ __forceinline__ void store_tile(uint16_t* base, int width, int col0, const long* rows, int n_lane,
                                           const f32x16_t& acc) {
#pragma unroll
  for (int e = 0; e < 16; ++e)
    if (rows[e] >= 0) base[size_t(rows[e]) * width + col0 + n_lane] = f32_to_bf16(acc[e]);
}

// The array, first column and row width of the 32-column tile starting at output n0.
__device__ __forceinline__ uint16_t* column_target(const ProjectParams& p, int n0, int* col0, int* width) {
  if (n0 < p.head_dim) { *col0 = n0; *width = p.head_dim; return p.k_s; }
  if (n0 < 2 * p.head_dim) { *col0 = n0 - p.head_dim; *width = p.head_dim; return p.v_s; }
  if (n0 < 2 * p.head_dim + p.hr) { *col0 = n0 - 2 * p.head_dim; *width = p.hr; return p.z_k; }
  *col0 = n0 - 2 * p.head_dim - p.hr; *width = p.hr; return p.z_v;
}

// Cache row (sequence-major slot index) of output row m, or -1 if m is past
// the tokens or its slot is outside the cache.
__device__ __forceinline__ long cache_row(const ProjectParams& p, int m) {
  if (m >= p.M) return -1;
  const int b = m / p.n_new, tok = m - b * p.n_new;
  const long slot = long(p.pos ? p.pos[b] : 0) + tok;
  return (slot < 0 || slot >= p.capacity) ? -1 : long(b) * p.capacity + slot;
}

// Workgroup barrier without the memory fence of __syncthreads, which would
// also wait for every global -> LDS transfer still in flight, the stages
// ahead included.  The stage about to be read is complete once each wave's
// explicit vmcnt wait before the barrier has passed; every LDS read of the
// previous stage has returned, since its MFMAs were issued before the barrier;
// the empty asm statements keep the compiler from moving LDS accesses across.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int TJ>
__global__ __attribute__((amdgpu_flat_work_group_size(kPgThreads, kPgThreads), amdgpu_waves_per_eu(2)))
void project_gemm_kernel(ProjectParams p) {
  using S = PgShape<TJ>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;                 // the wave's 64 x 32TJ part
  const int n_lane = lane & 31, hf = lane >> 5;

  // XCD-aware tile order (runs of whole row blocks per XCD)
  const int nr = (p.M + S::BM - 1) / S::BM, nc = (p.N + S::BN - 1) / S::BN, T = nr * nc;
  const int L = blockIdx.x;
  const int t = (T % 8 == 0) ? (L % 8) * (T / 8) + L / 8 : L;
  const int m0 = (t / nc) * S::BM, nb0 = (t % nc) * S::BN;

  // copy role: waves 0-3 the X rows m0.., waves 4-7 the W rows nb0..
  const bool x_role = wave < 4;
  const int w4 = wave & 3;
  const int rows_valid = x_role ? min(S::BM, p.M - m0) : min(S::BN, p.N - nb0);
  const uint16_t* src = x_role ? p.x + size_t(m0) * p.K : p.w + size_t(nb0) * p.K;
  const __amdgpu_buffer_rsrc_t res = buffer_resource(src, uint32_t(rows_valid) * p.K * 2);
  const int nxf = x_role ? S::A_XF : S::B_XF;
  const int region = x_role ? 0 : S::A_BYTES;
  uint32_t off[S::XF];
#pragma unroll
  for (int u = 0; u < S::XF; ++u) {
    const int row = (w4 * nxf + u) * kPgXferRows + lane / kPgChunks;
    const int ch = (lane % kPgChunks) ^ lds_swz(row, kPgChunks);
    off[u] = uint32_t(min(row, rows_valid - 1)) * p.K * 2 + ch * 16;
  }
  auto issue = [&](int ks, int stage) {
    unsigned char* dst = smem + stage * S::STAGE + region + w4 * nxf * 1024;
    const uint32_t k_off = uint32_t(ks) * kPgRowBytes;
#pragma unroll
    for (int u = 0; u < S::XF; ++u)
      if (u < nxf) dma16(res, off[u] + k_off, 0u, dst + u * 1024);
  };

  // operand reads: lane (row n_lane of a 32-row tile, half hf) takes chunk 2c + hf
  constexpr int KC = kPgBK / 16;                           // MFMA contraction chunks per stage
  int a_rd[2][KC], b_rd[TJ][KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ra = wm * 64 + i * 32 + n_lane;
      a_rd[i][c] = ra * kPgRowBytes + ((2 * c + hf) ^ lds_swz(ra, kPgChunks)) * 16;
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int rb = wn * 32 * TJ + j * 32 + n_lane;
      b_rd[j][c] = S::A_BYTES + rb * kPgRowBytes + ((2 * c + hf) ^ lds_swz(rb, kPgChunks)) * 16;
    }
  }

  f32x16_t acc[2][TJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16_t{};

  const int nsteps = p.K / kPgBK;
#pragma unroll
  for (int s = 0; s < kPgStages - 1; ++s)
    if (s < nsteps) issue(s, s);
  for (int ks = 0; ks < nsteps; ++ks) {
    // stage ks has landed once at most (kPgStages - 2) later stages of this
    // wave's transfers are outstanding (all of them near the end)
    if (ks + kPgStages - 2 < nsteps) {
      if (x_role) __builtin_amdgcn_s_waitcnt(vmcnt_imm((kPgStages - 2) * S::A_XF));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm((kPgStages - 2) * S::B_XF));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    stage_barrier();                                       // every wave's part landed; stage (ks-1) is free
    if (ks + kPgStages - 1 < nsteps) issue(ks + kPgStages - 1, (ks + kPgStages - 1) % kPgStages);
    const unsigned char* st = smem + (ks % kPgStages) * S::STAGE;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      u32x4 av[2], bv[TJ];
#pragma unroll
      for (int i = 0; i < 2; ++i) av[i] = *reinterpret_cast<const u32x4*>(st + a_rd[i][c]);
#pragma unroll
      for (int j = 0; j < TJ; ++j) bv[j] = *reinterpret_cast<const u32x4*>(st + b_rd[j][c]);
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i) acc[i][j] = mfma32(as_bf16x8(av[i]), as_bf16x8(bv[j]), acc[i][j]);
    }
  }

  // ---- epilogue: element e of tile (i, j) is row 8(e/4) + 4hf + e%4, column n_lane ----
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    long rows[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) rows[e] = cache_row(p, m0 + wm * 64 + i * 32 + 8 * (e / 4) + 4 * hf + (e % 4));
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int n0 = nb0 + wn * 32 * TJ + j * 32;
      if (n0 >= p.N) continue;
      int col0, width;
      uint16_t* base = column_target(p, n0, &col0, &width);
      store_tile(base, width, col0, rows, n_lane, acc[i][j]);
    }
  }
}

// ---------------------------------------------------------------------------
// Projection of a few tokens (at most 64 rows, e.g. one token per sequence in
// a decode step): the weight read dominates, so the work is spread over the
// output columns and the contraction.  A workgroup of 16 waves takes 32
// output columns and every row; wave w takes the 16-wide contraction chunks
// w, w + 16, ... (in runs of kPsGroup consecutive chunks).  Operands go
// straight from global memory to registers (lane (n_lane, hf) loads 16 bytes
// of W row n0 + n_lane and of X rows 32 i + n_lane, at contraction offset
// 16 c + 8 hf), PsUnroll<MT> chunks in flight per wave; the 16 partial tiles
// are summed in LDS at the end.  Each
// load instruction takes 32 bytes of each of 32 rows, so a 128-byte line is
// touched by four instructions: the loads keep the cached policy, and the L1
// serves the later touches.
// ---------------------------------------------------------------------------
constexpr int kPsThreads = 1024, kPsWaves = 16, kPsHalf = kPsWaves / 2;
constexpr int kPsGroup = 1;            // consecutive 16-wide chunks a wave takes together
template <int MT> constexpr int PsUnroll = MT == 1 ? 8 : 4;

template <int MT>   // 32-row tiles covering the rows
__global__ __launch_bounds__(kPsThreads) void project_skinny_kernel(ProjectParams p) {
  constexpr int U = PsUnroll<MT>;
  static_assert(U % kPsGroup == 0, "whole runs of chunks per iteration");
  __shared__ float s_red[kPsHalf * MT * 16 * 64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_lane = lane & 31, hf = lane >> 5;
  const int n0 = blockIdx.x * 32;
  const uint32_t row_bytes = uint32_t(p.K) * 2;
  const __amdgpu_buffer_rsrc_t wres = buffer_resource(p.w + size_t(n0) * p.K, uint32_t(min(32, p.N - n0)) * row_bytes);
  const __amdgpu_buffer_rsrc_t xres = buffer_resource(p.x, uint32_t(p.M) * row_bytes);   // rows >= M read zero
  const uint32_t w_off = uint32_t(min(n_lane, p.N - n0 - 1)) * row_bytes + hf * 16;
  uint32_t x_off[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) x_off[i] = uint32_t(i * 32 + n_lane) * row_bytes + hf * 16;

  f32x16_t acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x16_t{};
  const int kchunks = p.K / 16;
  for (int g0 = wave; g0 * kPsGroup < kchunks; g0 += kPsWaves * (U / kPsGroup)) {
    u32x4 bw[U], ax[U][MT];
    auto chunk = [&](int u) { return (g0 + kPsWaves * (u / kPsGroup)) * kPsGroup + u % kPsGroup; };
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t koff = uint32_t(min(chunk(u), kchunks - 1)) * 32;
      bw[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, int(w_off + koff), 0, kCached));
#pragma unroll
      for (int i = 0; i < MT; ++i)
        ax[u][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xres, int(x_off[i] + koff), 0, 0));
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (chunk(u) < kchunks)                             // uniform: chunks past the end add nothing
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[i] = mfma32(as_bf16x8(ax[u][i]), as_bf16x8(bw[u]), acc[i]);
  }

  // sum the 16 partial tiles: the upper 8 waves hand theirs to the lower 8,
  // which then share out the final sums
  auto red = [&](int w, int i, int e) -> float& { return s_red[((w * MT + i) * 16 + e) * 64 + lane]; };
  if (wave >= kPsHalf) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) red(wave - kPsHalf, i, e) = acc[i][e];
  }
  __syncthreads();
  if (wave < kPsHalf) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) red(wave, i, e) += acc[i][e];
  }
  __syncthreads();
  if (wave >= kPsHalf) return;
  int col0, width;
  uint16_t* base = column_target(p, n0, &col0, &width);
  // wave w sums and stores elements 2w and 2w + 1 of every row tile
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = 2 * wave + k;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kPsHalf; ++w) v += red(w, i, e);
      const long row = cache_row(p, i * 32 + 8 * (e / 4) + 4 * hf + (e % 4));
      if (row >= 0) base[size_t(row) * width + col0 + n_lane] = f32_to_bf16(v);
    }
}

// ---------------------------------------------------------------------------
// The same few-token projection with the contraction also split across
// workgroups, when the caller passes a workspace: the weight read (the whole
// cost) then spreads over (N / 32) x S workgroups instead of N / 32.
// Workgroup (column block, slice s) sums its slice of 16-wide chunks over
// its 4 waves and writes the fp32 partial C_s [M][N] to the workspace; a
// second kernel adds the S partials of each output, rounds once and stores
// at the cache slot.
// ---------------------------------------------------------------------------
constexpr int kPkThreads = 256, kPkWaves = 4, kPkUnroll = 4, kPkMaxSlices = 16;

int project_slices(int d_model) {
  const int chunks = d_model / 16;
  return max(1, min(kPkMaxSlices, chunks / kPkWaves));   // at least one chunk per wave and slice
}

template <int MT>
__global__ __launch_bounds__(kPkThreads) void project_splitk_kernel(ProjectParams p, float* ws, int slices) {
  __shared__ float s_red[kPkWaves * MT * 16 * 64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_lane = lane & 31, hf = lane >> 5;
  const int n0 = blockIdx.x * 32, sl = blockIdx.y;
  const int kchunks = p.K / 16;
  const int c_lo = sl * kchunks / slices, c_hi = (sl + 1) * kchunks / slices;
  const uint32_t row_bytes = uint32_t(p.K) * 2;
  const __amdgpu_buffer_rsrc_t wres = buffer_resource(p.w + size_t(n0) * p.K, uint32_t(min(32, p.N - n0)) * row_bytes);
  const __amdgpu_buffer_rsrc_t xres = buffer_resource(p.x, uint32_t(p.M) * row_bytes);   // rows >= M read zero
  const uint32_t w_off = uint32_t(min(n_lane, p.N - n0 - 1)) * row_bytes + hf * 16;
  uint32_t x_off[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) x_off[i] = uint32_t(i * 32 + n_lane) * row_bytes + hf * 16;

  f32x16_t acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x16_t{};
  for (int c0 = c_lo + wave; c0 < c_hi; c0 += kPkWaves * kPkUnroll) {
    u32x4 bw[kPkUnroll], ax[kPkUnroll][MT];
#pragma unroll
    for (int u = 0; u < kPkUnroll; ++u) {
      const uint32_t koff = uint32_t(min(c0 + kPkWaves * u, c_hi - 1)) * 32;
      bw[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres, int(w_off + koff), 0, kCached));
#pragma unroll
      for (int i = 0; i < MT; ++i)
        ax[u][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xres, int(x_off[i] + koff), 0, 0));
    }
#pragma unroll
    for (int u = 0; u < kPkUnroll; ++u)
      if (c0 + kPkWaves * u < c_hi)                        // uniform
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[i] = mfma32(as_bf16x8(ax[u][i]), as_bf16x8(bw[u]), acc[i]);
  }
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) s_red[((wave * MT + i) * 16 + e) * 64 + lane] = acc[i][e];
  __syncthreads();
  // wave w adds up elements 4w .. 4w + 3 of every row tile and writes them
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = 4 * wave + k;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kPkWaves; ++w) v += s_red[((w * MT + i) * 16 + e) * 64 + lane];
      const int m = i * 32 + 8 * (e / 4) + 4 * hf + (e % 4);
      if (m < p.M) ws[(size_t(sl) * p.M + m) * p.N + n0 + n_lane] = v;
    }
}

// Thread t adds up outputs 4t .. 4t + 3 (N is a multiple of 32, so they share
// a row and an array) over the slices, all slices' loads issued together.
__global__ __launch_bounds__(256) void project_reduce_kernel(ProjectParams p, const float* ws, int slices) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (4 * t >= p.M * p.N) return;
  const int m = (4 * t) / p.N, n = 4 * t - m * p.N;
  float4 part[kPkMaxSlices];
#pragma unroll
  for (int s = 0; s < kPkMaxSlices; ++s)
    part[s] = s < slices ? *reinterpret_cast<const float4*>(ws + (size_t(s) * p.M + m) * p.N + n)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
  float4 v = part[0];
#pragma unroll
  for (int s = 1; s < kPkMaxSlices; ++s) {
    v.x += part[s].x; v.y += part[s].y; v.z += part[s].z; v.w += part[s].w;
  }
  const long row = cache_row(p, m);
  if (row < 0) return;
  int col0, width;
  uint16_t* base = column_target(p, n & ~31, &col0, &width);
  uint16_t* dst = base + size_t(row) * width + col0 + (n & 31);
  *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}

// ---------------------------------------------------------------------------
// Vector-ALU projection for the shapes the MFMA kernel does not take (fp32,
// or bf16 with array widths that are not multiples of 32): a 64 x 64 block of
// C per workgroup, 4 x 4 outputs per lane, the contraction staged through LDS
// 16 at a time, fp32 fused multiply-adds.  Same output placement.
// ---------------------------------------------------------------------------
constexpr int kPvT = 64, kPvK = 16;

template <class E>
__global__ __launch_bounds__(256) void project_append_valu_kernel(ProjectParams p) {
  using T = typename E::T;
  __shared__ float s_x[kPvK][kPvT + 4];
  __shared__ float s_w[kPvK][kPvT + 4];
  const T* x = reinterpret_cast<const T*>(p.x);
  const T* w = reinterpret_cast<const T*>(p.w);
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  const int m0 = blockIdx.y * kPvT, n0 = blockIdx.x * kPvT;
  // staging: lane loads row tid / 4 at contraction offsets 4(tid % 4) .. +3
  const int lrow = tid / 4, lk = (tid % 4) * 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < p.K; k0 += kPvK) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = k0 + lk + u, mr = m0 + lrow, nr = n0 + lrow;
      s_x[lk + u][lrow] = (mr < p.M && k < p.K) ? E::to_f32(x[size_t(mr) * p.K + k]) : 0.f;
      s_w[lk + u][lrow] = (nr < p.N && k < p.K) ? E::to_f32(w[size_t(nr) * p.K + k]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPvK; ++k) {
      float a[4], bb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) { a[u] = s_x[k][ty * 4 + u]; bb[u] = s_w[k][tx * 4 + u]; }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(a[u], bb[v], acc[u][v]);
    }
    __syncthreads();
  }
  T* outs[4] = {reinterpret_cast<T*>(p.k_s), reinterpret_cast<T*>(p.v_s), reinterpret_cast<T*>(p.z_k),
                reinterpret_cast<T*>(p.z_v)};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int m = m0 + ty * 4 + u;
    if (m >= p.M) continue;
    const int b = m / p.n_new, tok = m - b * p.n_new;
    const long slot = long(p.pos ? p.pos[b] : 0) + tok;
    if (slot < 0 || slot >= p.capacity) continue;
    const size_t row = size_t(b) * p.capacity + slot;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int n = n0 + tx * 4 + v;
      if (n >= p.N) continue;
      int which, col, width;
      if (n < p.head_dim) { which = 0; col = n; width = p.head_dim; }
      else if (n < 2 * p.head_dim) { which = 1; col = n - p.head_dim; width = p.head_dim; }
      else if (n < 2 * p.head_dim + p.hr) { which = 2; col = n - 2 * p.head_dim; width = p.hr; }
      else { which = 3; col = n - 2 * p.head_dim - p.hr; width = p.hr; }
      outs[which][row * width + col] = E::from_f32(acc[u][v]);
    }
  }
}

// ---------------------------------------------------------------------------
// Packing of the projection weights into the output-major matrix the
// projection reads: row n of W holds the d_model weights of output n, for
// n < d_h the columns of W^K_shared [d][d_h], then W^V_shared, then column j
// of U^K_h [H][d][r] at row 2 d_h + h r + j, then U^V_h.  A transpose through
// LDS in 32 x 32 tiles; elements are copied bit-exactly.
// ---------------------------------------------------------------------------
struct PackParams {
  const unsigned char* wk; const unsigned char* wv; const unsigned char* uk; const unsigned char* uv;
  unsigned char* out;
  int d_model, head_dim, rank, hr, N, es;
};

__device__ __forceinline__ const unsigned char* pack_src(const PackParams& p, int k, int n) {
  if (n < p.head_dim) return p.wk + (size_t(k) * p.head_dim + n) * p.es;
  if (n < 2 * p.head_dim) return p.wv + (size_t(k) * p.head_dim + n - p.head_dim) * p.es;
  const bool is_k = n < 2 * p.head_dim + p.hr;
  const int c = n - 2 * p.head_dim - (is_k ? 0 : p.hr), h = c / p.rank, j = c - h * p.rank;
  return (is_k ? p.uk : p.uv) + ((size_t(h) * p.d_model + k) * p.rank + j) * p.es;
}

__global__ __launch_bounds__(256) void pack_projection_kernel(PackParams p) {
  __shared__ uint32_t tile[32][33];
  const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;
  const int n0 = blockIdx.x * 32, k0 = blockIdx.y * 32;
#pragma unroll
  for (int u = 0; u < 4; ++u) {                           // read: consecutive lanes along n
    const int k = k0 + ty + 8 * u, n = n0 + tx;
    uint32_t v = 0;
    if (k < p.d_model && n < p.N) {
      const unsigned char* s = pack_src(p, k, n);
      v = p.es == 2 ? uint32_t(*reinterpret_cast<const uint16_t*>(s)) : *reinterpret_cast<const uint32_t*>(s);
    }
    tile[ty + 8 * u][tx] = v;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u) {                           // write: consecutive lanes along k
    const int n = n0 + ty + 8 * u, k = k0 + tx;
    if (k >= p.d_model || n >= p.N) continue;
    unsigned char* d = p.out + (size_t(n) * p.d_model + k) * p.es;
    const uint32_t v = tile[tx][ty + 8 * u];
    if (p.es == 2) *reinterpret_cast<uint16_t*>(d) = uint16_t(v);
    else *reinterpret_cast<uint32_t*>(d) = v;
  }
}

bool project_mfma_supported(int dtype, int head_dim, int rank, int heads, int d_model) {
  return dtype == 1 && head_dim % 32 == 0 && (heads * rank) % 32 == 0 && d_model % kPjBK == 0 && d_model > 0;
}

// Compute units of the current device.
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

template <int TJ>
hipError_t launch_gemm(const ProjectParams& p, dim3 grid, hipStream_t st) {
  const hipError_t attr = allow_dynamic_lds<&project_gemm_kernel<TJ>>(PgShape<TJ>::LDS);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((project_gemm_kernel<TJ>), grid, dim3(kPgThreads), size_t(PgShape<TJ>::LDS), st, p);
  return hipGetLastError();
}

size_t project_ws_bytes(long M, long N, int d_model) {
  return size_t(project_slices(d_model)) * size_t(M) * size_t(N) * sizeof(float);
}

size_t project_workspace_bytes(int dtype, int batch, int n_new, int heads, int head_dim, int rank, int d_model) {
  const long M = long(batch) * n_new, N = 2L * (head_dim + long(heads) * rank);
  if (!project_mfma_supported(dtype, head_dim, rank, heads, d_model) || M > 64 || M <= 0) return 0;
  const int tj = N % 320 == 0 ? 5 : 4;
  if (d_model % kPgBK == 0 && (M + 255) / 256 * ((N + 64 * tj - 1) / (64 * tj)) >= device_cus()) return 0;
  return project_ws_bytes(M, N, d_model);
}

const char* project_kernel_name(int dtype, int batch, int n_new, int heads, int head_dim, int rank, int d_model,
                                bool with_workspace) {
  if (!project_mfma_supported(dtype, head_dim, rank, heads, d_model)) return "project_append_valu_kernel";
  const long M = long(batch) * n_new, N = 2L * (head_dim + long(heads) * rank);
  const int tj = N % 320 == 0 ? 5 : 4;
  if (d_model % kPgBK == 0 && (M + 255) / 256 * ((N + 64 * tj - 1) / (64 * tj)) >= device_cus())
    return "project_gemm_kernel";
  if (M <= 64) return with_workspace ? "project_splitk_kernel" : "project_skinny_kernel";
  return "project_append_kernel";
}

hipError_t launch_project_append(const ProjectArgs& a, hipStream_t st) {
  ProjectParams p;
  p.x = static_cast<const uint16_t*>(a.x);
  p.w = static_cast<const uint16_t*>(a.w);
  p.k_s = static_cast<uint16_t*>(a.k_s); p.v_s = static_cast<uint16_t*>(a.v_s);
  p.z_k = static_cast<uint16_t*>(a.z_k); p.z_v = static_cast<uint16_t*>(a.z_v);
  p.pos = a.pos;
  p.M = a.batch * a.n_new;
  p.hr = a.heads * a.rank;
  p.N = 2 * (a.head_dim + p.hr);
  p.K = a.d_model;
  p.n_new = a.n_new;
  p.head_dim = a.head_dim;
  p.capacity = a.capacity;
  if (p.M <= 0) return hipSuccess;
  if (project_mfma_supported(a.dtype, a.head_dim, a.rank, a.heads, a.d_model)) {
    const int tj = p.N % 320 == 0 ? 5 : 4;
    const long big_tiles = long((p.M + 255) / 256) * ((p.N + 64 * tj - 1) / (64 * tj));
    if (p.K % kPgBK == 0 && big_tiles >= device_cus()) {
      // enough large tiles to fill the chip: the 256-row, 8-wave kernel
      const dim3 grid{unsigned(big_tiles)};
      if (tj == 5) return launch_gemm<5>(p, grid, st);
      return launch_gemm<4>(p, grid, st);
    }
    if (p.M <= 64 && a.ws != nullptr && a.ws_bytes >= project_ws_bytes(p.M, p.N, p.K)) {
      // a few tokens, with a workspace: the contraction split across workgroups too
      const int slices = project_slices(p.K);
      const dim3 grid(unsigned(p.N / 32), unsigned(slices));
      if (p.M <= 32) hipLaunchKernelGGL(project_splitk_kernel<1>, grid, dim3(kPkThreads), 0, st, p, a.ws, slices);
      else hipLaunchKernelGGL(project_splitk_kernel<2>, grid, dim3(kPkThreads), 0, st, p, a.ws, slices);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(project_reduce_kernel, dim3(unsigned((p.M * p.N / 4 + 255) / 256)), dim3(256), 0, st, p,
                         static_cast<const float*>(a.ws), slices);
      return hipGetLastError();
    }
    if (p.M <= 64) {
      // a few tokens: spread the weight read over columns and contraction
      const dim3 grid{unsigned(p.N / 32)};
      if (p.M <= 32) hipLaunchKernelGGL(project_skinny_kernel<1>, grid, dim3(kPsThreads), 0, st, p);
      else hipLaunchKernelGGL(project_skinny_kernel<2>, grid, dim3(kPsThreads), 0, st, p);
      return hipGetLastError();
    }
    const dim3 grid((p.N + kPjBN - 1) / kPjBN, (p.M + kPjBM - 1) / kPjBM);
    hipLaunchKernelGGL(project_append_kernel, grid, dim3(kPjThreads), 0, st, p);
  } else {
    const dim3 grid((p.N + kPvT - 1) / kPvT, (p.M + kPvT - 1) / kPvT);
    if (a.dtype == 1) hipLaunchKernelGGL(project_append_valu_kernel<BF16>, grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL(project_append_valu_kernel<F32>, grid, dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_pack_projection(const PackArgs& a, hipStream_t st) {
  PackParams p;
  p.wk = static_cast<const unsigned char*>(a.wk_shared); p.wv = static_cast<const unsigned char*>(a.wv_shared);
  p.uk = static_cast<const unsigned char*>(a.u_k); p.uv = static_cast<const unsigned char*>(a.u_v);
  p.out = static_cast<unsigned char*>(a.w_packed);
  p.d_model = a.d_model; p.head_dim = a.head_dim; p.rank = a.rank; p.hr = a.heads * a.rank;
  p.N = 2 * (a.head_dim + p.hr);
  p.es = a.dtype == 1 ? 2 : 4;
  if (p.d_model <= 0) return hipSuccess;
  const dim3 grid((p.N + 31) / 32, (p.d_model + 31) / 32);
  hipLaunchKernelGGL(pack_projection_kernel, grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t project_prepare() {
  hipError_t e = allow_dynamic_lds<&project_gemm_kernel<4>>(PgShape<4>::LDS);
  if (e == hipSuccess) e = allow_dynamic_lds<&project_gemm_kernel<5>>(PgShape<5>::LDS);
  return e;
}

}  // namespace lrkv
