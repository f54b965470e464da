// LRKV causal prefill for the shapes the MFMA prefills do not take: fp32
// storage, head widths 16 and 32, an odd number of heads at an odd rank,
// and ranks 123, 125 and 127 (any rank up to 128, head widths 16-128 are
// accepted).  Same operation and arguments as prefill_kernel (slides
// "Compute logits without expanding historical keys", Eq. (6) with the
// causal mask, and "Aggregate values before the residual up-projection",
// Eq. (7)), in the absorbed form with fp32 arithmetic throughout:
//   S = scale * [Q_h | Q_h B^K_h] . [K_s | R^K_h]^T,
//   [O_s | O_z] = softmax(S) . [V_s | R^V_h],  O = (O_s + O_z (B^V_h)^T) / l.
// Per-head keys and values are never formed.
//
// Work decomposition: a workgroup takes 32 query rows of one head; thread t
// serves query t / 8 with the 7 others of its aligned group of 8 lanes.  The
// augmented query rows (q and q B^K_h) sit in LDS; key tiles of 32 tokens
// (shared rows plus this head's latents, converted to fp32) are staged in
// LDS, lane j of a query's group scores keys j, j+8, j+16, j+24 of the tile
// (16-byte LDS reads, the query's 4 columns reused for the 4 keys), the
// group shares the running max by shuffles, and lane j accumulates the
// augmented output dims 32c + 4j .. 32c + 4j + 3.
#include "lrkv_device.h"
#include "lrkv_internal.h"

#include <utility>

namespace lrkv {

constexpr int kPgQ = 32;                    // query rows per workgroup
constexpr int kPgK = 32;                    // key tokens per tile
constexpr int kPgThreads = 256;             // 8 lanes per query row
constexpr int kPgMaxDims = 128 + kPrefillGenericMaxRank;
constexpr int kPgBlocks = (kPgMaxDims + 31) / 32;   // 32-dim blocks of the augmented row, at most
static_assert(kPgQ * 8 == kPgThreads, "8 lanes per query row");

// LDS row stride (floats) of the augmented rows: a multiple of 4 for 16-byte
// reads, and 4 more when that is a multiple of 32, so that the 8 rows the
// lanes of a group read at one column cover distinct banks.
__host__ __device__ constexpr int pg_stride(int dims) {
  const int s = (dims + 3) & ~3;
  return s % 32 == 0 ? s + 4 : s;
}
// LDS floats: augmented queries, key tile, value tile ([32][stride] each)
// and the weights [32][kPgK + 4].
static int prefill_generic_lds_floats(int dims) { return 3 * kPgQ * pg_stride(dims) + kPgQ * (kPgK + 4); }

template <class E>
__device__ __forceinline__ float pg_elem(const void* base, size_t i) {
  return E::to_f32(static_cast<const typename E::T*>(base)[i]);
}

// 8 consecutive elements of a shared row (16-byte aligned), as loaded
template <class E> struct PgRaw8;
template <> struct PgRaw8<BF16> { u32x4 w; };
template <> struct PgRaw8<F32> { float4 x, y; };

template <class E>
__device__ __forceinline__ PgRaw8<E> pg_load8(const void* base, size_t i) {
  PgRaw8<E> r;
  if constexpr (E::kBytes == 2) {
    r.w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + i);
  } else {
    r.x = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + i);
    r.y = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + i + 4);
  }
  return r;
}

// the 8 elements as fp32 into LDS (16-byte aligned)
template <class E>
__device__ __forceinline__ void pg_store8(float* dst, const PgRaw8<E>& r) {
  if constexpr (E::kBytes == 2) {
    const uint32_t v[4] = {r.w.x, r.w.y, r.w.z, r.w.w};
    *reinterpret_cast<float4*>(dst) = make_float4(__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xFFFF0000u),
                                                  __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xFFFF0000u));
    *reinterpret_cast<float4*>(dst + 4) = make_float4(__uint_as_float(v[2] << 16), __uint_as_float(v[2] & 0xFFFF0000u),
                                                      __uint_as_float(v[3] << 16), __uint_as_float(v[3] & 0xFFFF0000u));
  } else {
    *reinterpret_cast<float4*>(dst) = r.x;
    *reinterpret_cast<float4*>(dst + 4) = r.y;
  }
}

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// NB: 32-dim blocks covering the augmented row (D rounded up to 4 <= 32 NB).
template <class E, int NB>
__global__ __attribute__((amdgpu_flat_work_group_size(kPgThreads, kPgThreads), amdgpu_waves_per_eu(2)))
void prefill_generic_kernel(PrefillArgs a, int n_qblocks) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int DH = a.head_dim, R = a.rank, H = a.heads, L = a.seq_len;
  const int D = DH + R, DS = pg_stride(D), D4 = (D + 3) & ~3;
  float* const s_q = smem;                       // [kPgQ][DS]
  float* const s_k = s_q + kPgQ * DS;            // [kPgK][DS]
  float* const s_v = s_k + kPgK * DS;            // [kPgK][DS]
  float* const s_p = s_v + kPgK * DS;            // [kPgQ][kPgK + 4]
  const int qb = n_qblocks - 1 - int(blockIdx.x);   // heaviest blocks first
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, qi = tid >> 3, j8 = tid & 7;
  int start = a.start ? a.start[b] : 0;
  start = start < 0 ? 0 : (start > a.max_start ? a.max_start : start);
  const int q0 = qb * kPgQ;
  const int nkeys = start + L;                   // keys [0, nkeys) of this sequence
  const int qpos = start + q0 + qi;              // position of this lane's query
  const int kend = min(start + q0 + kPgQ, nkeys);
  const int ntiles = (kend + kPgK - 1) / kPgK;
  const int c8 = DH / 8;                         // 8-dim chunks of a shared row

  // augmented query rows; rows past the sequence repeat its last row (their
  // results are never stored).  Columns D .. D4-1 are zero in every row.
  for (int i = tid; i < kPgQ * c8; i += kPgThreads) {
    const int r = i / c8, c = i % c8, row = min(q0 + r, L - 1);
    pg_store8<E>(s_q + r * DS + 8 * c, pg_load8<E>(a.q, ((size_t(b) * L + row) * H + h) * DH + 8 * c));
  }
  for (int i = tid; i < kPgQ * (D4 - D); i += kPgThreads) {
    const int r = i / (D4 - D), x = D + i % (D4 - D);
    s_q[r * DS + x] = 0.f;
    s_k[r * DS + x] = 0.f;
    s_v[r * DS + x] = 0.f;
  }
  __syncthreads();
  for (int i = tid; i < kPgQ * R; i += kPgThreads) {
    const int r = i / R, j = i % R;
    float acc = 0.f;
    for (int d = 0; d < DH; ++d) acc = __builtin_fmaf(s_q[r * DS + d], pg_elem<E>(a.b_k, (size_t(h) * DH + d) * R + j), acc);
    s_q[r * DS + DH + j] = acc;
  }

  float m = -INFINITY, l = 0.f;
  // this lane accumulates the augmented dims 32c + 4 j8 + e, e < 4; a lane
  // whose dims of block c reach past D4 reads the row's last 4 columns
  // instead (in bounds; those accumulators are never used)
  float4 acc[NB];
  int vcol[NB];
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    acc[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    vcol[c] = min(32 * c + 4 * j8, D4 - 4);
  }
  const float* const qrow = s_q + qi * DS;
  float* const prow = s_p + qi * (kPgK + 4);
  for (int kt = 0; kt < ntiles; ++kt) {
    const int t0 = kt * kPgK;
    __syncthreads();                             // the previous tile is consumed (and s_q complete)
    // key and value tile, converted to fp32: tokens past the last key
    // repeat it (masked below)
    for (int i = tid; i < kPgK * c8; i += kPgThreads) {
      const int r = i / c8, c = i % c8;
      const size_t off = (size_t(b) * a.kv_stride + min(t0 + r, nkeys - 1)) * DH + 8 * c;
      const PgRaw8<E> kr = pg_load8<E>(a.k_s, off), vr = pg_load8<E>(a.v_s, off);
      pg_store8<E>(s_k + r * DS + 8 * c, kr);
      pg_store8<E>(s_v + r * DS + 8 * c, vr);
    }
    for (int i = tid; i < kPgK * R; i += kPgThreads) {
      const int r = i / R, j = i % R;
      const size_t idx = ((size_t(b) * a.kv_stride + min(t0 + r, nkeys - 1)) * H + h) * R + j;
      const float zk = pg_elem<E>(a.z_k, idx), zv = pg_elem<E>(a.z_v, idx);
      s_k[r * DS + DH + j] = zk;
      s_v[r * DS + DH + j] = zv;
    }
    __syncthreads();
    // logits of keys j8 + 8u (log2 units); key t is seen iff t <= qpos
    float dot[kPgK / 8];
#pragma unroll
    for (int u = 0; u < kPgK / 8; ++u) dot[u] = 0.f;
#pragma unroll 2
    for (int x = 0; x < D4; x += 4) {
      const float4 qv = ld4(qrow + x);
#pragma unroll
      for (int u = 0; u < kPgK / 8; ++u) {
        const float4 kv = ld4(s_k + (j8 + 8 * u) * DS + x);
        dot[u] = __builtin_fmaf(qv.x, kv.x, dot[u]);
        dot[u] = __builtin_fmaf(qv.y, kv.y, dot[u]);
        dot[u] = __builtin_fmaf(qv.z, kv.z, dot[u]);
        dot[u] = __builtin_fmaf(qv.w, kv.w, dot[u]);
      }
    }
    float sc[kPgK / 8];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < kPgK / 8; ++u) {
      const int t = t0 + j8 + 8 * u;
      sc[u] = (t <= qpos && t < nkeys) ? dot[u] * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, sc[u]);
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    // key 0 is in the first tile and seen by every query, so m is finite from
    // there on; a later tile may hide every key from a query (mx = -inf)
    const float mn = fmaxf(m, mx);
    const float alpha = fast_exp2(m - mn);       // 0 on the first tile
    m = mn;
    l *= alpha;
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      acc[c].x *= alpha; acc[c].y *= alpha; acc[c].z *= alpha; acc[c].w *= alpha;
    }
#pragma unroll
    for (int u = 0; u < kPgK / 8; ++u) {
      const float pe = fast_exp2(sc[u] - m);
      l += pe;
      prow[j8 + 8 * u] = pe;
    }
    __syncthreads();
    for (int k = 0; k < kPgK; k += 4) {
      const float4 pk = ld4(prow + k);
      const float pw[4] = {pk.x, pk.y, pk.z, pk.w};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const float* vrow = s_v + (k + kk) * DS;
        float4 vv[NB];
#pragma unroll
        for (int c = 0; c < NB; ++c) vv[c] = ld4(vrow + vcol[c]);
#pragma unroll
        for (int c = 0; c < NB; ++c) {
          acc[c].x = __builtin_fmaf(pw[kk], vv[c].x, acc[c].x);
          acc[c].y = __builtin_fmaf(pw[kk], vv[c].y, acc[c].y);
          acc[c].z = __builtin_fmaf(pw[kk], vv[c].z, acc[c].z);
          acc[c].w = __builtin_fmaf(pw[kk], vv[c].w, acc[c].w);
        }
      }
    }
  }
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) l += __shfl_xor(l, o);

  // epilogue: O = (O_s + O_z (B^V_h)^T) / l, the augmented row through LDS
  __syncthreads();
  float* const arow = s_k + qi * DS;             // kPgQ rows of the key tile's space
#pragma unroll
  for (int c = 0; c < NB; ++c)
    if (32 * c + 4 * j8 < D4) *reinterpret_cast<float4*>(arow + 32 * c + 4 * j8) = acc[c];
  __syncthreads();
  if (q0 + qi >= L) return;
  const size_t orow = ((size_t(b) * L + q0 + qi) * H + h) * DH;
  const float inv = 1.f / l;
  for (int d = j8; d < DH; d += 8) {
    float o = arow[d];
    for (int j = 0; j < R; ++j) o = __builtin_fmaf(arow[DH + j], pg_elem<E>(a.b_v, (size_t(h) * DH + d) * R + j), o);
    static_cast<typename E::T*>(a.out)[orow + d] = E::from_f32(o * inv);
  }
}

bool prefill_generic_supported(int dtype, int head_dim, int rank, int heads) {
  return (dtype == 0 || dtype == 1) && head_dim >= 16 && head_dim <= 128 && head_dim % 8 == 0 && rank >= 0 &&
         rank <= kPrefillGenericMaxRank && heads >= 1 && heads <= 65535;
}

template <class E, int NB>
static bool pg_launch_one(int nb, dim3 grid, size_t lds, hipStream_t st, const PrefillArgs& a, int nqb) {
  if (nb != NB) return false;
  hipLaunchKernelGGL((prefill_generic_kernel<E, NB>), grid, dim3(kPgThreads), lds, st, a, nqb);
  return true;
}

template <class E, int... NB>
static hipError_t pg_launch(int nb, dim3 grid, size_t lds, hipStream_t st, const PrefillArgs& a, int nqb,
                            std::integer_sequence<int, NB...>) {
  const bool done = (pg_launch_one<E, NB + 1>(nb, grid, lds, st, a, nqb) || ...);
  return done ? hipGetLastError() : hipErrorInvalidValue;
}

template <class E, int... NB>
static hipError_t pg_prepare(std::integer_sequence<int, NB...>) {
  const int lds = prefill_generic_lds_floats(kPgMaxDims) * int(sizeof(float));
  hipError_t e = hipSuccess;
  ((e = e == hipSuccess ? allow_dynamic_lds<&prefill_generic_kernel<E, NB + 1>>(lds) : e), ...);
  return e;
}

hipError_t launch_prefill_generic(int dtype, const PrefillArgs& a, hipStream_t st) {
  // the training forward's log-sum-exp output is the MFMA kernel's only
  if (!prefill_generic_supported(dtype, a.head_dim, a.rank, a.heads) || a.batch > 65535 || a.lse)
    return hipErrorInvalidValue;
  const int nqb = (a.seq_len + kPgQ - 1) / kPgQ;
  const int dims = a.head_dim + a.rank, nb = (((dims + 3) & ~3) + 31) / 32;
  const size_t lds = size_t(prefill_generic_lds_floats(dims)) * sizeof(float);
  const dim3 grid{unsigned(nqb), unsigned(a.heads), unsigned(a.batch)};
  const hipError_t e = prefill_generic_prepare();   // the limit is set once, for the largest shape
  if (e != hipSuccess) return e;
  const auto blocks = std::make_integer_sequence<int, kPgBlocks>{};
  return dtype == 1 ? pg_launch<BF16>(nb, grid, lds, st, a, nqb, blocks) : pg_launch<F32>(nb, grid, lds, st, a, nqb, blocks);
}

hipError_t prefill_generic_prepare() {
  const auto blocks = std::make_integer_sequence<int, kPgBlocks>{};
  const hipError_t e = pg_prepare<BF16>(blocks);
  return e == hipSuccess ? pg_prepare<F32>(blocks) : e;
}

}  // namespace lrkv
