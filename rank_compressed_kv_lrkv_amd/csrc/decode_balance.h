// Length-balanced split-K partition of a decode launch, computed on the device.
//
// The host knows only an upper bound on the sequence lengths; the lengths
// themselves live in device memory.  A ragged batch split into fixed-size
// partitions sized from that bound leaves most compute units idle (a batch
// of 16 sequences of 1K..64K tokens split 4096 tokens at a time gives about
// 115 partitions for 256 compute units).  Instead, every workgroup of the
// scan reads all lengths and derives the same partition:
//   - the item size u is the smallest multiple of kBalStep, at least
//     kBalMinItem, for which the items, ceil(len_b / u) per sequence,
//     number at most max(cap, sequences with tokens);
//   - items are numbered sequence by sequence: item P_b + s of sequence b
//     covers its tokens [s u, min((s+1) u, len_b)).
// With cap = the number of resident scan workgroups, every item runs in one
// round, and no item is longer than u (the uniform 8K-context batch of 32
// sequences on 256 compute units gets u = 1024, exactly the fixed split).
// The scan records each sequence's first item and the item size in the
// workspace for the merge.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lrkv {

constexpr int kBalMaxBatch = 256;                // sequences a balanced launch takes (kBalLanes per lane)
constexpr int kBalLanes = kBalMaxBatch / 64;
constexpr int kBalStep = 32;                     // item sizes are multiples of one tile
constexpr int kBalMinItem = 128;                 // at least one tile per wave of a scan workgroup
constexpr int kBalMaxLen = 1 << 24;              // lengths a balanced launch takes (exact float arithmetic)

struct BalLens {
  int v[kBalLanes];                              // lane l: lengths of sequences l, l + 64, ...
  int chunks;                                    // chunks of 64 sequences in use (uniform)
};

// Inclusive prefix sum over the wave: DPP shifts within each row of 16
// lanes, then the totals of the rows below added through readlane.
__device__ __forceinline__ int bal_wave_scan(int x, int lane) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1 (lanes past the row read 0)
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = lane >> 4;
  return x + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}
__device__ __forceinline__ int bal_wave_sum(int x, int lane) {
  return __builtin_amdgcn_readlane(bal_wave_scan(x, lane), 63);
}

// ceil(a / u) for 0 <= a < 2^24 (exact in float) and 1 <= u < 2^24, exact:
// the float estimate is within one of the quotient and is corrected by
// integer comparisons.
__device__ __forceinline__ int bal_ceil_div(int a, int u, float inv_u) {
  int n = int(__builtin_ceilf(float(a) * inv_u));
  n -= (n > 0 && (n - 1) * u >= a);
  n += (n * u < a);
  n -= (n > 0 && (n - 1) * u >= a);
  return n;
}

__device__ __forceinline__ BalLens bal_load(const int32_t* seq_lens, int batch, int max_len, int lane) {
  BalLens L;
  L.chunks = (batch + 63) / 64;
#pragma unroll
  for (int k = 0; k < kBalLanes; ++k) {
    const int b = lane + 64 * k;
    int v = b < batch ? seq_lens[b] : 0;
    L.v[k] = v < 0 ? 0 : (v > max_len ? max_len : v);
  }
  return L;
}

// Items for item size u (uniform).
__device__ __forceinline__ int bal_count(const BalLens& L, int u, int lane) {
  const float inv = 1.f / float(u);
  int n = 0;
#pragma unroll
  for (int k = 0; k < kBalLanes; ++k)
    if (k < L.chunks) n += bal_ceil_div(L.v[k], u, inv);
  return bal_wave_sum(n, lane);
}

// The item size for this launch (0 if every length is 0); max_len bounds
// every length.  With T tokens over nz non-empty sequences and limit items
// allowed, count(u) >= T/u and count(u) <= T/u + nz, so the answer lies
// between ceil(T/limit) and ceil(T/(limit - nz)) (or max_len when
// limit == nz), a range of a few tile multiples searched by bisection.
__device__ __forceinline__ int bal_item_size(const BalLens& L, int max_len, int cap, int lane) {
  int nz = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < kBalLanes; ++k) {
    nz += L.v[k] > 0;
    tot += L.v[k];                               // < 2^32 as unsigned: at most 256 lengths below 2^24
  }
  nz = bal_wave_sum(nz, lane);
  if (nz == 0) return 0;
  const unsigned T = unsigned(bal_wave_sum(tot, lane));
  const int limit = max(cap, nz);
  const int top = (max_len + kBalStep - 1) / kBalStep;             // u = max_len qualifies
  const int floor_u = kBalMinItem / kBalStep;
  int lo = max(floor_u, int((T + unsigned(limit) - 1) / unsigned(limit) + kBalStep - 1) / kBalStep);
  int hi = limit > nz ? int((T + unsigned(limit - nz) - 1) / unsigned(limit - nz) + kBalStep - 1) / kBalStep : top;
  hi = max(floor_u, min(hi, top));
  lo = min(lo, hi);
  // smallest u = kBalStep * x in [lo, hi] with count(u) <= limit (hi qualifies)
  while (lo < hi) {
    const int mid = (lo + hi) / 2;
    if (bal_count(L, mid * kBalStep, lane) <= limit) hi = mid; else lo = mid + 1;
  }
  return lo * kBalStep;
}

// The sequence and token range of item i (false if i is past the last item).
__device__ __forceinline__ bool bal_item(const BalLens& L, int u, int i, int lane, int* b_out, int* lo, int* hi) {
  const float inv = 1.f / float(u);
  int carry = 0;
#pragma unroll
  for (int k = 0; k < kBalLanes; ++k) {
    if (k >= L.chunks) break;
    const int n = bal_ceil_div(L.v[k], u, inv);
    const int incl = bal_wave_scan(n, lane);
    const int excl = incl - n;
    const uint64_t hit = __builtin_amdgcn_ballot_w64(carry + excl <= i && i < carry + incl);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      const int s = i - carry - __builtin_amdgcn_readlane(excl, src);
      const int len = __builtin_amdgcn_readlane(L.v[k], src);
      *b_out = 64 * k + src;
      *lo = s * u;
      *hi = min(len, (s + 1) * u);
      return true;
    }
    carry += __builtin_amdgcn_readlane(incl, 63);
  }
  return false;
}

// The same partition in closed form when every length is the same L > 0
// (the common uniform batch): with k = limit / batch items allowed per
// sequence, the smallest admissible u is ceil(L / k) rounded up to the item
// step (and at least kBalMinItem), and item i is sequence i / ceil(L / u),
// piece i % ceil(L / u).  Returns false, touching nothing, if the lengths
// differ or are 0 (the general path applies).
__device__ __forceinline__ bool bal_uniform(const BalLens& L, int batch, int cap, int i, int lane, int* u_out,
                                            int* b_out, int* lo, int* hi, bool* valid) {
  const int l0 = __builtin_amdgcn_readfirstlane(L.v[0]);      // sequence 0
  int diff = 0;
#pragma unroll
  for (int k = 0; k < kBalLanes; ++k)
    if (k < L.chunks) diff += (lane + 64 * k < batch && L.v[k] != l0);
  if (l0 <= 0 || bal_wave_sum(diff, lane) != 0) return false;
  const int per_max = max(cap, batch) / batch;                 // items one sequence may have
  int u = (l0 + per_max - 1) / per_max;
  u = max(kBalMinItem, (u + kBalStep - 1) / kBalStep * kBalStep);
  const int per = (l0 + u - 1) / u;                            // items per sequence
  *u_out = u;
  *valid = i < batch * per;
  if (*valid) {
    *b_out = i / per;
    const int s = i - *b_out * per;
    *lo = s * u;
    *hi = min(l0, (s + 1) * u);
  }
  return true;
}

}  // namespace lrkv
