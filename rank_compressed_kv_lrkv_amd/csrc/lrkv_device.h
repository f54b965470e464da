// Device helpers for the LRKV kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lrkv {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
// Native 128-bit vector: register-resident copies of it never go through memory.
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }

// Round to nearest even; gfx950 has a native packed convert for this.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x) { return uint16_t(pack_bf16x2(x, 0.f) & 0xffffu); }

// Element traits.  A "pair" is two consecutive elements used as one operand
// of a 2-wide dot product; for bf16 that is one 32-bit register feeding
// v_dot2_f32_bf16, for fp32 a float2 evaluated as two FMAs.
struct F32 {
  using T = float;
  using Pair = float2;
  static constexpr int kBytes = 4;
  __device__ static __forceinline__ float dot2(float acc, Pair a, Pair b) {
    return __builtin_fmaf(a.y, b.y, __builtin_fmaf(a.x, b.x, acc));
  }
  __device__ static __forceinline__ Pair make_pair(float lo, float hi) { return make_float2(lo, hi); }
  __device__ static __forceinline__ float lo(Pair p) { return p.x; }
  __device__ static __forceinline__ float hi(Pair p) { return p.y; }
  __device__ static __forceinline__ float to_f32(T x) { return x; }
  __device__ static __forceinline__ T from_f32(float x) { return x; }
  // Interleave element i of a and element i of b.
  __device__ static __forceinline__ Pair zip(T a, T b) { return make_float2(a, b); }
};

struct BF16 {
  using T = uint16_t;
  using Pair = uint32_t;
  static constexpr int kBytes = 2;
  __device__ static __forceinline__ float dot2(float acc, Pair a, Pair b) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), acc, false);
  }
  __device__ static __forceinline__ Pair make_pair(float lo, float hi) { return pack_bf16x2(lo, hi); }
  __device__ static __forceinline__ float lo(Pair p) { return __uint_as_float(p << 16); }
  __device__ static __forceinline__ float hi(Pair p) { return __uint_as_float(p & 0xffff0000u); }
  __device__ static __forceinline__ float to_f32(T x) { return bf16_to_f32(x); }
  __device__ static __forceinline__ T from_f32(float x) { return f32_to_bf16(x); }
  __device__ static __forceinline__ Pair zip(T a, T b) { return uint32_t(a) | (uint32_t(b) << 16); }
};

// Pair i (compile-time) of registers viewed as consecutive 32-bit words.
template <class E>
__device__ __forceinline__ typename E::Pair pair_at(const uint32_t* w, int i);
template <>
__device__ __forceinline__ BF16::Pair pair_at<BF16>(const uint32_t* w, int i) { return w[i]; }
template <>
__device__ __forceinline__ F32::Pair pair_at<F32>(const uint32_t* w, int i) {
  return make_float2(__uint_as_float(w[2 * i]), __uint_as_float(w[2 * i + 1]));
}
// Element i (compile-time) of registers viewed as consecutive 32-bit words.
template <class E>
__device__ __forceinline__ typename E::T elem_at(const uint32_t* w, int i);
template <>
__device__ __forceinline__ BF16::T elem_at<BF16>(const uint32_t* w, int i) {
  return uint16_t((i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xffffu));
}
template <>
__device__ __forceinline__ F32::T elem_at<F32>(const uint32_t* w, int i) { return __uint_as_float(w[i]); }

// Load NB bytes (NB == 2 or a multiple of 4) into 32-bit words w[0..ceil(NB/4)),
// using 16-, 8- and 4-byte accesses; p must be aligned to min(NB, 16).
template <int NB>
__device__ __forceinline__ void load_words(uint32_t* w, const void* p) {
  if constexpr (NB == 2) {
    w[0] = *reinterpret_cast<const uint16_t*>(p);
  } else {
    static_assert(NB % 4 == 0, "load size");
    const unsigned char* c = static_cast<const unsigned char*>(p);
    int o = 0;
#pragma unroll
    for (; o + 16 <= NB; o += 16) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(c + o);
      w[o / 4] = v.x; w[o / 4 + 1] = v.y; w[o / 4 + 2] = v.z; w[o / 4 + 3] = v.w;
    }
    if constexpr (NB % 16 >= 8) {
      constexpr int o8 = NB / 16 * 16;
      const uint2 v = *reinterpret_cast<const uint2*>(c + o8);
      w[o8 / 4] = v.x; w[o8 / 4 + 1] = v.y;
    }
    if constexpr (NB % 8 == 4) {
      constexpr int o4 = NB / 8 * 8;
      w[o4 / 4] = *reinterpret_cast<const uint32_t*>(c + o4);
    }
  }
}

// Raw buffer resource over `bytes` bytes at `base` (gfx9 descriptor word 3:
// no swizzle, no format conversion).  Loads through it take a per-lane byte
// offset plus a uniform one; offsets at or past `bytes` read zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_resource(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), short(0), int(bytes), 0x00020000);
}

// Cache-policy operand of a buffer load.  kStream sets the gfx950
// non-temporal bit: the data is read once, so the caches treat its lines as
// streaming (evicted first, not kept for reuse).  The cache scans use it for
// every load of cache rows and latents; on the 671 MB decode scan it takes
// the sustained read rate from about 5.1 to 6.0 TB/s.
constexpr int kCached = 0;
constexpr int kStream = 2;

// Load NB bytes (2 or a multiple of 4) at byte voff + soff of a buffer
// resource into 32-bit words w[0..ceil(NB/4)), using 16-, 8-, 4- and 2-byte
// accesses; the offset must be aligned to min(NB, 16).
template <int NB, int POLICY = kCached>
__device__ __forceinline__ void buffer_words(uint32_t* w, __amdgpu_buffer_rsrc_t res, uint32_t voff, uint32_t soff) {
  if constexpr (NB == 2) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b16(res, int(voff), int(soff), POLICY);
    return;
  }
  static_assert(NB == 2 || NB % 4 == 0, "load size");
  int o = 0;
#pragma unroll
  for (; o + 16 <= NB; o += 16) {
    const u32x4 v =
        __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(res, int(voff + o), int(soff), POLICY));
    w[o / 4] = v.x; w[o / 4 + 1] = v.y; w[o / 4 + 2] = v.z; w[o / 4 + 3] = v.w;
  }
  if constexpr (NB % 16 >= 8) {
    constexpr int o8 = NB / 16 * 16;
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(res, int(voff + o8), int(soff), POLICY);
    w[o8 / 4] = v[0]; w[o8 / 4 + 1] = v[1];
  }
  if constexpr (NB % 8 == 4) {
    constexpr int o4 = NB / 8 * 8;
    w[o4 / 4] = __builtin_amdgcn_raw_buffer_load_b32(res, int(voff + o4), int(soff), POLICY);
  }
}

// Pair (element i of word array a, element i of word array b), i compile-time.
template <class E>
__device__ __forceinline__ typename E::Pair zip_at(const uint32_t* a, const uint32_t* b, int i);
template <>
__device__ __forceinline__ BF16::Pair zip_at<BF16>(const uint32_t* a, const uint32_t* b, int i) {
  return (i & 1) ? __builtin_amdgcn_perm(b[i >> 1], a[i >> 1], 0x07060302u)
                 : __builtin_amdgcn_perm(b[i >> 1], a[i >> 1], 0x05040100u);
}
template <>
__device__ __forceinline__ F32::Pair zip_at<F32>(const uint32_t* a, const uint32_t* b, int i) {
  return make_float2(__uint_as_float(a[i]), __uint_as_float(b[i]));
}

// Byte-sized vector type for loads of NB bytes (NB in {2, 4, 8, 16}).
template <int NB> struct VecBytes;
template <> struct VecBytes<2> { using V = uint16_t; };
template <> struct VecBytes<4> { using V = uint32_t; };
template <> struct VecBytes<8> { using V = uint2; };
template <> struct VecBytes<16> { using V = uint4; };

// Copy NB bytes (a multiple of 8, or 2/4) from p to dst using the widest
// aligned accesses; p and dst must be aligned to min(NB, 16).
template <int NB>
__device__ __forceinline__ void copy_bytes(void* dst, const void* p) {
  if constexpr (NB >= 16) {
#pragma unroll
    for (int i = 0; i < NB / 16; ++i)
      reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(p)[i];
  } else {
    *reinterpret_cast<typename VecBytes<NB>::V*>(dst) = *reinterpret_cast<const typename VecBytes<NB>::V*>(p);
  }
}

template <int NB>
__device__ __forceinline__ void zero_bytes(void* dst) {
  if constexpr (NB >= 16) {
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) reinterpret_cast<uint4*>(dst)[i] = make_uint4(0, 0, 0, 0);
  } else {
    *reinterpret_cast<typename VecBytes<NB>::V*>(dst) = typename VecBytes<NB>::V{};
  }
}

// ---------------------------------------------------------------------------
// Reductions inside aligned groups of G lanes (G in {2, 4, 8}) with DPP:
// quad_perm swaps for distances 1 and 2, row_half_mirror to pair the two
// quads of an 8-lane group.  After the calls every lane of the group holds
// the group result.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

constexpr int kDppSwap1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppSwap2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within each 8
constexpr int kDppRev4 = 0x1B;        // quad_perm [3,2,1,0]
constexpr int kDppEven = 0xA0;        // quad_perm [0,0,2,2]: value of the even lane of each pair
constexpr int kDppOdd = 0xF5;         // quad_perm [1,1,3,3]: value of the odd lane of each pair

template <int G>
__device__ __forceinline__ float group_max(float v) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
  if constexpr (G >= 2) v = fmaxf(v, dpp_mov<kDppSwap1>(v));
  if constexpr (G >= 4) v = fmaxf(v, dpp_mov<kDppSwap2>(v));
  if constexpr (G >= 8) v = fmaxf(v, dpp_mov<kDppHalfMirror>(v));
  return v;
}

template <int G>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
  if constexpr (G >= 2) v += dpp_mov<kDppSwap1>(v);
  if constexpr (G >= 4) v += dpp_mov<kDppSwap2>(v);
  if constexpr (G >= 8) v += dpp_mov<kDppHalfMirror>(v);
  return v;
}

// Value held by lane `src` (0 <= src < G) of this lane's aligned G-group,
// through the LDS crossbar swizzle (bit-mask mode, no memory traffic).
template <int G, int SRC>
__device__ __forceinline__ uint32_t group_bcast(uint32_t v) {
  constexpr int and_mask = 0x1F & ~(G - 1);
  constexpr int pattern = and_mask | (SRC << 5);
  return uint32_t(__builtin_amdgcn_ds_swizzle(int(v), pattern));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// bf16 MFMA, LDS transpose reads and global-to-LDS transfers (gfx950).
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;

// D = A.B + C with A 32x16, B 16x32 (bf16), C/D 32x32 fp32.  Lane l holds
// A row l%32 and B column l%32 at k-slots 8(l/32)..8(l/32)+7, and D column
// l%32 at rows 8(i/4) + 4(l/32) + i%4 in element i.
__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8_t, v); }

// LDS transpose read of 4 bf16.  Within each group of 16 lanes, lane 4a+c
// receives element c of the 8-byte rows addressed by lanes 4k+a, k = 0..3
// (element k of the result from lane 4k+a).  With lane 4k+a addressing token
// k at features 4a..4a+3, lane 4a+c gets feature 4a+c of tokens 0..3: a
// column of a row-major tile.
__device__ __forceinline__ uint2 lds_read_tr16(const unsigned char* p) {
  const i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(p));
  return __builtin_bit_cast(uint2, r);
}

// 16 bytes per lane from global memory straight into LDS through a buffer
// resource: lane i reads the resource at byte voff + soff (soff uniform) and
// writes bytes [16i, 16i+16) after `lds` (wave-uniform).
template <int POLICY = kCached>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t res, uint32_t voff, uint32_t soff, unsigned char* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(res, (__attribute__((address_space(3))) void*)(lds), 16, int(voff),
                                           int(soff), 0, POLICY);
}

// Swizzle of unpadded LDS tiles: 16-byte chunk ch of row r sits at position
// ch ^ lds_swz(r, chunks).  gfx950 LDS has 64 banks of 4 bytes and serves
// 16-byte reads 16 lanes per cycle, 8-byte and transpose reads 32 lanes per
// cycle.  The swizzle is the bit-reversed low 4 bits of the row index, masked
// to the chunks per row: a bijection on every 8 (or 16) consecutive rows, so
// 16-byte reads of one chunk from 16 rows are conflict-free, and its bits 1-2
// follow r&3, so a transpose read's 4 rows x 2 chunks land on 8 distinct
// positions.
__device__ __forceinline__ int lds_swz(int row, int chunks) {
  const int r = row & 15;
  return (((r & 1) << 3) | ((r & 2) << 1) | ((r & 4) >> 1) | ((r & 8) >> 3)) & (chunks - 1);
}

}  // namespace lrkv
