// C ABI of liblrkv: host-side validation, planning and dispatch.
// Every check runs before anything is enqueued; a call that returns an error
// has launched nothing.  No memory is allocated and nothing synchronises.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>

#include "../../include/lrkv.h"
#include "decode_balance.h"
#include "lrkv_internal.h"

#include <algorithm>

namespace {

using lrkv::DecodePlan;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
int elem_bytes(int32_t dtype) { return dtype == LRKV_BF16 ? 2 : 4; }

// Compute units of the current device, queried once per device.
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

lrkv_status check_sizes(int32_t dtype, int32_t batch, int32_t heads, int32_t head_dim, int32_t rank,
                        int64_t capacity) {
  if (dtype != LRKV_F32 && dtype != LRKV_BF16) return LRKV_ERR_DTYPE;
  if (batch < 0 || heads < 1 || head_dim < 1 || rank < 0 || capacity < 1) return LRKV_ERR_SHAPE;
  if (capacity > INT32_MAX) return LRKV_ERR_SHAPE;
  // shared rows are copied and staged in 16-byte chunks; latents may have any
  // rank (each kernel states the ranks it takes)
  const int es = elem_bytes(dtype);
  if ((int64_t(head_dim) * es) % 16 != 0) return LRKV_ERR_SHAPE;
  if (rank > INT32_MAX / std::max(heads, 1) / 4) return LRKV_ERR_SHAPE;
  return LRKV_OK;
}

// engine: 0 = the default for the shape, 1 = the vector-ALU scan
// (decode_split_kernel), 2 = the MFMA scan (decode_mfma_kernel), 3 = the
// any-rank scan (decode_generic_kernel), 4 = the any-rank MFMA scan
// (decode_mfma_any_kernel).  The default takes the MFMA scan where it
// applies, else the vector-ALU scan, else the any-rank MFMA scan where it
// is preferred, else the any-rank scan.
lrkv_status plan_decode(int32_t dtype, int32_t batch, int32_t heads, int32_t head_dim, int32_t rank,
                        int64_t capacity, int64_t max_len, int32_t split_tokens, DecodePlan* pl, int32_t engine = 0) {
  lrkv_status st = check_sizes(dtype, batch, heads, head_dim, rank, capacity);
  if (st != LRKV_OK) return st;
  if (engine < 0 || engine > 4) return LRKV_ERR_SHAPE;
  const bool tuned = lrkv::decode_supported(dtype, head_dim, rank, heads);
  const bool any = lrkv::decode_generic_supported(dtype, head_dim, rank, heads);
  const bool any_mfma = lrkv::decode_mfma_any_supported(dtype, head_dim, rank, heads);
  if (engine == 1 && !tuned) return LRKV_ERR_SHAPE;
  if (engine == 2 && !lrkv::decode_mfma_supported(dtype, head_dim, rank, heads)) return LRKV_ERR_SHAPE;
  if (engine == 3 && !any) return LRKV_ERR_SHAPE;
  if (engine == 4 && !any_mfma) return LRKV_ERR_SHAPE;
  if (engine == 0 && !tuned && !any) return LRKV_ERR_SHAPE;
  if (max_len < 0 || split_tokens < 0) return LRKV_ERR_SHAPE;
  if (max_len > capacity) return LRKV_ERR_CAPACITY;
  if (split_tokens != 0 && split_tokens % lrkv::kDecodeTile != 0) return LRKV_ERR_SHAPE;

  pl->batch = batch; pl->heads = heads; pl->head_dim = head_dim; pl->rank = rank; pl->dtype = dtype;
  pl->capacity = capacity; pl->max_len = int(max_len);
  const bool any_mfma_default = lrkv::decode_mfma_any_preferred(dtype, head_dim, rank, heads);
  pl->mfma_any = engine == 4 || (engine == 0 && !tuned && any_mfma_default);
  pl->generic = engine == 3 || (engine == 0 && !tuned && !any_mfma_default);
  pl->mfma = !pl->generic && !pl->mfma_any && engine != 1 &&
             lrkv::decode_mfma_supported(dtype, head_dim, rank, heads);
  pl->group = (rank == 4 || heads > 32) ? 4 : 8;
  int hp = 1;
  while (hp < heads) hp <<= 1;
  pl->heads_pow2 = hp;
  pl->slots = (pl->mfma || pl->generic || pl->mfma_any) ? 1 : lrkv::kDecodeThreads / (hp * pl->group);
  if (pl->slots < 1) return LRKV_ERR_SHAPE;

  const int tile = lrkv::kDecodeTile;
  int split = split_tokens;
  if (split == 0) {
    // Workgroups over the whole batch: about two per compute unit for the
    // vector-ALU scan; for the MFMA scan (one resident workgroup per compute
    // unit) about one, in whole 32-token tiles per wave.
    // The any-rank scan runs one workgroup per group of 256 / G heads (G
    // lanes per head) with up to 64 KB of LDS, two resident per compute
    // unit: about four per compute unit (two rounds).  The any-rank MFMA
    // scan runs one workgroup per group of 32 heads, one resident per
    // compute unit: about one per compute unit, in whole 32-token tiles per
    // wave.
    const int64_t gh = 256 / lrkv::generic_lanes_per_head(heads, head_dim);
    const int64_t groups = pl->mfma ? heads / 32 : pl->mfma_any ? (heads + 31) / 32 : pl->generic ? (heads + gh - 1) / gh : 1;
    const int64_t total = int64_t(batch) * max_len * groups;
    const int64_t target = (pl->mfma || pl->mfma_any ? 1 : pl->generic ? 4 : 2) * int64_t(device_cu_count());
    const int64_t unit = (pl->mfma || pl->mfma_any) ? 2 * tile : tile;
    int64_t s = (total + target - 1) / (target > 0 ? target : 1);
    s = (s + unit - 1) / unit * unit;
    // at least two tiles per split: a small cache split one tile at a time
    // leaves the merge more partial states than the scan saves time (the
    // 8 x 2048-token bf16 batch: 20.3 us per step at 64 tokens, 15.5 at 128)
    if (s < 2 * tile) s = 2 * tile;
    const int64_t cap = (max_len + unit - 1) / unit * unit;
    if (s > cap) s = cap < unit ? unit : cap;
    split = int(s);
  }
  // Default split of the MFMA scan over a batch the device-side partition
  // takes: items balanced over the actual lengths (up to cap + batch items).
  pl->balanced = pl->mfma && split_tokens == 0 && batch <= lrkv::kBalMaxBatch && max_len < lrkv::kBalMaxLen;
  pl->bal_cap = device_cu_count();
  // The kernels address one split's rows and latents through 32-bit buffer
  // offsets (a balanced item is at most max_len tokens), with the top 1 KB of
  // the offset range left for reads meant to fall outside every range.
  const int64_t es = dtype == 1 ? 2 : 4;
  const int64_t span = pl->balanced ? std::max<int64_t>(max_len, 1) : split;
  if (span * std::max<int64_t>(int64_t(head_dim), int64_t(heads) * rank) * es >= (int64_t(1) << 32) - 1024)
    return LRKV_ERR_SHAPE;
  // the any-rank MFMA scan also forms offsets of up to 256 tokens past its
  // split (zero reads of the tiles after the last)
  if (pl->mfma_any && (span + 256) * int64_t(heads) * rank * es >= (int64_t(1) << 32)) return LRKV_ERR_SHAPE;
  pl->split_tokens = split;
  if (pl->balanced) {
    // the partition makes at most max(cap, non-empty sequences) items: no
    // workgroup beyond those (one more round of empty workgroups would trail
    // the scan)
    pl->n_splits = max_len > 0 ? std::max(pl->bal_cap, int(batch)) : 0;
    pl->partials = pl->n_splits;
  } else {
    pl->n_splits = int((max_len + split - 1) / split);
    pl->partials = pl->n_splits * pl->slots;
  }
  const size_t states = (pl->balanced ? size_t(1) : size_t(batch)) * size_t(pl->partials) * size_t(heads);
  pl->ws_ml_bytes = (states * 2 * sizeof(float) + 255) / 256 * 256;
  pl->ws_acc_bytes = (states * size_t(head_dim + rank) * sizeof(float) + 255) / 256 * 256;
  pl->ws_meta_bytes = pl->balanced ? (size_t(batch + 1) * sizeof(int) + 255) / 256 * 256 : 0;
  pl->ws_qt_bytes = pl->mfma_any ? (size_t(batch) * heads * rank * sizeof(float) + 255) / 256 * 256 : 0;
  return LRKV_OK;
}

size_t workspace_bytes_of(const DecodePlan& pl) {
  return pl.ws_ml_bytes + pl.ws_acc_bytes + pl.ws_meta_bytes + pl.ws_qt_bytes;
}

// Device scratch of lrkv_decode_noalloc: the split-K partial states of a
// decode, for callers that cannot allocate.  One copy per device, alive until
// the process ends; every lrkv_decode_noalloc call on a device writes its
// copy, so calls that overlap on one device race.  Nothing in it has to
// start at zero: the scan writes every state the merge reads.
constexpr size_t kScratchBytes = size_t(16) << 20;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

// Device address of the current device's copy of `scratch`, looked up once
// per device with that device current.  In host code the array's name is
// only a stand-in for the symbol, never a device address.
hipError_t scratch_address(void** out) {
  static std::atomic<void*> addr[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u)) return hipErrorInvalidSymbol;
    addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* lrkv_status_string(int32_t s) {
  switch (s) {
    case LRKV_OK: return "ok";
    case LRKV_ERR_NULL: return "null pointer";
    case LRKV_ERR_SHAPE: return "invalid or unsupported shape";
    case LRKV_ERR_DTYPE: return "invalid dtype";
    case LRKV_ERR_ALIGN: return "pointer not 16-byte aligned";
    case LRKV_ERR_CAPACITY: return "length exceeds cache capacity";
    case LRKV_ERR_WORKSPACE: return "workspace missing or too small";
    case LRKV_ERR_DEVICE: return "HIP runtime or launch failure";
    case LRKV_ERR_SCRATCH: return "request exceeds the library's fixed device scratch";
    default: return "unknown status";
  }
}

lrkv_status lrkv_init(void) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LRKV_ERR_DEVICE;
  (void)device_cu_count();
  for (hipError_t (*prep)() : {lrkv::decode_mfma_prepare, lrkv::decode_mfma_any_prepare, lrkv::prefill_prepare,
                               lrkv::prefill_wide_prepare, lrkv::prefill_generic_prepare, lrkv::project_prepare,
                               lrkv::train_prepare})
    if (prep() != hipSuccess) return LRKV_ERR_DEVICE;
  return LRKV_OK;
}

int64_t lrkv_cache_elems_per_token(int32_t num_heads, int32_t head_dim, int32_t rank) {
  if (num_heads < 1 || head_dim < 1 || rank < 0) return -1;
  return 2 * (int64_t(head_dim) + int64_t(num_heads) * int64_t(rank));
}

const char* lrkv_decode_scan_kernel(int32_t dtype, int32_t num_heads, int32_t head_dim, int32_t rank) {
  if (check_sizes(dtype, 1, num_heads, head_dim, rank, 1) != LRKV_OK) return nullptr;
  if (!lrkv::decode_supported(dtype, head_dim, rank, num_heads)) {
    if (lrkv::decode_mfma_any_preferred(dtype, head_dim, rank, num_heads)) return "decode_mfma_any_kernel";
    return lrkv::decode_generic_supported(dtype, head_dim, rank, num_heads) ? "decode_generic_kernel" : nullptr;
  }
  return lrkv::decode_mfma_supported(dtype, head_dim, rank, num_heads) ? "decode_mfma_kernel" : "decode_split_kernel";
}

lrkv_status lrkv_decode_workspace_size(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim,
                                       int32_t rank, int64_t capacity, int64_t max_len, int32_t split_tokens,
                                       size_t* bytes) {
  if (!bytes) return LRKV_ERR_NULL;
  DecodePlan pl;
  const lrkv_status st = plan_decode(dtype, batch, num_heads, head_dim, rank, capacity, max_len, split_tokens, &pl);
  if (st != LRKV_OK) return st;
  *bytes = workspace_bytes_of(pl);
  return LRKV_OK;
}

lrkv_status lrkv_decode_workspace_size_ex(int32_t engine, int32_t dtype, int32_t batch, int32_t num_heads,
                                          int32_t head_dim, int32_t rank, int64_t capacity, int64_t max_len,
                                          int32_t split_tokens, size_t* bytes) {
  if (!bytes) return LRKV_ERR_NULL;
  DecodePlan pl;
  const lrkv_status st =
      plan_decode(dtype, batch, num_heads, head_dim, rank, capacity, max_len, split_tokens, &pl, engine);
  if (st != LRKV_OK) return st;
  *bytes = workspace_bytes_of(pl);
  return LRKV_OK;
}

static lrkv_status decode_phases(int phase, int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim,
                                 int32_t rank, int64_t capacity, const void* k_shared, const void* v_shared,
                                 const void* z_k, const void* z_v, const int32_t* seq_lens, int64_t max_len,
                                 const void* q, const void* b_k, const void* b_v, float scale, int32_t split_tokens,
                                 void* out, void* workspace, size_t workspace_bytes, void* stream,
                                 int32_t engine = 0) {
  if (phase < 1 || phase > 3) return LRKV_ERR_SHAPE;
  DecodePlan pl;
  const lrkv_status st =
      plan_decode(dtype, batch, num_heads, head_dim, rank, capacity, max_len, split_tokens, &pl, engine);
  if (st != LRKV_OK) return st;
  if (batch == 0) return LRKV_OK;
  const bool scan = phase & 1, combine = phase & 2;
  if (!seq_lens) return LRKV_ERR_NULL;
  if (scan && (!k_shared || !v_shared || !q)) return LRKV_ERR_NULL;
  if (scan && rank > 0 && (!z_k || !z_v || !b_k)) return LRKV_ERR_NULL;
  if (combine && (!out || (rank > 0 && !b_v))) return LRKV_ERR_NULL;
  const size_t need = workspace_bytes_of(pl);
  if (!workspace || workspace_bytes < need) return LRKV_ERR_WORKSPACE;
  if (!aligned16(workspace) || !aligned4(seq_lens)) return LRKV_ERR_ALIGN;
  if (scan && (!aligned16(k_shared) || !aligned16(v_shared) || !aligned16(q))) return LRKV_ERR_ALIGN;
  if (scan && rank > 0 && (!aligned16(z_k) || !aligned16(z_v) || !aligned16(b_k))) return LRKV_ERR_ALIGN;
  if (combine && (!aligned16(out) || (rank > 0 && !aligned16(b_v)))) return LRKV_ERR_ALIGN;

  const float sc = (scale > 0.f && std::isfinite(scale)) ? scale : 1.0f / std::sqrt(float(head_dim));
  lrkv::DecodeArgs a;
  a.k_s = k_shared; a.v_s = v_shared; a.z_k = z_k; a.z_v = z_v;
  a.seq_lens = seq_lens; a.q = q; a.b_k = b_k; a.b_v = b_v;
  a.scale_log2 = sc * 1.4426950408889634f;
  a.out = out;
  a.ws_ml = static_cast<float*>(workspace);
  a.ws_acc = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + pl.ws_ml_bytes);
  a.ws_meta = reinterpret_cast<int*>(static_cast<unsigned char*>(workspace) + pl.ws_ml_bytes + pl.ws_acc_bytes);
  a.ws_qt = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + pl.ws_ml_bytes + pl.ws_acc_bytes +
                                     pl.ws_meta_bytes);
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const hipError_t e = pl.mfma_any ? lrkv::launch_decode_mfma_any(pl, a, phase, hs) : lrkv::launch_decode(pl, a, phase, hs);
  return e == hipSuccess ? LRKV_OK : LRKV_ERR_DEVICE;
}

#define LRKV_DECODE_ARGS                                                                                        \
  int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim, int32_t rank, int64_t capacity,         \
      const void *k_shared, const void *v_shared, const void *z_k, const void *z_v, const int32_t *seq_lens,   \
      int64_t max_len, const void *q, const void *b_k, const void *b_v, float scale, int32_t split_tokens,     \
      void *out, void *workspace, size_t workspace_bytes, void *stream
#define LRKV_DECODE_PASS                                                                                   \
  dtype, batch, num_heads, head_dim, rank, capacity, k_shared, v_shared, z_k, z_v, seq_lens, max_len, q, b_k, \
      b_v, scale, split_tokens, out, workspace, workspace_bytes, stream

lrkv_status lrkv_decode(LRKV_DECODE_ARGS) { return decode_phases(3, LRKV_DECODE_PASS); }
lrkv_status lrkv_decode_ex(int32_t engine, int32_t phases, LRKV_DECODE_ARGS) {
  return decode_phases(phases, LRKV_DECODE_PASS, engine);
}

lrkv_status lrkv_decode_noalloc(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim, int32_t rank,
                                int64_t capacity, const void* k_shared, const void* v_shared, const void* z_k,
                                const void* z_v, const int32_t* seq_lens, int64_t max_len, const void* q,
                                const void* b_k, const void* b_v, float scale, int32_t split_tokens, void* out,
                                void* stream) {
  DecodePlan pl;
  const lrkv_status st = plan_decode(dtype, batch, num_heads, head_dim, rank, capacity, max_len, split_tokens, &pl);
  if (st != LRKV_OK) return st;
  if (workspace_bytes_of(pl) > kScratchBytes) return LRKV_ERR_SCRATCH;
  if (batch == 0) return LRKV_OK;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return LRKV_ERR_DEVICE;
  return decode_phases(3, dtype, batch, num_heads, head_dim, rank, capacity, k_shared, v_shared, z_k, z_v, seq_lens,
                       max_len, q, b_k, b_v, scale, split_tokens, out, ws, kScratchBytes, stream);
}
lrkv_status lrkv_decode_partial(LRKV_DECODE_ARGS) { return decode_phases(1, LRKV_DECODE_PASS); }
lrkv_status lrkv_decode_combine(LRKV_DECODE_ARGS) { return decode_phases(2, LRKV_DECODE_PASS); }

lrkv_status lrkv_append(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim, int32_t rank,
                        int64_t capacity, void* k_shared, void* v_shared, void* z_k, void* z_v,
                        const int32_t* pos, int32_t n_new, const void* new_k_s, const void* new_v_s,
                        const void* new_z_k, const void* new_z_v, void* stream) {
  const lrkv_status st = check_sizes(dtype, batch, num_heads, head_dim, rank, capacity);
  if (st != LRKV_OK) return st;
  if (n_new < 0) return LRKV_ERR_SHAPE;
  if (batch == 0 || n_new == 0) return LRKV_OK;
  if (!k_shared || !v_shared || !pos || !new_k_s || !new_v_s) return LRKV_ERR_NULL;
  if (rank > 0 && (!z_k || !z_v || !new_z_k || !new_z_v)) return LRKV_ERR_NULL;
  if (!aligned16(k_shared) || !aligned16(v_shared) || !aligned16(new_k_s) || !aligned16(new_v_s) ||
      !aligned4(pos))
    return LRKV_ERR_ALIGN;
  if (rank > 0 && (!aligned16(z_k) || !aligned16(z_v) || !aligned16(new_z_k) || !aligned16(new_z_v)))
    return LRKV_ERR_ALIGN;
  lrkv::AppendArgs a;
  a.dtype = dtype; a.batch = batch; a.heads = num_heads; a.head_dim = head_dim; a.rank = rank;
  a.capacity = capacity; a.k_s = k_shared; a.v_s = v_shared; a.z_k = z_k; a.z_v = z_v;
  a.pos = pos; a.pos_max = INT32_MAX; a.n_new = n_new;
  a.new_k_s = new_k_s; a.new_v_s = new_v_s; a.new_z_k = new_z_k; a.new_z_v = new_z_v;
  const hipError_t e = lrkv::launch_append(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LRKV_OK : LRKV_ERR_DEVICE;
}

namespace {

// Shapes outside the MFMA prefill's envelope run on the vector-ALU kernel
// (one workgroup per 32 queries of a head and sequence: grid limits).
bool prefill_generic_ok(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim, int32_t rank) {
  return lrkv::prefill_generic_supported(dtype, head_dim, rank, num_heads) && batch <= 65535;
}

// Which prefill kernel a shape runs on: the bf16 MFMA kernel at ranks 0, 8,
// 16 and 32; its padded form at the other ranks it takes; else the vector-ALU kernel.
enum class PrefillEngine { kMfma, kWide, kGeneric, kNone };

PrefillEngine prefill_engine(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim, int32_t rank) {
  if (lrkv::prefill_supported(dtype, head_dim, rank, num_heads)) return PrefillEngine::kMfma;
  if (lrkv::prefill_wide_supported(dtype, head_dim, rank, num_heads)) return PrefillEngine::kWide;
  return prefill_generic_ok(dtype, batch, num_heads, head_dim, rank) ? PrefillEngine::kGeneric : PrefillEngine::kNone;
}

lrkv_status run_prefill(PrefillEngine eng, int32_t dtype, const lrkv::PrefillArgs& p, hipStream_t s) {
  const hipError_t e = eng == PrefillEngine::kMfma   ? lrkv::launch_prefill(p, s)
                       : eng == PrefillEngine::kWide ? lrkv::launch_prefill_wide(p, s)
                                                     : lrkv::launch_prefill_generic(dtype, p, s);
  return e == hipSuccess ? LRKV_OK : LRKV_ERR_DEVICE;
}

}  // namespace

const char* lrkv_prefill_kernel(int32_t dtype, int32_t num_heads, int32_t head_dim, int32_t rank) {
  if (check_sizes(dtype, 1, num_heads, head_dim, rank, 1) != LRKV_OK) return nullptr;
  switch (prefill_engine(dtype, 1, num_heads, head_dim, rank)) {
    case PrefillEngine::kMfma: return "prefill_kernel";
    case PrefillEngine::kWide: return "prefill_wide_kernel";
    case PrefillEngine::kGeneric: return "prefill_generic_kernel";
    default: return nullptr;
  }
}

lrkv_status lrkv_prefill(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim, int32_t rank,
                         int64_t capacity, void* k_shared, void* v_shared, void* z_k, void* z_v, int32_t seq_len,
                         const void* q, const void* k_s, const void* v_s, const void* z_k_new,
                         const void* z_v_new, const void* b_k, const void* b_v, float scale, void* out,
                         void* stream) {
  const lrkv_status st = check_sizes(dtype, batch, num_heads, head_dim, rank, capacity);
  if (st != LRKV_OK) return st;
  const PrefillEngine eng = prefill_engine(dtype, batch, num_heads, head_dim, rank);
  if (eng == PrefillEngine::kNone) return LRKV_ERR_SHAPE;
  if (seq_len < 0) return LRKV_ERR_SHAPE;
  // the MFMA kernels address one sequence's rows and latents through 32-bit
  // buffer offsets (the padded one reads up to 128 bytes past a latent row)
  if (eng != PrefillEngine::kGeneric &&
      int64_t(seq_len) * std::max<int64_t>(int64_t(head_dim), int64_t(num_heads) * rank) * 2 >=
          (int64_t(1) << 32) - 1024)
    return LRKV_ERR_SHAPE;
  // the cache is written when its pointers are given (the latent ones only count for rank > 0)
  const int want = rank > 0 ? 4 : 2;
  const int ncache = (k_shared != nullptr) + (v_shared != nullptr) + (rank > 0 ? (z_k != nullptr) + (z_v != nullptr) : 0);
  const bool write_cache = ncache == want;
  if (ncache != 0 && ncache != want) return LRKV_ERR_NULL;
  if (write_cache && seq_len > capacity) return LRKV_ERR_CAPACITY;
  if (batch == 0 || seq_len == 0) return LRKV_OK;
  if (!q || !k_s || !v_s || !out) return LRKV_ERR_NULL;
  if (rank > 0 && (!z_k_new || !z_v_new || !b_k || !b_v)) return LRKV_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_s) || !aligned16(v_s) || !aligned16(out)) return LRKV_ERR_ALIGN;
  if (rank > 0 && (!aligned16(z_k_new) || !aligned16(z_v_new) || !aligned16(b_k) || !aligned16(b_v)))
    return LRKV_ERR_ALIGN;
  if (write_cache && (!aligned16(k_shared) || !aligned16(v_shared) ||
                      (rank > 0 && (!aligned16(z_k) || !aligned16(z_v)))))
    return LRKV_ERR_ALIGN;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (write_cache) {
    lrkv::AppendArgs a;
    a.dtype = dtype; a.batch = batch; a.heads = num_heads; a.head_dim = head_dim; a.rank = rank;
    a.capacity = capacity; a.k_s = k_shared; a.v_s = v_shared; a.z_k = z_k; a.z_v = z_v;
    a.pos = nullptr; a.pos_max = INT32_MAX; a.n_new = seq_len;
    a.new_k_s = k_s; a.new_v_s = v_s; a.new_z_k = z_k_new; a.new_z_v = z_v_new;
    if (lrkv::launch_append(a, s) != hipSuccess) return LRKV_ERR_DEVICE;
  }
  const float sc = (scale > 0.f && std::isfinite(scale)) ? scale : 1.0f / std::sqrt(float(head_dim));
  lrkv::PrefillArgs p;
  p.batch = batch; p.heads = num_heads; p.head_dim = head_dim; p.rank = rank; p.seq_len = seq_len;
  p.q = q; p.k_s = k_s; p.v_s = v_s; p.z_k = z_k_new; p.z_v = z_v_new; p.b_k = b_k; p.b_v = b_v;
  p.scale_log2 = sc * 1.4426950408889634f;
  p.out = out;
  p.kv_stride = seq_len; p.start = nullptr; p.max_start = 0;
  return run_prefill(eng, dtype, p, s);
}

lrkv_status lrkv_prefill_chunk(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim, int32_t rank,
                               int64_t capacity, void* k_shared, void* v_shared, void* z_k, void* z_v,
                               const int32_t* start_pos, int32_t max_start, int32_t n_new, const void* q,
                               const void* k_s, const void* v_s, const void* z_k_new, const void* z_v_new,
                               const void* b_k, const void* b_v, float scale, void* out, void* stream) {
  const lrkv_status st = check_sizes(dtype, batch, num_heads, head_dim, rank, capacity);
  if (st != LRKV_OK) return st;
  const PrefillEngine eng = prefill_engine(dtype, batch, num_heads, head_dim, rank);
  if (eng == PrefillEngine::kNone) return LRKV_ERR_SHAPE;
  if (n_new < 0 || max_start < 0) return LRKV_ERR_SHAPE;
  if (int64_t(max_start) + n_new > capacity) return LRKV_ERR_CAPACITY;
  // the MFMA kernels address one sequence's keys (history and new tokens) through 32-bit buffer offsets
  if (eng != PrefillEngine::kGeneric &&
      (int64_t(max_start) + n_new) * std::max<int64_t>(int64_t(head_dim), int64_t(num_heads) * rank) * 2 >=
          (int64_t(1) << 32) - 1024)
    return LRKV_ERR_SHAPE;
  if (batch == 0 || n_new == 0) return LRKV_OK;
  if (!k_shared || !v_shared || !start_pos || !q || !k_s || !v_s || !out) return LRKV_ERR_NULL;
  if (rank > 0 && (!z_k || !z_v || !z_k_new || !z_v_new || !b_k || !b_v)) return LRKV_ERR_NULL;
  if (!aligned16(k_shared) || !aligned16(v_shared) || !aligned4(start_pos) || !aligned16(q) || !aligned16(k_s) ||
      !aligned16(v_s) || !aligned16(out))
    return LRKV_ERR_ALIGN;
  if (rank > 0 && (!aligned16(z_k) || !aligned16(z_v) || !aligned16(z_k_new) || !aligned16(z_v_new) ||
                   !aligned16(b_k) || !aligned16(b_v)))
    return LRKV_ERR_ALIGN;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  lrkv::AppendArgs a;
  a.dtype = dtype; a.batch = batch; a.heads = num_heads; a.head_dim = head_dim; a.rank = rank;
  a.capacity = capacity; a.k_s = k_shared; a.v_s = v_shared; a.z_k = z_k; a.z_v = z_v;
  a.pos = start_pos; a.pos_max = max_start; a.n_new = n_new;
  a.new_k_s = k_s; a.new_v_s = v_s; a.new_z_k = z_k_new; a.new_z_v = z_v_new;
  if (lrkv::launch_append(a, s) != hipSuccess) return LRKV_ERR_DEVICE;
  const float sc = (scale > 0.f && std::isfinite(scale)) ? scale : 1.0f / std::sqrt(float(head_dim));
  lrkv::PrefillArgs p;
  p.batch = batch; p.heads = num_heads; p.head_dim = head_dim; p.rank = rank; p.seq_len = n_new;
  p.q = q; p.k_s = k_shared; p.v_s = v_shared; p.z_k = z_k; p.z_v = z_v; p.b_k = b_k; p.b_v = b_v;
  p.scale_log2 = sc * 1.4426950408889634f;
  p.out = out;
  p.kv_stride = int(capacity); p.start = start_pos; p.max_start = max_start;
  return run_prefill(eng, dtype, p, s);
}

namespace {

// Shared validation of the training entry points' sizes.
lrkv_status check_train_sizes(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim, int32_t rank,
                              int32_t seq_len) {
  const lrkv_status st = check_sizes(dtype, batch, num_heads, head_dim, rank, 1);
  if (st != LRKV_OK) return st;
  if (!lrkv::train_supported(dtype, head_dim, rank, num_heads)) return LRKV_ERR_SHAPE;
  if (seq_len < 0) return LRKV_ERR_SHAPE;
  if (int64_t(batch) * seq_len >= (int64_t(1) << 31)) return LRKV_ERR_SHAPE;
  if (int64_t(seq_len) * std::max<int64_t>(int64_t(head_dim), int64_t(num_heads) * rank) * 2 >= (int64_t(1) << 32))
    return LRKV_ERR_SHAPE;
  return LRKV_OK;
}

float resolve_scale(float scale, int32_t head_dim) {
  return (scale > 0.f && std::isfinite(scale)) ? scale : 1.0f / std::sqrt(float(head_dim));
}

}  // namespace

lrkv_status lrkv_train_forward(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim, int32_t rank,
                               int32_t seq_len, const void* q, const void* k_s, const void* v_s, const void* z_k,
                               const void* z_v, const void* b_k, const void* b_v, float scale, void* out, float* lse,
                               void* stream) {
  const lrkv_status st = check_train_sizes(dtype, batch, num_heads, head_dim, rank, seq_len);
  if (st != LRKV_OK) return st;
  if (batch == 0 || seq_len == 0) return LRKV_OK;
  if (!q || !k_s || !v_s || !out || !lse) return LRKV_ERR_NULL;
  if (rank > 0 && (!z_k || !z_v || !b_k || !b_v)) return LRKV_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_s) || !aligned16(v_s) || !aligned16(out) || !aligned4(lse)) return LRKV_ERR_ALIGN;
  if (rank > 0 && (!aligned16(z_k) || !aligned16(z_v) || !aligned16(b_k) || !aligned16(b_v))) return LRKV_ERR_ALIGN;
  lrkv::PrefillArgs p;
  p.batch = batch; p.heads = num_heads; p.head_dim = head_dim; p.rank = rank; p.seq_len = seq_len;
  p.q = q; p.k_s = k_s; p.v_s = v_s; p.z_k = z_k; p.z_v = z_v; p.b_k = b_k; p.b_v = b_v;
  p.scale_log2 = resolve_scale(scale, head_dim) * 1.4426950408889634f;
  p.out = out;
  p.kv_stride = seq_len; p.start = nullptr; p.max_start = 0;
  p.lse = lse;
  return lrkv::launch_prefill(p, static_cast<hipStream_t>(stream)) == hipSuccess ? LRKV_OK : LRKV_ERR_DEVICE;
}

lrkv_status lrkv_train_backward_workspace_size(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim,
                                               int32_t rank, int32_t seq_len, size_t* bytes) {
  if (!bytes) return LRKV_ERR_NULL;
  const lrkv_status st = check_train_sizes(dtype, batch, num_heads, head_dim, rank, seq_len);
  if (st != LRKV_OK) return st;
  *bytes = lrkv::train_backward_ws_bytes(batch, num_heads, head_dim, rank, seq_len);
  return LRKV_OK;
}

lrkv_status lrkv_train_backward(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim, int32_t rank,
                                int32_t seq_len, const void* q, const void* k_s, const void* v_s, const void* z_k,
                                const void* z_v, const void* b_k, const void* b_v, const void* out, const float* lse,
                                const void* d_out, float scale, float* dq, float* dk_s, float* dv_s, float* dz_k,
                                float* dz_v, float* db_k, float* db_v, void* workspace, size_t workspace_bytes,
                                void* stream) {
  const lrkv_status st = check_train_sizes(dtype, batch, num_heads, head_dim, rank, seq_len);
  if (st != LRKV_OK) return st;
  const size_t need = lrkv::train_backward_ws_bytes(batch, num_heads, head_dim, rank, seq_len);
  const bool empty = batch == 0 || seq_len == 0;
  if (rank > 0 && (!db_k || !db_v)) return LRKV_ERR_NULL;
  if (rank > 0 && (!aligned4(db_k) || !aligned4(db_v))) return LRKV_ERR_ALIGN;
  if (!empty) {
    if (!q || !k_s || !v_s || !out || !lse || !d_out || !dq || !dk_s || !dv_s) return LRKV_ERR_NULL;
    if (rank > 0 && (!z_k || !z_v || !b_k || !b_v || !dz_k || !dz_v)) return LRKV_ERR_NULL;
    if (!workspace) return LRKV_ERR_NULL;
    if (workspace_bytes < need) return LRKV_ERR_WORKSPACE;
    if (!aligned16(q) || !aligned16(k_s) || !aligned16(v_s) || !aligned16(out) || !aligned16(lse) ||
        !aligned16(d_out) || !aligned16(dq) || !aligned4(dk_s) || !aligned4(dv_s) || !aligned16(workspace))
      return LRKV_ERR_ALIGN;
    if (rank > 0 && (!aligned16(z_k) || !aligned16(z_v) || !aligned16(b_k) || !aligned16(b_v) || !aligned4(dz_k) ||
                     !aligned4(dz_v)))
      return LRKV_ERR_ALIGN;
  }
  lrkv::TrainArgs a;
  a.batch = batch; a.heads = num_heads; a.head_dim = head_dim; a.rank = rank; a.seq_len = seq_len;
  a.q = q; a.k_s = k_s; a.v_s = v_s; a.z_k = z_k; a.z_v = z_v; a.b_k = b_k; a.b_v = b_v;
  a.out = out; a.lse = lse; a.d_out = d_out;
  a.scale = resolve_scale(scale, head_dim);
  a.dq = dq; a.dk_s = dk_s; a.dv_s = dv_s; a.dz_k = dz_k; a.dz_v = dz_v; a.db_k = db_k; a.db_v = db_v;
  a.ws = workspace;
  return lrkv::launch_train_backward(a, static_cast<hipStream_t>(stream)) == hipSuccess ? LRKV_OK : LRKV_ERR_DEVICE;
}

lrkv_status lrkv_pack_projection(int32_t dtype, int32_t num_heads, int32_t head_dim, int32_t rank,
                                 int32_t d_model, const void* wk_shared, const void* wv_shared,
                                 const void* u_k, const void* u_v, void* w_packed, void* stream) {
  if (dtype != LRKV_F32 && dtype != LRKV_BF16) return LRKV_ERR_DTYPE;
  if (num_heads < 1 || head_dim < 1 || rank < 0 || d_model < 0) return LRKV_ERR_SHAPE;
  if ((int64_t(head_dim) + int64_t(num_heads) * rank) * 2 * std::max(d_model, 1) * elem_bytes(dtype) >=
      (int64_t(1) << 40))
    return LRKV_ERR_SHAPE;
  if (d_model == 0) return LRKV_OK;
  if (!wk_shared || !wv_shared || !w_packed) return LRKV_ERR_NULL;
  if (rank > 0 && (!u_k || !u_v)) return LRKV_ERR_NULL;
  const uintptr_t mask = uintptr_t(elem_bytes(dtype) - 1);
  for (const void* ptr : {wk_shared, wv_shared, u_k, u_v, static_cast<const void*>(w_packed)})
    if (reinterpret_cast<uintptr_t>(ptr) & mask) return LRKV_ERR_ALIGN;
  lrkv::PackArgs a;
  a.dtype = dtype; a.heads = num_heads; a.head_dim = head_dim; a.rank = rank; a.d_model = d_model;
  a.wk_shared = wk_shared; a.wv_shared = wv_shared; a.u_k = u_k; a.u_v = u_v; a.w_packed = w_packed;
  return lrkv::launch_pack_projection(a, static_cast<hipStream_t>(stream)) == hipSuccess ? LRKV_OK : LRKV_ERR_DEVICE;
}

const char* lrkv_project_kernel(int32_t dtype, int32_t batch, int32_t n_new, int32_t num_heads, int32_t head_dim,
                                int32_t rank, int32_t d_model, int32_t with_workspace) {
  if (check_sizes(dtype, batch, num_heads, head_dim, rank, 1) != LRKV_OK) return nullptr;
  if (batch < 1 || n_new < 1 || d_model < 1 || d_model > 65536 || int64_t(batch) * n_new >= INT32_MAX) return nullptr;
  return lrkv::project_kernel_name(dtype, batch, n_new, num_heads, head_dim, rank, d_model, with_workspace != 0);
}

lrkv_status lrkv_project_workspace_size(int32_t dtype, int32_t batch, int32_t n_new, int32_t num_heads,
                                        int32_t head_dim, int32_t rank, int32_t d_model, size_t* bytes) {
  if (!bytes) return LRKV_ERR_NULL;
  const lrkv_status st = check_sizes(dtype, batch, num_heads, head_dim, rank, 1);
  if (st != LRKV_OK) return st;
  if (n_new < 0 || d_model < 1 || d_model > 65536 || int64_t(batch) * n_new >= INT32_MAX) return LRKV_ERR_SHAPE;
  *bytes = lrkv::project_workspace_bytes(dtype, batch, n_new, num_heads, head_dim, rank, d_model);
  return LRKV_OK;
}

lrkv_status lrkv_project_append(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim,
                                int32_t rank, int64_t capacity, void* k_shared, void* v_shared, void* z_k,
                                void* z_v, const int32_t* pos, int32_t n_new, int32_t d_model, const void* x,
                                const void* w_packed, void* workspace, size_t workspace_bytes, void* stream) {
  const lrkv_status st = check_sizes(dtype, batch, num_heads, head_dim, rank, capacity);
  if (st != LRKV_OK) return st;
  if (n_new < 0 || d_model < 1 || d_model > 65536) return LRKV_ERR_SHAPE;
  if (int64_t(batch) * n_new >= INT32_MAX) return LRKV_ERR_SHAPE;
  if ((int64_t(head_dim) + int64_t(num_heads) * rank) * 2 >= INT32_MAX) return LRKV_ERR_SHAPE;
  if (batch == 0 || n_new == 0) return LRKV_OK;
  if (!k_shared || !v_shared || !pos || !x || !w_packed) return LRKV_ERR_NULL;
  if (rank > 0 && (!z_k || !z_v)) return LRKV_ERR_NULL;
  if (!aligned16(k_shared) || !aligned16(v_shared) || !aligned4(pos) || !aligned16(x) || !aligned16(w_packed))
    return LRKV_ERR_ALIGN;
  if (rank > 0 && (!aligned16(z_k) || !aligned16(z_v))) return LRKV_ERR_ALIGN;
  if (workspace && !aligned16(workspace)) return LRKV_ERR_ALIGN;
  lrkv::ProjectArgs a;
  a.dtype = dtype; a.batch = batch; a.heads = num_heads; a.head_dim = head_dim; a.rank = rank;
  a.d_model = d_model; a.n_new = n_new; a.capacity = capacity;
  a.k_s = k_shared; a.v_s = v_shared; a.z_k = z_k; a.z_v = z_v; a.pos = pos; a.x = x; a.w = w_packed;
  a.ws = static_cast<float*>(workspace);
  a.ws_bytes = workspace ? workspace_bytes : 0;
  return lrkv::launch_project_append(a, static_cast<hipStream_t>(stream)) == hipSuccess ? LRKV_OK
                                                                                        : LRKV_ERR_DEVICE;
}

// Plain MHA decode (the matched-shape baseline): fixed splits of the context,
// about two workgroups per compute unit by default.
static lrkv_status plan_mha(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim, int64_t capacity,
                            int64_t max_len, int32_t split_tokens, int* split_out, int* n_splits, size_t* ws_ml,
                            size_t* ws_acc) {
  if (dtype != LRKV_F32 && dtype != LRKV_BF16) return LRKV_ERR_DTYPE;
  if (batch < 0 || num_heads < 1 || capacity < 1 || capacity > INT32_MAX || max_len < 0 || split_tokens < 0)
    return LRKV_ERR_SHAPE;
  if (!lrkv::mha_supported(dtype, head_dim)) return LRKV_ERR_SHAPE;
  if (max_len > capacity) return LRKV_ERR_CAPACITY;
  if (split_tokens % 64 != 0) return LRKV_ERR_SHAPE;
  int64_t split = split_tokens;
  if (split == 0) {
    const int64_t groups = (num_heads + 31) / 32;
    const int64_t target = 2 * int64_t(device_cu_count());
    split = (int64_t(batch) * max_len * groups + target - 1) / target;
    split = std::max<int64_t>(64, (split + 63) / 64 * 64);
    split = std::min<int64_t>(split, std::max<int64_t>(64, (max_len + 63) / 64 * 64));
  }
  // one split's rows (and the loads of a step past its end) are addressed
  // through 32-bit buffer offsets
  if ((split + 64) * num_heads * head_dim * elem_bytes(dtype) >= (int64_t(1) << 32)) return LRKV_ERR_SHAPE;
  const int64_t ns = max_len > 0 ? (max_len + split - 1) / split : 0;
  *split_out = int(split);
  *n_splits = int(ns);
  *ws_ml = (size_t(batch) * ns * num_heads * 2 * sizeof(float) + 255) / 256 * 256;   // keeps the sums 16-byte aligned
  *ws_acc = size_t(batch) * ns * num_heads * head_dim * sizeof(float);
  return LRKV_OK;
}

lrkv_status lrkv_mha_decode_workspace_size(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim,
                                           int64_t capacity, int64_t max_len, int32_t split_tokens, size_t* bytes) {
  if (!bytes) return LRKV_ERR_NULL;
  int split, ns;
  size_t ml, acc;
  const lrkv_status st = plan_mha(dtype, batch, num_heads, head_dim, capacity, max_len, split_tokens, &split, &ns,
                                  &ml, &acc);
  if (st != LRKV_OK) return st;
  *bytes = ml + acc;
  return LRKV_OK;
}

lrkv_status lrkv_mha_decode(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim, int64_t capacity,
                            const void* k, const void* v, const int32_t* seq_lens, int64_t max_len, const void* q,
                            float scale, int32_t split_tokens, void* out, void* workspace, size_t workspace_bytes,
                            void* stream) {
  int split, ns;
  size_t ml, acc;
  const lrkv_status st = plan_mha(dtype, batch, num_heads, head_dim, capacity, max_len, split_tokens, &split, &ns,
                                  &ml, &acc);
  if (st != LRKV_OK) return st;
  if (batch == 0) return LRKV_OK;
  if (!k || !v || !seq_lens || !q || !out) return LRKV_ERR_NULL;
  if (ns > 0 && (!workspace || workspace_bytes < ml + acc)) return LRKV_ERR_WORKSPACE;
  if (!aligned16(k) || !aligned16(v) || !aligned16(q) || !aligned16(out) || !aligned4(seq_lens) ||
      (ns > 0 && !aligned16(workspace)))
    return LRKV_ERR_ALIGN;
  const float sc = (scale > 0.f && std::isfinite(scale)) ? scale : 1.0f / std::sqrt(float(head_dim));
  lrkv::MhaArgs a;
  a.dtype = dtype; a.batch = batch; a.heads = num_heads; a.head_dim = head_dim; a.max_len = int(max_len);
  a.split_tokens = split; a.n_splits = ns; a.phase = 3; a.capacity = capacity;
  a.k = k; a.v = v; a.seq_lens = seq_lens; a.q = q; a.scale_log2 = sc * 1.4426950408889634f; a.out = out;
  a.ws_ml = static_cast<float*>(workspace);
  a.ws_acc = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + ml);
  if (ns == 0) {
    // every length is 0: the output is all zeros, produced by the merge alone
    a.n_splits = 1;
    a.phase = 2;
    a.ws_ml = a.ws_acc = nullptr;
  }
  return lrkv::launch_mha_decode(a, static_cast<hipStream_t>(stream)) == hipSuccess ? LRKV_OK : LRKV_ERR_DEVICE;
}

}  // extern "C"
