// Internal launch interface between the C-ABI host layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace lrkv {

// Raise a kernel's dynamic-LDS limit to `bytes`, once per device (the
// attribute belongs to the kernel on the device current at the call).
template <auto Kernel>
hipError_t allow_dynamic_lds(int bytes) {
  static std::atomic<uint64_t> done{0};        // bit d: set on device d
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? uint64_t(1) << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(Kernel), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Per-device set-up done at a kernel's first launch (the dynamic-LDS limit
// of every kernel that needs more than the default), done for every kernel
// at once; each returns the first failure.
hipError_t decode_mfma_prepare();
hipError_t decode_mfma_any_prepare();
hipError_t prefill_prepare();
hipError_t project_prepare();
hipError_t train_prepare();

constexpr int kDecodeThreads = 256;  // one workgroup = 4 wave64
constexpr int kDecodeTile = 64;      // cache tokens staged in LDS per step

struct DecodePlan {
  int batch, heads, head_dim, rank, dtype;
  int64_t capacity;
  int max_len;
  int split_tokens;   // tokens per split (multiple of kDecodeTile)
  int n_splits;       // ceil(max_len / split_tokens)
  int group;          // lanes per head (G)
  int heads_pow2;     // heads rounded up to a power of two
  int slots;          // independent token streams per workgroup
  int partials;       // n_splits * slots partial states per (sequence, head)
  bool mfma;          // scan on the MFMA kernel (one partial state per workgroup: slots = 1)
  bool generic;       // scan and merge of the any-rank kernels (one partial state per split: slots = 1)
  bool mfma_any;      // scan on the any-rank MFMA kernel, merge of the any-rank kernels (fixed splits)
  bool balanced;      // length-balanced items computed on the device (MFMA scan, default split):
                      // n_splits = partials = max(bal_cap, batch) items, state index item * heads + h
  int bal_cap;        // items the partition aims for (resident scan workgroups)
  size_t ws_ml_bytes, ws_acc_bytes, ws_meta_bytes;
  size_t ws_qt_bytes;  // any-rank MFMA scan: the absorbed query [batch][heads][rank] fp32
};

struct DecodeArgs {
  const void* k_s; const void* v_s; const void* z_k; const void* z_v;
  const int32_t* seq_lens;
  const void* q; const void* b_k; const void* b_v;
  float scale_log2;   // softmax scale times log2(e)
  void* out;
  float* ws_ml;       // [batch][partials][heads] x (m, l)
  float* ws_acc;      // [batch][partials][heads][head_dim + rank]
  int* ws_meta;       // balanced partition: first item of each sequence [batch], then the item size
  float* ws_qt;       // any-rank MFMA scan: absorbed query [batch][heads][rank]
};

// Returns false if (dtype, head_dim, rank, heads) is outside the compiled envelope.
bool decode_supported(int dtype, int head_dim, int rank, int heads);
// Shapes the MFMA scan takes: bf16, head_dim 64 or 128, rank 0/8/16/32,
// heads a multiple of 32 up to 64.
bool decode_mfma_supported(int dtype, int head_dim, int rank, int heads);
constexpr int kMfmaSlots = 1;        // partial states per MFMA-scan workgroup
// The any-rank scan (decode_generic.hip): bf16 or fp32, head_dim 16/32/64/128,
// any rank up to kGenericMaxRank, up to kGenericMaxHeads heads.
constexpr int kGenericMaxRank = 128;
constexpr int kGenericMaxHeads = 1024;
constexpr int kGenericMaxDims = 128 + kGenericMaxRank;   // head_dim + rank
bool decode_generic_supported(int dtype, int head_dim, int rank, int heads);
// Lanes per head of the any-rank scan (8, 16 or 32); 256 / that many heads per workgroup.
int generic_lanes_per_head(int heads, int head_dim);
hipError_t launch_decode_generic(const DecodePlan& plan, const DecodeArgs& args, int phase, hipStream_t stream);
hipError_t launch_decode_mfma_scan(const DecodePlan& plan, const DecodeArgs& args, hipStream_t stream);
// The any-rank MFMA scan (decode_mfma_any.hip): bf16, head_dim 128, ranks 8 to
// kGenericMaxRank with heads * rank even; its merge is the any-rank merge.
bool decode_mfma_any_supported(int dtype, int head_dim, int rank, int heads);
// Supported, and the default over decode_generic_kernel.
bool decode_mfma_any_preferred(int dtype, int head_dim, int rank, int heads);
hipError_t launch_decode_mfma_any(const DecodePlan& plan, const DecodeArgs& args, int phase, hipStream_t stream);
// phase: 1 = split-K scan only, 2 = combine only, 3 = both (every plan but
// the any-rank MFMA scan's, which launch_decode_mfma_any runs).
hipError_t launch_decode(const DecodePlan& plan, const DecodeArgs& args, int phase, hipStream_t stream);

struct AppendArgs {
  int dtype, batch, heads, head_dim, rank;
  int64_t capacity;
  void* k_s; void* v_s; void* z_k; void* z_v;
  const int32_t* pos;      // device [batch], or NULL: slot 0 for every sequence
  int pos_max;             // positions are clamped to [0, pos_max] (INT32_MAX: no clamp)
  int n_new;
  const void* new_k_s; const void* new_v_s; const void* new_z_k; const void* new_z_v;
};
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);

struct PrefillArgs {
  int batch, heads, head_dim, rank, seq_len;
  const void* q; const void* k_s; const void* v_s; const void* z_k; const void* z_v;
  const void* b_k; const void* b_v;
  float scale_log2;
  void* out;
  int kv_stride;           // tokens per sequence in k_s/v_s/z_k/z_v (seq_len, or the cache capacity)
  const int32_t* start;    // device [batch] history lengths, or NULL (no history)
  int max_start;           // start is clamped to [0, max_start]
  float* lse = nullptr;    // optional [batch][seq_len][heads] natural log-sum-exp of each row's logits
};
bool prefill_supported(int dtype, int head_dim, int rank, int heads);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// The bf16 MFMA prefill at the other ranks up to 128 (latents padded to 64 or 128 rows in LDS).
bool prefill_wide_supported(int dtype, int head_dim, int rank, int heads);
hipError_t launch_prefill_wide(const PrefillArgs& a, hipStream_t stream);
hipError_t prefill_wide_prepare();
// The vector-ALU prefill for the other shapes: bf16 or fp32, head_dim 16-128
// (a multiple of 8), any rank up to kPrefillGenericMaxRank, at most 65535
// heads and sequences.
constexpr int kPrefillGenericMaxRank = 128;
bool prefill_generic_supported(int dtype, int head_dim, int rank, int heads);
hipError_t launch_prefill_generic(int dtype, const PrefillArgs& a, hipStream_t stream);
hipError_t prefill_generic_prepare();

struct TrainArgs {
  int batch, heads, head_dim, rank, seq_len;
  const void* q; const void* k_s; const void* v_s; const void* z_k; const void* z_v;   // bf16, fresh tokens
  const void* b_k; const void* b_v;
  const void* out; const float* lse; const void* d_out;   // forward output (bf16), its lse, upstream gradient (bf16)
  float scale;
  float* dq; float* dk_s; float* dv_s; float* dz_k; float* dz_v; float* db_k; float* db_v;   // fp32 gradients
  void* ws;                // train_backward_ws_bytes bytes
};
// Shapes the training backward takes: bf16, head_dim 64 or 128, rank 0/8/16/32,
// heads a multiple of 4.
bool train_supported(int dtype, int head_dim, int rank, int heads);
size_t train_backward_ws_bytes(int batch, int heads, int head_dim, int rank, int seq_len);
hipError_t launch_train_backward(const TrainArgs& a, hipStream_t stream);

struct ProjectArgs {
  int dtype, batch, heads, head_dim, rank, d_model, n_new;
  int64_t capacity;
  void* k_s; void* v_s; void* z_k; void* z_v;
  const int32_t* pos;      // device [batch]
  const void* x;           // [batch][n_new][d_model]
  const void* w;           // packed projection [2(head_dim + heads*rank)][d_model]
  float* ws;               // optional workspace for the split-contraction path (NULL: not used)
  size_t ws_bytes;
};
// Shapes the MFMA projection takes: bf16, head_dim and heads*rank multiples
// of 32, d_model a multiple of 32 (others run on the vector-ALU kernel).
bool project_mfma_supported(int dtype, int head_dim, int rank, int heads, int d_model);
hipError_t launch_project_append(const ProjectArgs& a, hipStream_t stream);
// Name of the kernel launch_project_append runs for these sizes on the current
// device, with or without a workspace of project_workspace_bytes.
const char* project_kernel_name(int dtype, int batch, int n_new, int heads, int head_dim, int rank, int d_model,
                                bool with_workspace);
// Workspace bytes that let these sizes split the contraction across workgroups (0: no use for one).
size_t project_workspace_bytes(int dtype, int batch, int n_new, int heads, int head_dim, int rank, int d_model);
size_t project_ws_bytes(long M, long N, int d_model);

struct PackArgs {
  int dtype, heads, head_dim, rank, d_model;
  const void* wk_shared; const void* wv_shared;   // [d_model][head_dim]
  const void* u_k; const void* u_v;               // [heads][d_model][rank]
  void* w_packed;                                 // [2(head_dim + heads*rank)][d_model]
};
hipError_t launch_pack_projection(const PackArgs& a, hipStream_t stream);

// The log-sum-exp merge of rank-0 partial states laid out [batch][partials][heads]
// (fixed splits), for caches without latents.
hipError_t launch_plain_merge(int dtype, int head_dim, const float* ws_ml, const float* ws_acc,
                              const int32_t* seq_lens, void* out, int heads, int partials, int split_tokens,
                              int max_len, int batch, hipStream_t stream);

struct MhaArgs {
  int dtype, batch, heads, head_dim, max_len, split_tokens, n_splits, phase;   // phase: 1 scan, 2 merge, 3 both
  int64_t capacity;
  const void* k; const void* v;      // [batch][capacity][heads][head_dim]
  const int32_t* seq_lens;
  const void* q;                     // [batch][heads][head_dim]
  float scale_log2;
  void* out;
  float* ws_ml; float* ws_acc;       // [batch][n_splits][heads] x (m, l); [batch][n_splits][heads][head_dim]
};
bool mha_supported(int dtype, int head_dim);
hipError_t launch_mha_decode(const MhaArgs& a, hipStream_t stream);

}  // namespace lrkv
