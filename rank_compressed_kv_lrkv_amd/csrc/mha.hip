// Plain multi-head attention decode over a full per-head K/V cache: the
// baseline the LRKV cache is measured against at a matched shape.  Every head
// caches its own key and value rows, 2 H d_h elements per token (slide "Can
// heads share storage while keeping distinct K/V features?": the MHA cache
// that LRKV's 2(d_h + H r) is compared with), and each head attends with its
// own rows: out[b][h] = softmax_t(scale q_bh . k[t][h]) applied to v[t][h].
//
// The work is one matrix-vector product per head and token, so the scan is
// HBM-bound on the vector ALUs: a workgroup (4 waves) takes one sequence, one
// split of its tokens and 32 heads; 8 lanes share a head, each owning d_h/8
// dimensions in 16-byte pieces: piece c of lane g is bytes
// [128 c + 16 g, 128 c + 16 g + 16) of the head's row, so each load
// instruction of a wave reads one whole 128-byte line of each of its 8 heads.
// MhaUnroll tokens are loaded together (non-temporal, through buffer
// resources, so tokens past the split read zeros), then scored with a DPP
// sum over the 8 lanes, folded into a running max / sum / output in the log2
// domain, and written as one partial state per (split, head) in the layout
// the LRKV decode merge reads (rank 0: no up-projection).
#include "lrkv_device.h"
#include "lrkv_internal.h"

namespace lrkv {

constexpr int kMhaThreads = 256;
constexpr int kMhaHeads = 32;            // heads per workgroup (8 per wave)
constexpr int kMhaLanes = 8;             // lanes per head

template <class E>
constexpr int MhaUnroll = E::kBytes == 2 ? 8 : 4;   // tokens in flight per step

struct MhaParams {
  const void* k; const void* v; const int32_t* seq_lens; const void* q;
  float scale_log2;
  int heads, partials, max_len, split_tokens;
  int64_t capacity;
  float* ws_ml; float* ws_acc;
};

template <class E, int DH>
__global__ __launch_bounds__(kMhaThreads) void mha_split_kernel(MhaParams p) {
  using T = typename E::T;
  constexpr int DPL = DH / kMhaLanes;                  // dimensions per lane
  constexpr int SB = DPL * E::kBytes;                  // bytes of a lane's slice of a row
  constexpr int U = MhaUnroll<E>;
  const int split = blockIdx.x, b = blockIdx.y, hg = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane % kMhaLanes;
  const int H = p.heads;
  const int hh = hg * kMhaHeads + wave * (64 / kMhaLanes) + lane / kMhaLanes;
  const bool active = hh < H;
  const int hc = active ? hh : H - 1;                  // inactive lanes read a valid row, write nothing
  int len = p.seq_lens[b];
  len = len < 0 ? 0 : (len > p.max_len ? p.max_len : len);
  const int t0 = split * p.split_tokens;
  if (t0 >= len) return;                               // uniform over the workgroup
  const int n = min(p.split_tokens, len - t0);

  constexpr int NPC = SB / 16;                         // 16-byte pieces per lane
  constexpr int EPC = 16 / E::kBytes;                  // elements per piece
  // query slice, pre-scaled into the log2 domain: element e of the lane is
  // dimension (128 (e / EPC) + 16 g) / kBytes + e % EPC
  float qf[DPL];
  {
    const unsigned char* qrow = reinterpret_cast<const unsigned char*>(static_cast<const T*>(p.q) +
                                                                        (size_t(b) * H + hc) * DH);
    uint32_t w[SB / 4];
#pragma unroll
    for (int c = 0; c < NPC; ++c) load_words<16>(w + 4 * c, qrow + 128 * c + 16 * g);
#pragma unroll
    for (int e = 0; e < DPL; ++e) qf[e] = E::to_f32(elem_at<E>(w, e)) * p.scale_log2;
  }
  // resources over the split's tokens (the host keeps them below 4 GiB)
  const uint32_t tok_bytes = uint32_t(H) * DH * E::kBytes;
  const size_t row0 = (size_t(b) * size_t(p.capacity) + size_t(t0)) * size_t(H) * DH;
  const __amdgpu_buffer_rsrc_t kres = buffer_resource(static_cast<const T*>(p.k) + row0, uint32_t(n) * tok_bytes);
  const __amdgpu_buffer_rsrc_t vres = buffer_resource(static_cast<const T*>(p.v) + row0, uint32_t(n) * tok_bytes);
  const uint32_t lane_off = uint32_t(hc) * DH * E::kBytes + uint32_t(g) * 16;

  float m = -INFINITY, l = 0.f, o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.f;
  for (int t = 0; t < n; t += U) {
    uint32_t kw[U][SB / 4], vw[U][SB / 4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t off = uint32_t(t + u) * tok_bytes + lane_off;
#pragma unroll
      for (int c = 0; c < NPC; ++c) {
        buffer_words<16, kStream>(kw[u] + 4 * c, kres, off + 128 * c, 0u);
        buffer_words<16, kStream>(vw[u] + 4 * c, vres, off + 128 * c, 0u);
      }
    }
    float s[U];
    float mx = m;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) d = __builtin_fmaf(qf[e], E::to_f32(elem_at<E>(kw[u], e)), d);
      d = group_sum<kMhaLanes>(d);
      s[u] = t + u < n ? d : -INFINITY;
      mx = fmaxf(mx, s[u]);
    }
    const float sc = fast_exp2(m - mx);                // 0 on the first step (m = -inf)
    l *= sc;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] *= sc;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float pu = fast_exp2(s[u] - mx);           // tokens past the split: 0
      l += pu;
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] = __builtin_fmaf(pu, E::to_f32(elem_at<E>(vw[u], e)), o[e]);
    }
    m = mx;
  }
  if (!active) return;
  const size_t pidx = (size_t(b) * p.partials + split) * H + hh;
  if (g == 0) *reinterpret_cast<float2*>(p.ws_ml + 2 * pidx) = make_float2(m, l);
  float* const acc = p.ws_acc + pidx * DH;
#pragma unroll
  for (int c = 0; c < NPC; ++c) {
    float* dst = acc + (128 * c + 16 * g) / E::kBytes;
#pragma unroll
    for (int e = 0; e < EPC; e += 4)
      *reinterpret_cast<float4*>(dst + e) =
          make_float4(o[EPC * c + e], o[EPC * c + e + 1], o[EPC * c + e + 2], o[EPC * c + e + 3]);
  }
}

template <class E, int DH>
static hipError_t launch_mha_t(const MhaArgs& a, hipStream_t st) {
  MhaParams p;
  p.k = a.k; p.v = a.v; p.seq_lens = a.seq_lens; p.q = a.q;
  p.scale_log2 = a.scale_log2;
  p.heads = a.heads; p.partials = a.n_splits; p.max_len = a.max_len; p.split_tokens = a.split_tokens;
  p.capacity = a.capacity;
  p.ws_ml = a.ws_ml; p.ws_acc = a.ws_acc;
  if (a.phase & 1) {
    const dim3 grid(a.n_splits, a.batch, (a.heads + kMhaHeads - 1) / kMhaHeads);
    hipLaunchKernelGGL((mha_split_kernel<E, DH>), grid, dim3(kMhaThreads), 0, st, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!(a.phase & 2)) return hipSuccess;
  return launch_plain_merge(a.dtype, DH, a.ws_ml, a.ws_acc, a.seq_lens, a.out, a.heads, a.n_splits, a.split_tokens,
                            a.max_len, a.batch, st);
}

bool mha_supported(int dtype, int head_dim) {
  return (dtype == 0 || dtype == 1) && (head_dim == 64 || head_dim == 128);
}

hipError_t launch_mha_decode(const MhaArgs& a, hipStream_t st) {
  if (a.batch <= 0 || a.n_splits <= 0) return hipSuccess;
  if (a.dtype == 1) return a.head_dim == 64 ? launch_mha_t<BF16, 64>(a, st) : launch_mha_t<BF16, 128>(a, st);
  return a.head_dim == 64 ? launch_mha_t<F32, 64>(a, st) : launch_mha_t<F32, 128>(a, st);
}

}  // namespace lrkv
