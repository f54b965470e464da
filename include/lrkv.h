/*
 * lrkv.h - C ABI of liblrkv: attention over an LRKV compressed KV cache on
 * AMD Instinct MI355X (gfx950).
 *
 * Method: Low-Rank Key Value Attention (O'Neill, Clancy, Matskevichus, Reid,
 * arXiv:2601.11471v3), in the slide discussion of that paper:
 *   - every head's K/V projection is a shared base plus a rank-r correction,
 *     W_h = W_shared + U_h B_h^T (slide "LRKV constrains differences between
 *     heads", Eqs. (2)-(3));
 *   - the cache stores, per token, one shared key row k_s and value row v_s of
 *     width d_h and, per head h, rank-r latents z^K_h and z^V_h; B_h are
 *     weights, not cache entries (slide "Cache shared features and compact
 *     per-head latents", Eqs. (4)-(5)); that is 2(d_h + H r) elements per
 *     token per layer (slide "Can heads share storage while keeping distinct
 *     K/V features?");
 *   - attention never expands per-head keys or values: the logits are
 *     q_h.k_s + (B^K_h^T q_h).z^K_h, scaled by 1/sqrt(d_h) and softmaxed
 *     (slide "Compute logits without expanding historical keys", Eq. (6)),
 *     and the output is a V_s + B^V_h (a R^V_h) (slide "Aggregate values
 *     before the residual up-projection", Eq. (7)).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library allocates no device memory (the one fixed scratch array of
 *     lrkv_decode_noalloc is part of its code object), keeps no per-call
 *     state, never synchronises, and enqueues all work on `stream` (a hipStream_t passed
 *     as void*; NULL is the default stream).  Results are ready when the
 *     stream has drained.  Since the calls only launch kernels (no
 *     allocation, memset, copy or synchronisation), a caller may capture
 *     them on a stream into a HIP graph and replay it; every replay reads the
 *     buffers' contents at replay time.  The first launch of some kernels on
 *     a device also raises their dynamic-LDS limit (a host-side attribute,
 *     not stream work); lrkv_init does this for every kernel at once, so
 *     after lrkv_init on a device no call needs an eager warm-up before
 *     capture.
 *   - `dtype` (lrkv_dtype) is the storage type of q, the cache, B^K, B^V,
 *     the new rows and the output, one type per call.  Arithmetic is fp32
 *     (bf16 products accumulate in fp32).
 *   - Dense row-major layouts (innermost index last):
 *       shared cache rows  k_shared, v_shared  [batch][capacity][head_dim]
 *       latent cache rows  z_k, z_v            [batch][capacity][num_heads][rank]
 *       residual factors   b_k, b_v            [num_heads][head_dim][rank]
 *     so the cache holds exactly 2(head_dim + num_heads*rank) elements per
 *     token slot.
 *   - Every pointer must be 16-byte aligned, and shared rows must be whole
 *     16-byte units: head_dim*elem_bytes % 16 == 0.  The latent run of a
 *     token (num_heads*rank elements) may have any length; rank == 0 is
 *     allowed and is MQA.
 *   - Decode envelope: head_dim in {16, 32, 64, 128}, and either a tuned
 *     scan's shape (rank in {0, 4, 8, 16, 32, 64}, bf16 needing rank % 8 ==
 *     0, 1 <= num_heads <= 64) or the any-rank scan's (rank 0..128, 1 <=
 *     num_heads <= 1024).  Prefill, chunk and training calls state their
 *     own envelopes.  Anything else returns LRKV_ERR_SHAPE before any
 *     launch.
 *   - Validation happens on the host before anything is enqueued; a call
 *     that returns an error has launched nothing.  A failed launch returns
 *     LRKV_ERR_DEVICE (from hipGetLastError).  No exception or abort crosses
 *     this interface.
 */
#ifndef LRKV_H
#define LRKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lrkv_status {
  LRKV_OK = 0,
  LRKV_ERR_NULL = 1,       /* a required pointer is NULL */
  LRKV_ERR_SHAPE = 2,      /* a size is invalid or outside the supported envelope */
  LRKV_ERR_DTYPE = 3,      /* dtype is not an lrkv_dtype */
  LRKV_ERR_ALIGN = 4,      /* a pointer is not 16-byte aligned */
  LRKV_ERR_CAPACITY = 5,   /* max_len or seq_len exceeds capacity */
  LRKV_ERR_WORKSPACE = 6,  /* workspace NULL or smaller than lrkv_decode_workspace_size */
  LRKV_ERR_DEVICE = 7,     /* a HIP runtime call or kernel launch failed */
  LRKV_ERR_SCRATCH = 8     /* lrkv_decode_noalloc: the call needs more than its fixed scratch */
} lrkv_status;

typedef enum lrkv_dtype {
  LRKV_F32 = 0,            /* IEEE binary32 */
  LRKV_BF16 = 1            /* bfloat16; outputs rounded to nearest-even */
} lrkv_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* lrkv_status_string(int32_t status);

/* Per-device set-up for the device current at the call: caches its compute
 * unit count and raises the dynamic-LDS limit of every kernel that needs
 * it.  Optional (each kernel's first launch does its own part); call it once
 * per device, outside any stream capture, before capturing library calls
 * into a HIP graph.  Idempotent and safe to call from several threads.
 * Returns LRKV_ERR_DEVICE if a HIP call fails.  Launches nothing. */
lrkv_status lrkv_init(void);

/* Cache elements per token per layer, 2(head_dim + num_heads*rank)
 * (slide "Can heads share storage while keeping distinct K/V features?",
 * and Eq. (9) of slide "The rank directly sets the theoretical cache
 * budget").  Returns -1 if an argument is negative or num_heads/head_dim is 0. */
int64_t lrkv_cache_elems_per_token(int32_t num_heads, int32_t head_dim, int32_t rank);

/* Append n_new tokens per sequence to the cache (slide "Cache shared
 * features and compact per-head latents", Eqs. (4)-(5): the shared rows
 * and the per-head latents are stored; B_h is not).
 *   pos      device int32 [batch]: first slot written for sequence b.
 *   new_k_s, new_v_s  [batch][n_new][head_dim];  new_z_k, new_z_v
 *   [batch][n_new][num_heads][rank].
 * Slot pos[b]+i of every cache array receives row i of sequence b,
 * bit-exactly; no other slot is touched.  Rows whose slot falls outside
 * [0, capacity) are dropped (pos is device data, so this cannot be
 * reported).  n_new == 0 is a no-op. */
lrkv_status lrkv_append(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim,
                        int32_t rank, int64_t capacity,
                        void* k_shared, void* v_shared, void* z_k, void* z_v,
                        const int32_t* pos, int32_t n_new,
                        const void* new_k_s, const void* new_v_s,
                        const void* new_z_k, const void* new_z_v, void* stream);

/* Bytes of device workspace lrkv_decode needs for these sizes and this
 * split (split_tokens == 0 selects the library's default for the device
 * that is current).  Written to *bytes.  The workspace holds the split-K
 * partial softmax states (fp32), and for decode_mfma_any_kernel also the
 * absorbed queries B^K_h^T q (fp32, batch * num_heads * rank). */
lrkv_status lrkv_decode_workspace_size(int32_t dtype, int32_t batch, int32_t num_heads,
                                       int32_t head_dim, int32_t rank, int64_t capacity,
                                       int64_t max_len, int32_t split_tokens, size_t* bytes);

/* Name of the kernel that runs the split-K scan of lrkv_decode for these
 * sizes: "decode_mfma_kernel" (bf16, head_dim 64 or 128, rank 0/8/16/32,
 * num_heads a multiple of 32 up to 64: the shared term runs on bf16 MFMA
 * across 32 heads), "decode_split_kernel" (the other shapes of the tuned
 * envelope: vector-ALU dot products), "decode_mfma_any_kernel" (bf16,
 * head_dim 128, any other rank from 8 to 128 with num_heads * rank even, up
 * to 1024 heads, except ranks above 112 with fewer than 32 heads; at the
 * pages' ranks such as 46, 51, 54, 55: the shared term on bf16 MFMA as in
 * decode_mfma_kernel, each lane's window of a latent row on 2-wide bf16
 * dots) or "decode_generic_kernel" (the remaining shapes up to rank 128 and
 * 1024 heads, fp32 included: vector-ALU, latents read element by element).
 * Returns NULL for a
 * shape outside the supported envelope.  Host-only: launches nothing; the
 * string is static. */
const char* lrkv_decode_scan_kernel(int32_t dtype, int32_t num_heads, int32_t head_dim, int32_t rank);

/* One decode step: for every sequence b and head h,
 *   out[b][h] = softmax_t( scale * (q_bh.k_s[t] + (B^K_h^T q_bh).z^K[t][h]) )
 *               applied to  v_s[t] + B^V_h z^V[t][h],   t < seq_lens[b],
 * computed in the absorbed form of Eqs. (6)-(7) without forming K_h, V_h.
 *   seq_lens  device int32 [batch]; each length is clamped to [0, max_len].
 *             A sequence of length 0 gets an all-zero output.
 *   max_len   host upper bound on the lengths, <= capacity (sizes the grid).
 *   q         [batch][num_heads][head_dim];   out [batch][num_heads][head_dim].
 *   b_k, b_v  [num_heads][head_dim][rank].
 *   scale     softmax scale; <= 0 selects 1/sqrt(head_dim).
 *   split_tokens  tokens per split-K partition (0 = default; otherwise a
 *             positive multiple of 64).  The partial states of all
 *             partitions are merged by a log-sum-exp combine.  A partition's
 *             shared rows and its latents must each span less than 4 GiB
 *             (split_tokens * max(head_dim, num_heads*rank) * elem_bytes),
 *             else LRKV_ERR_SHAPE.
 *   workspace device scratch of at least lrkv_decode_workspace_size bytes
 *             for the same arguments; contents on entry are ignored.
 * Every query attends to all of its sequence's cached tokens (the current
 * token is appended before the call); nothing inside the cache is masked. */
lrkv_status lrkv_decode(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim,
                        int32_t rank, int64_t capacity,
                        const void* k_shared, const void* v_shared,
                        const void* z_k, const void* z_v,
                        const int32_t* seq_lens, int64_t max_len,
                        const void* q, const void* b_k, const void* b_v, float scale,
                        int32_t split_tokens, void* out,
                        void* workspace, size_t workspace_bytes, void* stream);

/* The two phases of lrkv_decode, for callers that schedule them apart (for
 * instance to time the scan alone, or to move the partial states between
 * devices before combining).  Both take exactly the arguments of
 * lrkv_decode; each ignores the ones it does not use (partial: b_v, out;
 * combine: the cache pointers, q, b_k, scale).  lrkv_decode_partial runs the
 * split-K scan and leaves, in the workspace, one partial softmax state per
 * (sequence, partition, head): running max, running sum and the unnormalised
 * sums of a*v_s and a*z^V (Eqs. (6)-(7) restricted to the partition).
 * lrkv_decode_combine merges those states by log-sum-exp and applies B^V_h
 * once per head.  The same sizes, seq_lens, max_len and split_tokens must be
 * passed to both, and the workspace must not change in between. */
lrkv_status lrkv_decode_partial(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim,
                                int32_t rank, int64_t capacity,
                                const void* k_shared, const void* v_shared,
                                const void* z_k, const void* z_v,
                                const int32_t* seq_lens, int64_t max_len,
                                const void* q, const void* b_k, const void* b_v, float scale,
                                int32_t split_tokens, void* out,
                                void* workspace, size_t workspace_bytes, void* stream);
lrkv_status lrkv_decode_combine(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim,
                                int32_t rank, int64_t capacity,
                                const void* k_shared, const void* v_shared,
                                const void* z_k, const void* z_v,
                                const int32_t* seq_lens, int64_t max_len,
                                const void* q, const void* b_k, const void* b_v, float scale,
                                int32_t split_tokens, void* out,
                                void* workspace, size_t workspace_bytes, void* stream);

/* lrkv_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments and result as lrkv_decode, without the workspace.  The
 * split-K partial states go to a scratch array the library holds in device
 * memory, 16 MiB per device (allocated with the code object, held until the
 * process ends).  This call allocates nothing and calls no allocating
 * routine.  A call whose lrkv_decode_workspace_size exceeds 16 MiB returns
 * LRKV_ERR_SCRATCH before any launch (the default split of every shape with
 * batch*num_heads*(head_dim+rank) <= 4M fp32 per resident workgroup fits;
 * the 32 x 8192-token headline shape needs 4.6 MiB).  All calls on one
 * device share that device's scratch, so calls that overlap in time on one
 * device (two streams, or two host threads) race and give wrong results;
 * calls ordered on one stream are safe.  The first call on a device looks up
 * the scratch address once (no allocation; LRKV_ERR_DEVICE if it fails). */
lrkv_status lrkv_decode_noalloc(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim,
                                int32_t rank, int64_t capacity,
                                const void* k_shared, const void* v_shared,
                                const void* z_k, const void* z_v,
                                const int32_t* seq_lens, int64_t max_len,
                                const void* q, const void* b_k, const void* b_v, float scale,
                                int32_t split_tokens, void* out, void* stream);

/* lrkv_decode with an explicit choice of scan kernel, and of the phases to
 * run (for comparing the two scans on one shape, and timing them apart).
 *   engine  0: the default for the shape (as lrkv_decode_scan_kernel names);
 *           1: the vector-ALU scan, decode_split_kernel (the shapes of the
 *              tuned envelope), with its fixed splits;
 *           2: the MFMA scan, decode_mfma_kernel (only its shapes; others
 *              return LRKV_ERR_SHAPE);
 *           3: the any-rank scan, decode_generic_kernel, with its merge
 *              (every shape of the decode envelope);
 *           4: the any-rank MFMA scan, decode_mfma_any_kernel, with the
 *              any-rank merge (only its shapes).
 *   phases  1: the split-K scan (as lrkv_decode_partial), 2: the merge (as
 *           lrkv_decode_combine), 3: both (as lrkv_decode).
 * The remaining arguments are lrkv_decode's.  The workspace must be at least
 * lrkv_decode_workspace_size_ex(engine, ...) bytes for the same sizes and
 * split; the two phases of one decode must use the same engine. */
lrkv_status lrkv_decode_workspace_size_ex(int32_t engine, int32_t dtype, int32_t batch, int32_t num_heads,
                                          int32_t head_dim, int32_t rank, int64_t capacity,
                                          int64_t max_len, int32_t split_tokens, size_t* bytes);
lrkv_status lrkv_decode_ex(int32_t engine, int32_t phases,
                           int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim,
                           int32_t rank, int64_t capacity,
                           const void* k_shared, const void* v_shared,
                           const void* z_k, const void* z_v,
                           const int32_t* seq_lens, int64_t max_len,
                           const void* q, const void* b_k, const void* b_v, float scale,
                           int32_t split_tokens, void* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Name of the kernel lrkv_prefill and lrkv_prefill_chunk run for these
 * sizes: "prefill_kernel" (bf16 MFMA: head_dim 64 or 128, rank 0, 8, 16 or
 * 32), "prefill_wide_kernel" (the same with padded latents at the other
 * ranks up to 128, see lrkv_prefill) or
 * "prefill_generic_kernel" (vector ALU, fp32 arithmetic: the other shapes
 * with rank <= 128, head_dim 16-128 a multiple of 8, at most 65535 heads).
 * NULL outside all three.  Host-only: launches nothing; the string is
 * static. */
const char* lrkv_prefill_kernel(int32_t dtype, int32_t num_heads, int32_t head_dim, int32_t rank);

/* Causal prefill of seq_len fresh tokens per sequence (slides "Compute
 * logits without expanding historical keys" and "Aggregate values before
 * the residual up-projection" with seq_len queries; query i sees keys
 * j <= i):
 *   q   [batch][seq_len][num_heads][head_dim];  out same shape.
 *   k_s, v_s [batch][seq_len][head_dim];  z_k, z_v [batch][seq_len][num_heads][rank].
 * bf16 with head_dim 64 or 128 runs on bf16 MFMA with fp32 accumulation at
 * ranks 0, 8, 16 and 32, and with latents padded to 64 or 128 rows per head
 * at every other rank up to 128 except: an odd rank with an odd number of
 * heads, and ranks 123, 125 and 127.  There one sequence's rows and latents
 * must each span less than 4 GiB - 1 KiB (seq_len * max(head_dim,
 * num_heads*rank) * 2 bytes), else LRKV_ERR_SHAPE.  The other shapes with
 * rank <= 128 and head_dim 16-128 (a multiple of 8), at most 65535 heads and
 * sequences (fp32; the bf16 exceptions above; bf16 at head_dim 16 or 32)
 * run on a vector-ALU kernel with fp32 arithmetic (lrkv_prefill_kernel
 * names the kernel); anything else is LRKV_ERR_SHAPE.
 * If the cache pointers are all non-NULL (k_shared, v_shared, and for
 * rank > 0 also z_k, z_v) the tokens are also written, bit-exactly, to cache
 * slots [0, seq_len) of every sequence (seq_len must then be <= capacity);
 * if they are all NULL the cache is not touched. */
lrkv_status lrkv_prefill(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim,
                         int32_t rank, int64_t capacity,
                         void* k_shared, void* v_shared, void* z_k, void* z_v,
                         int32_t seq_len, const void* q,
                         const void* k_s, const void* v_s, const void* z_k_new, const void* z_v_new,
                         const void* b_k, const void* b_v, float scale, void* out, void* stream);

/* A prefill chunk, or a decode step of several tokens, over cached history:
 * n_new new tokens per sequence attend causally to the tokens already in the
 * cache and to each other (slide "Compute logits without expanding historical
 * keys" with historical keys in front of the causal mask).  For sequence b
 * with s = start_pos[b] tokens already cached:
 *   1. the new tokens are written, bit-exactly, to cache slots [s, s + n_new);
 *   2. new token i (position s + i) attends to cache tokens j <= s + i, in the
 *      absorbed form of Eqs. (6)-(7), on the same kernel lrkv_prefill takes
 *      for the shape.
 *   start_pos  device int32 [batch]; each value is clamped to [0, max_start].
 *   max_start  host upper bound on start_pos; max_start + n_new <= capacity
 *              (else LRKV_ERR_CAPACITY).
 *   q    [batch][n_new][num_heads][head_dim];  out same shape.
 *   k_s, v_s [batch][n_new][head_dim];  z_k_new, z_v_new [batch][n_new][num_heads][rank].
 *   The cache pointers are required (the cache is read and written; z_k and
 *   z_v may be NULL when rank == 0).
 * The shapes are those of lrkv_prefill.  On the MFMA kernels one sequence's
 * history and new tokens must span less than 4 GiB - 1 KiB ((max_start +
 * n_new) * max(head_dim, num_heads*rank) * 2 bytes), else LRKV_ERR_SHAPE.  With
 * start_pos all zero and an empty cache this is lrkv_prefill with the cache
 * written. */
lrkv_status lrkv_prefill_chunk(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim,
                               int32_t rank, int64_t capacity,
                               void* k_shared, void* v_shared, void* z_k, void* z_v,
                               const int32_t* start_pos, int32_t max_start, int32_t n_new,
                               const void* q, const void* k_s, const void* v_s,
                               const void* z_k_new, const void* z_v_new,
                               const void* b_k, const void* b_v, float scale, void* out, void* stream);

/* Training forward: the causal prefill of lrkv_prefill over fresh sequences
 * (no cache), also returning each query row's log-sum-exp for the backward
 * pass (slide "Training learns the base and residuals together": the base
 * and the residual factors are trained jointly, so the attention's
 * gradients reach K_s, V_s, the latents and B_h).
 *   q, out   [batch][seq_len][num_heads][head_dim];
 *   k_s, v_s [batch][seq_len][head_dim];  z_k, z_v [batch][seq_len][num_heads][rank];
 *   b_k, b_v [num_heads][head_dim][rank];
 *   lse      fp32 [batch][seq_len][num_heads], caller-allocated:
 *            lse[b][i][h] = ln sum_{j <= i} exp(scale * q_{b,i,h} . k_{h,j}).
 * Envelope: dtype LRKV_BF16, head_dim 64 or 128, rank 0, 8, 16 or 32,
 * num_heads a multiple of 4; else LRKV_ERR_SHAPE (LRKV_ERR_DTYPE for an
 * unknown dtype).  batch*seq_len below 2^31 and one sequence's rows and
 * latents under 4 GiB, else LRKV_ERR_SHAPE.  scale <= 0 or not finite means
 * 1/sqrt(head_dim).  Tensors 16-byte aligned, lse 4-byte aligned.  batch or
 * seq_len 0 writes nothing. */
lrkv_status lrkv_train_forward(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim,
                               int32_t rank, int32_t seq_len, const void* q,
                               const void* k_s, const void* v_s, const void* z_k, const void* z_v,
                               const void* b_k, const void* b_v, float scale, void* out, float* lse,
                               void* stream);

/* Workspace bytes lrkv_train_backward needs for these sizes (same envelope
 * and errors as lrkv_train_forward; NULL bytes gives LRKV_ERR_NULL). */
lrkv_status lrkv_train_backward_workspace_size(int32_t dtype, int32_t batch, int32_t num_heads,
                                               int32_t head_dim, int32_t rank, int32_t seq_len,
                                               size_t* bytes);

/* Training backward: the vector-Jacobian product of lrkv_train_forward's
 * output with the upstream gradient d_out (same layout and dtype as out),
 * through the absorbed forms of Eqs. (6)-(7) and then through
 * K_h = K_s + Z^K_h (B^K_h)^T and V_h = V_s + Z^V_h (B^V_h)^T (slide
 * "LRKV constrains differences between heads"):
 *   dq   fp32 [batch][seq_len][num_heads][head_dim];
 *   dk_s, dv_s fp32 [batch][seq_len][head_dim]   (summed over heads);
 *   dz_k, dz_v fp32 [batch][seq_len][num_heads][rank];
 *   db_k, db_v fp32 [num_heads][head_dim][rank]  (summed over sequences and tokens).
 * out and lse are the forward's outputs for the same inputs and scale.
 * Every gradient is overwritten (not accumulated into).  The probabilities
 * and their gradients enter bf16 MFMAs; all sums are fp32, in a fixed order
 * (results are deterministic).  workspace: at least
 * lrkv_train_backward_workspace_size bytes, 16-byte aligned, contents on
 * entry ignored.  batch or seq_len 0 only sets db_k and db_v to zero (rank
 * > 0).  Envelope and errors as lrkv_train_forward, plus
 * LRKV_ERR_WORKSPACE; gradient pointers need 4-byte alignment, dq 16. */
lrkv_status lrkv_train_backward(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim,
                                int32_t rank, int32_t seq_len, const void* q,
                                const void* k_s, const void* v_s, const void* z_k, const void* z_v,
                                const void* b_k, const void* b_v, const void* out, const float* lse,
                                const void* d_out, float scale,
                                float* dq, float* dk_s, float* dv_s, float* dz_k, float* dz_v,
                                float* db_k, float* db_v,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Packs the key/value projection weights into the output-major matrix that
 * lrkv_project_append reads (slide "LRKV constrains differences between
 * heads", Eqs. (2)-(3): each head's projection is W_shared + U_h B_h^T, and
 * the cache keeps only the products with W_shared and U_h).
 *   wk_shared, wv_shared  [d_model][head_dim];  u_k, u_v [num_heads][d_model][rank].
 *   w_packed  [2(head_dim + num_heads*rank)][d_model], caller-allocated:
 *     row n < head_dim is column n of wk_shared, the next head_dim rows the
 *     columns of wv_shared, row 2 head_dim + h*rank + j column j of u_k[h],
 *     and the last num_heads*rank rows the same for u_v.
 * Elements are copied bit-exactly.  Weights change rarely, so this runs once
 * per weight update, not per step.  Pointers need only element alignment;
 * u_k and u_v may be NULL when rank == 0. */
lrkv_status lrkv_pack_projection(int32_t dtype, int32_t num_heads, int32_t head_dim, int32_t rank,
                                 int32_t d_model, const void* wk_shared, const void* wv_shared,
                                 const void* u_k, const void* u_v, void* w_packed, void* stream);

/* Name of the kernel lrkv_project_append runs for these sizes on the current
 * device, with (with_workspace != 0) or without a workspace:
 * "project_gemm_kernel" (bf16 MFMA, 256-row tiles, when they are at least as
 * many as the device's compute units), "project_splitk_kernel" (bf16 MFMA,
 * at most 64 rows, with a workspace: the contraction split across
 * workgroups, then a reduction kernel), "project_skinny_kernel" (the same
 * rows without a workspace: one workgroup per 32 output columns),
 * "project_append_kernel" (bf16 MFMA, 128 x 128 tiles, the rows in between)
 * or "project_append_valu_kernel" (fp32, and bf16 widths that are not
 * multiples of 32).  NULL for invalid sizes.  Host-only: launches nothing;
 * the string is static. */
const char* lrkv_project_kernel(int32_t dtype, int32_t batch, int32_t n_new, int32_t num_heads, int32_t head_dim,
                                int32_t rank, int32_t d_model, int32_t with_workspace);

/* Bytes of device workspace with which lrkv_project_append splits the
 * contraction of these sizes across workgroups (fp32 partial sums); 0 where
 * the sizes have no use for one.  Written to *bytes. */
lrkv_status lrkv_project_workspace_size(int32_t dtype, int32_t batch, int32_t n_new, int32_t num_heads,
                                        int32_t head_dim, int32_t rank, int32_t d_model, size_t* bytes);

/* Fused projection + append: the cache rows of n_new new tokens computed from
 * their hidden states and written straight into the cache (slide "Cache
 * shared features and compact per-head latents", Eqs. (4)-(5)): for token i
 * of sequence b with hidden state x = x[b][i] (width d_model),
 *   k_s = x W^K_shared,  v_s = x W^V_shared,  z^K_h = x U^K_h,  z^V_h = x U^V_h,
 * as one product x . w_packed^T (w_packed from lrkv_pack_projection), fp32
 * accumulation, each result rounded once to dtype and stored at cache slot
 * pos[b] + i of its array.  Slots outside [0, capacity) are dropped, as in
 * lrkv_append.
 *   x    [batch][n_new][d_model];  pos device int32 [batch].
 *   workspace  optional (NULL, or at least lrkv_project_workspace_size
 *        bytes, 16-byte aligned; contents on entry ignored): for a few tokens
 *        it lets the contraction spread over more workgroups.  A smaller one
 *        is not used.
 * bf16 with head_dim, num_heads*rank and d_model multiples of 32 runs on bf16
 * MFMA; other shapes and fp32 on vector-ALU fused multiply-adds.  x, w_packed
 * and the cache pointers must be 16-byte aligned; z_k and z_v may be NULL
 * when rank == 0.  batch*n_new must be below 2^31 and d_model at most 65536,
 * else LRKV_ERR_SHAPE. */
lrkv_status lrkv_project_append(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim,
                                int32_t rank, int64_t capacity,
                                void* k_shared, void* v_shared, void* z_k, void* z_v,
                                const int32_t* pos, int32_t n_new, int32_t d_model,
                                const void* x, const void* w_packed, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Plain multi-head attention decode over a full per-head K/V cache, the
 * baseline LRKV's cache is compared with at a matched shape (slide "Can
 * heads share storage while keeping distinct K/V features?": MHA caches
 * 2 num_heads head_dim elements per token per layer).  For every sequence b
 * and head h:
 *   out[b][h] = softmax_t(scale * q_bh . k[b][t][h]) applied to v[b][t][h],
 *               t < seq_lens[b].
 *   k, v      [batch][capacity][num_heads][head_dim];  q, out [batch][num_heads][head_dim].
 *   seq_lens, max_len, scale: as for lrkv_decode (lengths clamped to
 *             [0, max_len], a sequence of length 0 gets zeros).
 *   split_tokens  tokens per split (0 = default, else a positive multiple of
 *             64); one split's rows must span less than 4 GiB.
 *   workspace at least lrkv_mha_decode_workspace_size bytes; contents on
 *             entry are ignored.
 * head_dim must be 64 or 128.  Partial states per (split, head) are merged
 * by the same log-sum-exp combine as lrkv_decode. */
lrkv_status lrkv_mha_decode_workspace_size(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim,
                                           int64_t capacity, int64_t max_len, int32_t split_tokens,
                                           size_t* bytes);
lrkv_status lrkv_mha_decode(int32_t dtype, int32_t batch, int32_t num_heads, int32_t head_dim, int64_t capacity,
                            const void* k, const void* v, const int32_t* seq_lens, int64_t max_len,
                            const void* q, float scale, int32_t split_tokens, void* out,
                            void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LRKV_H */
