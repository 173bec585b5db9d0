/*
 * gqa.h - C ABI of libgqa.so: grouped-query attention (GQA) over a KV cache
 * on AMD Instinct MI355X (gfx950).
 *
 * The operation.  A layer has Hq query heads and Hkv key/value heads, with
 * Hkv >= 1 dividing Hq; g = Hq / Hkv query heads form a group, and query
 * head h reads KV head h / g (integer division), i.e. consecutive blocks of
 * g query heads share one KV head (study.greatitself.com, "Grouped-Query and
 * Multi-Query Attention", section "Share keys and values without confusing
 * query-head identity"; lihaoran.work, section "Shared KV can still produce
 * different outputs").  For every query head the output is
 *
 *     out[h] = sum_t softmax_t(scale * q[h] . K[h/g, t]) * V[h/g, t]
 *
 * with its own distribution per query head.  The shared K/V rows are read in
 * place, once per group of query heads, and never copied per query head
 * (anrans.github.io, "Attention variants: MQA, GQA, MLA", section "Kernels do
 * not need to copy the KV heads").  MHA is Hkv = Hq and MQA is Hkv = 1.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or retains them.  Tensors are dense, row-major,
 *    head-major, with the shapes written next to each argument.
 *  - q, k, v, out and the workspace must be 16-byte aligned; lse and seq_lens
 *    4-byte aligned.
 *  - dtype selects the element type of q, k and v (gqa_dtype).  Outputs are
 *    always float32 (fp32 accumulation of bf16 products).
 *  - stream is a hipStream_t (NULL = the legacy default stream).  Calls only
 *    validate and enqueue; they return before the GPU work finishes, and a
 *    fault during execution surfaces at the caller's next synchronisation.
 *  - Arguments are validated on the host before any HIP call, so a bad call
 *    returns an error status and enqueues nothing.  Statuses are gqa_status
 *    values returned as int32_t; nothing is printed and nothing throws.
 *  - The library keeps no state besides a thread-local copy of the last HIP
 *    error text, so it is reentrant; two calls that share a workspace must
 *    be ordered on one stream.
 */
#ifndef GQA_H_
#define GQA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GQA_ABI_VERSION 1

typedef enum gqa_status {
  GQA_OK = 0,
  GQA_ERR_NULL = 1,        /* a required pointer is NULL                         */
  GQA_ERR_SHAPE = 2,       /* size < 1, Hkv not dividing Hq, or size overflow    */
  GQA_ERR_UNSUPPORTED = 3, /* head_dim not 64/128, dtype not allowed, bad range  */
  GQA_ERR_WORKSPACE = 4,   /* workspace smaller than the planning call requires  */
  GQA_ERR_HIP = 5,         /* the HIP runtime rejected a launch                  */
  GQA_ERR_ALIGN = 6        /* a pointer violates the alignment rule above        */
} gqa_status;

typedef enum gqa_dtype {
  GQA_F32 = 0,  /* IEEE float32                          */
  GQA_BF16 = 1, /* bfloat16 (upper half of a float32)     */
  GQA_FP8_E4M3 = 2 /* bf16 q with a KV cache of OCP E4M3 codes and per-KV-head
                      float32 scales (gqa_decode_fp8); valid for the plan,
                      gqa_decode_fp8* and gqa_decode_merge */
} gqa_dtype;

/* Version of this ABI (GQA_ABI_VERSION). */
int32_t gqa_abi_version(void);

/* Static, NUL-terminated name of a status code ("GQA_OK", ...); an unknown
 * code gives "GQA_ERR_UNKNOWN".  gqa_status_str is the same function under
 * the short name. */
const char* gqa_status_string(int32_t status);
const char* gqa_status_str(gqa_status status);

/* Text of the last HIP error seen by a call on this thread ("" if none). */
const char* gqa_last_hip_error(void);

/* Compute units and peak shader clock (kHz) of HIP device `device`, as
 * hipDeviceGetAttribute reports them, for deriving the roofline peaks of the
 * board a measurement runs on (the dense bf16 matrix-core rate is compute
 * units x 4,096 FLOP per clock on gfx950).  Host-side query, synchronous; no
 * kernel runs.  Errors: a null output pointer -> GQA_ERR_NULL (checked before
 * any HIP call), a failed query -> GQA_ERR_HIP (outputs left unchanged; this
 * call does not record the HIP error's text for gqa_last_hip_error). */
int32_t gqa_device_info(int32_t device, int32_t* compute_units, int32_t* max_clock_khz);

/*
 * Launch plan of a decode call.  Decode lays the cached tokens of every
 * (sequence, KV head, block of up to 16 query heads; for bf16 and E4M3
 * caches when the group has more than 16, up to 32 at head_dim 128 and up
 * to 80 at head_dim 64) end to end into one
 * stream and cuts it into equal ranges, one per workgroup, so ragged batches
 * stay balanced; a range's piece inside one sequence is attended by one
 * workgroup for all query heads of the group, and a sequence that spans
 * several pieces is finished by a log-sum-exp merge.  This partition is an
 * implementation choice, not something the pages specify.
 *
 * split_tokens: 0 lets the device size the ranges from the actual lengths
 *   (about one range per resident workgroup); otherwise a positive multiple
 *   of 32 that fixes the range size (GQA_ERR_UNSUPPORTED if not).
 * Outputs (any may be NULL): the fixed range size (0 when chosen on the
 *   device), the number of workgroups launched, and the workspace bytes that
 *   gqa_decode / gqa_decode_split / gqa_decode_merge need for this shape.
 * Pure host arithmetic: never touches the GPU.
 */
int32_t gqa_decode_plan(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t max_seq_len, int32_t dtype,
                        int32_t split_tokens, int32_t* range_tokens_out,
                        int32_t* workgroups_out, int64_t* workspace_bytes_out);

/*
 * Workspace bytes that cover gqa_decode (and its two stages) for every
 * number of KV heads that divides num_q_heads, every dtype and automatic
 * ranges (split_tokens = 0), given only the batch, the query heads, the head
 * dimension and the cache capacity: the largest size gqa_decode_plan reports
 * over those KV-head counts.  Returns 0 when the arguments are invalid (a
 * size below 1, head_dim not 64 or 128, or a size overflow).  Pure host
 * arithmetic.
 */
size_t gqa_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_seq_len);

/*
 * One decode step of GQA over a KV cache: every query head of every sequence
 * attends to the first seq_lens[b] cached tokens of its KV head.
 *
 *   q         [batch, num_q_heads, head_dim]                     dtype
 *   k_cache   [batch, num_kv_heads, max_seq_len, head_dim]       dtype
 *   v_cache   [batch, num_kv_heads, max_seq_len, head_dim]       dtype
 *   seq_lens  [batch] int32, device memory, never read on the host; values
 *             are clamped to [0, max_seq_len]; slots past seq_lens[b] are
 *             never read (they may hold garbage, NaN included).  A length of
 *             0 gives an all-zero output row.
 *   out       [batch, num_q_heads, head_dim] float32
 *   scale     multiplies q . k (1/sqrt(head_dim) for standard attention)
 *   dtype     GQA_F32 or GQA_BF16; head_dim 64 or 128
 *   workspace device scratch of at least the bytes gqa_decode_plan reports
 *             (its contents on entry do not matter; they are overwritten)
 *
 * Runs gqa_decode_split then gqa_decode_merge on the same stream.
 * Limits: max_seq_len * head_dim * 4 < 2^31.
 */
int32_t gqa_decode(const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* seq_lens, float* out, int32_t batch,
                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                   int32_t max_seq_len, float scale, int32_t dtype,
                   int32_t split_tokens, void* workspace, int64_t workspace_bytes,
                   void* stream);

/*
 * gqa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, and harnesses that forbid hipMalloc.
 * Same arguments, result and errors as gqa_decode, minus the workspace: the
 * library keeps a device scratch array of 16 MiB per GPU (it exists from
 * the library's load until the process ends) and this call neither
 * allocates nor frees anything.  A shape whose workspace (gqa_decode_plan)
 * exceeds 16 MiB gets GQA_ERR_WORKSPACE; fp32 and bf16 only.
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (different streams, or threads without ordering) race and must be
 * serialised by the caller.
 */
int32_t gqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* seq_lens, float* out, int32_t batch,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t max_seq_len, float scale, int32_t dtype,
                           int32_t split_tokens, void* stream);

/*
 * First stage of gqa_decode (the kernel that reads the KV cache).  Rows of
 * out whose sequence falls in a single range are written in final form;
 * every other (sequence, query head) leaves one normalised partial output
 * and its log-sum-exp per range in the workspace, with an index of them.
 * Arguments as for gqa_decode.
 */
int32_t gqa_decode_split(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* seq_lens, float* out, int32_t batch,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t max_seq_len, float scale, int32_t dtype,
                         int32_t split_tokens, void* workspace, int64_t workspace_bytes,
                         void* stream);

/*
 * Second stage of gqa_decode: the remaining rows of out [batch, num_q_heads,
 * head_dim] float32, each the combination of its partials weighted by
 * exp(lse_c - max_c lse_c), and zeros for empty sequences.  The shape
 * arguments must equal those of the gqa_decode_split call that filled the
 * workspace, with no other use of the workspace in between.
 */
int32_t gqa_decode_merge(const int32_t* seq_lens, float* out, int32_t batch,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t max_seq_len, int32_t dtype, int32_t split_tokens,
                         const void* workspace, int64_t workspace_bytes, void* stream);

/*
 * One decode step over a paged KV cache: the same attention as gqa_decode,
 * with the cache stored in a shared pool of fixed-size pages addressed
 * through a block table (deepconcepts.dev, "Grouped-Query Attention",
 * section "Checking it on a real system": paged attention changes how the
 * cache bytes are stored, not what attention computes; lihaoran.work,
 * "Check the actual deployment": it acts on cache organisation, GQA on
 * sharing structure).
 *
 *   k_pages, v_pages  [num_pages, num_kv_heads, page_size, head_dim] bf16
 *   block_table       [batch, max_pages_per_seq] int32, device memory:
 *                     entry [b, i] is the page holding tokens
 *                     i*page_size .. (i+1)*page_size - 1 of sequence b.
 *                     Only entries covering tokens below seq_lens[b] are
 *                     read; an entry outside [0, num_pages) is clamped into
 *                     the pool (wrong output, never an out-of-bounds read).
 *   page_size         a power of two, 1 .. 65536
 *   seq_lens          as for gqa_decode, clamped to [0, max_pages_per_seq *
 *                     page_size]
 *   workspace         at least what gqa_decode_plan reports for
 *                     max_seq_len = max_pages_per_seq * page_size
 *   dtype             GQA_BF16 only; head_dim 64 or 128
 * Other arguments as for gqa_decode (the two stages run on the same stream).
 */
int32_t gqa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                         const int32_t* block_table, const int32_t* seq_lens, float* out,
                         int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t page_size, int32_t num_pages,
                         int32_t max_pages_per_seq, float scale, int32_t dtype,
                         int32_t split_tokens, void* workspace, int64_t workspace_bytes,
                         void* stream);

/*
 * First stage of gqa_decode_paged (the kernel that reads the pages), with the
 * same outputs and workspace contents as gqa_decode_split; gqa_decode_merge
 * with max_seq_len = max_pages_per_seq * page_size completes it.  Arguments
 * as for gqa_decode_paged.
 */
int32_t gqa_decode_paged_split(const void* q, const void* k_pages, const void* v_pages,
                               const int32_t* block_table, const int32_t* seq_lens, float* out,
                               int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t page_size, int32_t num_pages,
                               int32_t max_pages_per_seq, float scale, int32_t dtype,
                               int32_t split_tokens, void* workspace, int64_t workspace_bytes,
                               void* stream);

/*
 * One decode step over an FP8 KV cache (deepconcepts.dev, "Grouped-Query
 * Attention", section "Checking it on a real system": quantising the cache
 * halves its bytes again; anrans.github.io, "Other ways to shrink the KV
 * cache": K and V stored in FP8).  The cache holds OCP E4M3 codes (sign, 4
 * exponent bits with bias 7, 3 mantissa bits); the value of a code of KV
 * head kv is code_value * k_scale[kv] (K) or * v_scale[kv] (V).  Attention
 * is then exactly that of gqa_decode over the decoded values.
 *
 *   q                 [batch, num_q_heads, head_dim] bf16
 *   k_cache, v_cache  [batch, num_kv_heads, max_seq_len, head_dim] uint8 codes
 *   k_scale, v_scale  [num_kv_heads] float32, device memory
 *   workspace         at least what gqa_decode_plan reports with dtype
 *                     GQA_FP8_E4M3
 * Other arguments, limits and errors as for gqa_decode; head_dim 64 or 128.
 * Codes of cached tokens are read as stored (NaN codes give NaN outputs);
 * slots past seq_lens[b] are never read.
 */
int32_t gqa_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                       const float* k_scale, const float* v_scale, const int32_t* seq_lens,
                       float* out, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t max_seq_len, float scale, int32_t split_tokens,
                       void* workspace, int64_t workspace_bytes, void* stream);

/*
 * First stage of gqa_decode_fp8 (the kernel that reads the cache); complete
 * it with gqa_decode_merge (dtype GQA_FP8_E4M3).  Arguments as for
 * gqa_decode_fp8.
 */
int32_t gqa_decode_fp8_split(const void* q, const void* k_cache, const void* v_cache,
                             const float* k_scale, const float* v_scale, const int32_t* seq_lens,
                             float* out, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t max_seq_len, float scale, int32_t split_tokens,
                             void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Decode over wide cached rows that are both key and value: the decode shape
 * of multi-head latent attention with weight absorption, in which all query
 * heads share one cached latent row per token that serves as the key and,
 * in its leading columns, as the value (anrans.github.io, "Attention
 * variants: MQA, GQA, MLA", section "MLA: multi-head latent attention":
 * 512 latent + 64 rotary-key columns, an MQA with a very large head
 * dimension).  For query head h and KV head j = h / g:
 *
 *     out[h] = sum_t softmax_t(scale * q[h] . row[j, t]) * row[j, t][0 : head_dim_v]
 *
 *   q        [batch, num_q_heads, head_dim_qk]               bf16 (absorbed query
 *            followed by the rotary query)
 *   kv_cache [batch, num_kv_heads, max_seq_len, head_dim_qk] bf16 (latent row
 *            followed by the rotary key); rows at or past seq_lens[b] are never read
 *   seq_lens [batch] int32 on the device, clamped to 0 .. max_seq_len
 *   out      [batch, num_q_heads, head_dim_v] float32; a sequence with no
 *            tokens gets zeros
 *   head_dim_qk must be 576 and head_dim_v 512 (GQA_ERR_UNSUPPORTED
 *   otherwise); any group size g.  Limits: (max_seq_len + 64) * 1152 < 2^31.
 *   split_tokens  0 = automatic token ranges per (sequence, KV head), else a
 *                 positive multiple of 32 tokens per range
 *   workspace     partial results when a sequence spans several ranges: at
 *                 least what gqa_decode_wide_plan reports (may be NULL when
 *                 that is 0), 16-byte aligned
 *
 * gqa_decode_wide_plan reports, for the same arguments, the number of token
 * ranges per sequence and the workspace bytes.  Errors as gqa_decode.
 */
int32_t gqa_decode_wide_plan(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim_qk, int32_t head_dim_v, int32_t max_seq_len,
                             int32_t split_tokens, int32_t* ranges_out,
                             int64_t* workspace_bytes_out);

int32_t gqa_decode_wide(const void* q, const void* kv_cache, const int32_t* seq_lens, float* out,
                        int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim_qk, int32_t head_dim_v, int32_t max_seq_len, float scale,
                        int32_t split_tokens, void* workspace, int64_t workspace_bytes,
                        void* stream);

/*
 * Causal GQA over a whole prompt (prefill): query row i of head h attends to
 * keys 0..i of KV head h / g (lower-triangular mask broadcast over the
 * group; anrans.github.io, "Kernels do not need to copy the KV heads").
 *
 *   q    [batch, num_q_heads, seq_len, head_dim]   bf16
 *   k, v [batch, num_kv_heads, seq_len, head_dim]  bf16
 *   out  [batch, num_q_heads, seq_len, head_dim]   float32
 *   lse  [batch, num_q_heads, seq_len] float32 natural log-sum-exp of the
 *        scaled scores of each row, or NULL to skip it
 *   dtype must be GQA_BF16; head_dim 64 or 128.
 * Limits: seq_len * head_dim * 4 < 2^31 (GQA_ERR_SHAPE otherwise).
 */
int32_t gqa_prefill_causal(const void* q, const void* k, const void* v, float* out,
                           float* lse, int32_t batch, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t seq_len, int32_t head_dim,
                           float scale, int32_t dtype, void* stream);

/*
 * Workspace bytes that gqa_prefill_causal_backward needs for this shape
 * (two floats per query row, rounded up to 256 bytes).  Same shape rules and
 * statuses as gqa_prefill_causal with dtype GQA_BF16.
 */
int32_t gqa_prefill_backward_workspace(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t seq_len, int32_t head_dim,
                                       int64_t* workspace_bytes_out);

/*
 * Gradients of causal GQA prefill (the training backward pass).  A shared
 * K or V row collects gradient from every query head of its group: dk and
 * dv of KV head j are sums over query heads j*g .. j*g+g-1, formed inside
 * the library without copying K/V per query head and without per-head
 * gradient buffers (study.greatitself.com, "Grouped-Query and Multi-Query
 * Attention", section "Share keys and values without confusing query-head
 * identity", training paragraph).  With P the causal softmax of one query
 * head and dout the gradient of the loss with respect to its output:
 *
 *     dv[j] = sum_h P_h^T dout_h            dS_h = P_h * (dout_h V^T - rowsum(dout_h * out_h))
 *     dq_h  = scale dS_h K[j]               dk[j] = scale sum_h dS_h^T q_h
 *
 *   q, dout [batch, num_q_heads, seq_len, head_dim]   bf16
 *   k, v    [batch, num_kv_heads, seq_len, head_dim]  bf16
 *   out     [batch, num_q_heads, seq_len, head_dim]   float32, and
 *   lse     [batch, num_q_heads, seq_len]             float32: the out and lse
 *           that gqa_prefill_causal returned for the same q, k, v and scale
 *           (P is recomputed from lse; out only enters rowsum(dout * out))
 *   dq      [batch, num_q_heads, seq_len, head_dim]   float32, overwritten
 *   dk, dv  [batch, num_kv_heads, seq_len, head_dim]  float32, overwritten
 *   workspace   device scratch of at least gqa_prefill_backward_workspace
 *               bytes, 16-byte aligned; its contents on entry do not matter
 *   dtype must be GQA_BF16; head_dim 64 or 128.
 *
 * Two kernels run in order on `stream`; results are bitwise reproducible
 * (no atomics).  Errors: GQA_ERR_NULL for any NULL pointer (lse is required
 * here), GQA_ERR_WORKSPACE for a short workspace, otherwise as
 * gqa_prefill_causal.
 */
int32_t gqa_prefill_causal_backward(const void* q, const void* k, const void* v, const float* out,
                                    const float* lse, const void* dout, float* dq, float* dk,
                                    float* dv, int32_t batch, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t seq_len, int32_t head_dim,
                                    float scale, int32_t dtype, void* workspace,
                                    int64_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H_ */
