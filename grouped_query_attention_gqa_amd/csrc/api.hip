// C ABI of libgqa.so (declared in include/gqa.h): argument validation, split
// planning and kernel launches.  Validation is pure host arithmetic done
// before any HIP call, so every error path is reachable without a GPU.

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include <hip/hip_runtime.h>

#include "gqa.h"
#include "gqa_launch.hpp"

namespace {

thread_local char g_last_hip_error[256] = "";

int32_t hip_status(hipError_t e) {
  if (e == hipSuccess) return GQA_OK;
  const char* s = hipGetErrorString(e);
  strncpy(g_last_hip_error, s ? s : "unknown HIP error", sizeof(g_last_hip_error) - 1);
  g_last_hip_error[sizeof(g_last_hip_error) - 1] = '\0';
  return GQA_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int32_t check_heads(int32_t batch, int32_t hq, int32_t hkv, int32_t d, int32_t dtype) {
  if (batch < 1 || hq < 1 || hkv < 1 || hq % hkv != 0) return GQA_ERR_SHAPE;
  if (d != 64 && d != 128) return GQA_ERR_UNSUPPORTED;
  if (dtype != GQA_F32 && dtype != GQA_BF16 && dtype != GQA_FP8_E4M3) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

// Decode launch plan: the work is one stream of (unit, token) pairs cut into
// equal ranges (see decode.hip).  With split_tokens == 0 the range size is
// picked on the device from the actual lengths for kPersistentWorkgroups
// resident workgroups; otherwise it is split_tokens.
int32_t make_plan(int32_t batch, int32_t hq, int32_t hkv, int32_t d, int32_t tcap, int32_t dtype,
                  int32_t split_tokens, float scale, gqa::DecodeShape* s) {
  int32_t st = check_heads(batch, hq, hkv, d, dtype);
  if (st != GQA_OK) return st;
  if (tcap < 1) return GQA_ERR_SHAPE;
  if (split_tokens < 0 || split_tokens % gqa::kRangeQuantum != 0) return GQA_ERR_UNSUPPORTED;
  // Element offsets are 64-bit; buffer offsets inside one segment are
  // 32-bit, so one sequence's cache row must stay below 2 GiB.
  const int64_t kv_elems = (int64_t)batch * hkv * (int64_t)tcap * d;
  if (kv_elems / d / tcap / hkv != batch || kv_elems > (INT64_MAX / 8)) return GQA_ERR_SHAPE;
  if ((int64_t)tcap * d * 4 > INT32_MAX) return GQA_ERR_SHAPE;
  const int64_t g = hq / hkv;
  const int64_t nhb = (g + gqa::kDecodeHeadBlock - 1) / gqa::kDecodeHeadBlock;
  // bf16 and E4M3 caches put several head blocks in one unit when the group
  // has more than one block: two at head_dim 128 (one pass over the KV head
  // for up to 32 heads), up to five at head_dim 64 (up to 80 heads)
  const int hbu = (dtype == GQA_F32 || nhb == 1)
                      ? 1
                      : (d == 64 ? (int)std::min<int64_t>(nhb, gqa::kMaxHeadBlocks64) : 2);
  const int64_t nhg = (nhb + hbu - 1) / hbu;
  const int64_t units = (int64_t)batch * hkv * nhg;
  const int64_t work = units * (int64_t)tcap;   // upper bound on token-units
  int64_t ranges, grid;
  if (split_tokens == 0) {
    grid = (work + gqa::kMinRange - 1) / gqa::kMinRange;
    if (grid > gqa::kPersistentWorkgroups) grid = gqa::kPersistentWorkgroups;
    ranges = grid;   // the device picks Q >= W / grid
  } else {
    ranges = (work + split_tokens - 1) / split_tokens;
    grid = ranges < gqa::kPersistentWorkgroups ? ranges : gqa::kPersistentWorkgroups;
  }
  const int64_t slots = ranges + units;
  if (units > INT32_MAX || slots > INT32_MAX / (gqa::kDecodeHeadBlock * hbu)) return GQA_ERR_SHAPE;
  s->batch = batch;
  s->hb = hbu;
  s->nhg = (int)nhg;
  s->hq = hq;
  s->hkv = hkv;
  s->d = d;
  s->tcap = tcap;
  s->units = (int)units;
  s->q_fixed = split_tokens;
  s->grid = (int)grid;
  s->max_slots = slots;
  s->scale = scale;
  s->dtype = dtype;
  return GQA_OK;
}

// Shape rules of the causal prefill entry points (forward and backward).
int32_t check_prefill(int32_t batch, int32_t hq, int32_t hkv, int32_t n, int32_t d, int32_t dtype) {
  int32_t st = check_heads(batch, hq, hkv, d, dtype);
  if (st != GQA_OK) return st;
  if (n < 1) return GQA_ERR_SHAPE;
  if (dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
  const int64_t q_elems = (int64_t)batch * hq * (int64_t)n * d;
  if (q_elems / d / n / hq != batch || q_elems > (INT64_MAX / 8)) return GQA_ERR_SHAPE;
  // one head's rows are addressed with 32-bit buffer offsets
  if ((int64_t)n * d * 4 > INT32_MAX) return GQA_ERR_SHAPE;
  const int64_t g = hq / hkv;
  const int64_t gw = (g % 4 == 0) ? 4 : (g % 2 == 0 ? 2 : 1);
  const int64_t tiles = (n + 128 / gw - 1) / (128 / gw);
  if ((int64_t)batch * hkv * (g / gw) * tiles > INT32_MAX) return GQA_ERR_SHAPE;
  return GQA_OK;
}

// The backward's workspace holds two floats per query row: lse * log2(e)
// and D = rowsum(dout * out).
int64_t backward_workspace_bytes(int32_t batch, int32_t hq, int32_t n) {
  return ((int64_t)batch * hq * n * 8 + 255) / 256 * 256;
}

// Wide-row decode plan: head blocks of kWideHeadBlock, and with
// split_tokens == 0 enough token ranges that about 256 workgroups run.
int32_t make_wide_plan(int32_t batch, int32_t hq, int32_t hkv, int32_t d_k, int32_t d_v, int32_t tcap,
                       int32_t split_tokens, float scale, gqa::WideShape* s) {
  if (batch < 1 || hq < 1 || hkv < 1 || hq % hkv != 0 || tcap < 1) return GQA_ERR_SHAPE;
  if (d_k != gqa::kWideDK || d_v != gqa::kWideDV) return GQA_ERR_UNSUPPORTED;
  if (split_tokens < 0 || split_tokens % gqa::kRangeQuantum != 0) return GQA_ERR_UNSUPPORTED;
  if (((int64_t)tcap + 64) * d_k * 2 > INT32_MAX) return GQA_ERR_SHAPE;   // 32-bit buffer offsets per cache row
  if ((int64_t)hq * d_k * 2 > INT32_MAX) return GQA_ERR_SHAPE;
  const int64_t g = hq / hkv;
  const int64_t nhb = (g + gqa::kWideHeadBlock - 1) / gqa::kWideHeadBlock;
  const int64_t units = (int64_t)batch * hkv * nhb;
  int64_t split = split_tokens;
  if (split == 0) {
    const int64_t want = units >= 256 ? 1 : (256 + units - 1) / units;
    split = (tcap + want - 1) / want;
    split = (split + gqa::kRangeQuantum - 1) / gqa::kRangeQuantum * gqa::kRangeQuantum;
  }
  const int64_t nranges = (tcap + split - 1) / split;
  const int64_t space = (int64_t)batch * hkv * nranges;
  const int64_t grid = (space + 7) / 8 * 8 * nhb;
  if (grid > INT32_MAX || nranges * units * gqa::kWideHeadBlock * gqa::kWideDV > (INT64_MAX / 8))
    return GQA_ERR_SHAPE;
  s->batch = batch;
  s->hq = hq;
  s->hkv = hkv;
  s->tcap = tcap;
  s->nhb = (int)nhb;
  s->units = (int)units;
  s->split = (int)split;
  s->nranges = (int)nranges;
  s->grid = (int)grid;
  s->scale = scale;
  return GQA_OK;
}

// Scratch of gqa_decode_noalloc: device memory that exists from the moment
// the code object is loaded on a GPU until the process ends, one copy per
// GPU, so that the entry point never allocates.  Host code never passes the
// array's name to a kernel (on the host it only names the symbol): it uses
// the device address that hipGetSymbolAddress returns for the current GPU.
constexpr int64_t kNoAllocScratchBytes = 16ll << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<char*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current GPU, looked up on the first
// call on each GPU.  The decode kernels overwrite every scratch byte they
// read (the split kernel writes the unit index and the partials that the
// merge kernel reads), so nothing in it needs clearing.
int32_t noalloc_scratch(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return GQA_ERR_UNSUPPORTED;
  char* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_status(e);
      p = static_cast<char*>(addr);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return GQA_OK;
}

}  // namespace

extern "C" {

int32_t gqa_abi_version(void) { return GQA_ABI_VERSION; }

const char* gqa_status_string(int32_t status) {
  switch (status) {
    case GQA_OK: return "GQA_OK";
    case GQA_ERR_NULL: return "GQA_ERR_NULL";
    case GQA_ERR_SHAPE: return "GQA_ERR_SHAPE";
    case GQA_ERR_UNSUPPORTED: return "GQA_ERR_UNSUPPORTED";
    case GQA_ERR_WORKSPACE: return "GQA_ERR_WORKSPACE";
    case GQA_ERR_HIP: return "GQA_ERR_HIP";
    case GQA_ERR_ALIGN: return "GQA_ERR_ALIGN";
    default: return "GQA_ERR_UNKNOWN";
  }
}

const char* gqa_status_str(gqa_status status) { return gqa_status_string((int32_t)status); }

const char* gqa_last_hip_error(void) { return g_last_hip_error; }

size_t gqa_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_seq_len) {
  // the largest plan over the KV-head counts that divide num_q_heads (bf16
  // plans bound fp32 and E4M3 ones: the same units or fewer, no wider rows)
  int64_t most = 0;
  for (int64_t a = 1; a * a <= num_q_heads; ++a) {
    if (num_q_heads % a != 0) continue;
    const int32_t hkvs[2] = {(int32_t)a, (int32_t)(num_q_heads / a)};
    for (int32_t hkv : hkvs) {
      gqa::DecodeShape s;
      if (make_plan(batch, num_q_heads, hkv, head_dim, max_seq_len, GQA_BF16, 0, 1.f, &s) != GQA_OK) return 0;
      const int64_t t = gqa::decode_workspace_layout(s).total;
      if (t > most) most = t;
    }
  }
  return (size_t)most;
}

int32_t gqa_decode_plan(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t max_seq_len, int32_t dtype,
                        int32_t split_tokens, int32_t* range_tokens_out,
                        int32_t* workgroups_out, int64_t* workspace_bytes_out) {
  gqa::DecodeShape s;
  const int32_t st = make_plan(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, dtype,
                               split_tokens, 1.f, &s);
  if (st != GQA_OK) return st;
  if (range_tokens_out) *range_tokens_out = s.q_fixed;
  if (workgroups_out) *workgroups_out = s.grid;
  if (workspace_bytes_out) *workspace_bytes_out = gqa::decode_workspace_layout(s).total;
  return GQA_OK;
}

static int32_t decode_prepare(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* seq_lens, const void* workspace,
                              int64_t workspace_bytes, int32_t batch, int32_t hq, int32_t hkv,
                              int32_t d, int32_t tcap, float scale, int32_t dtype,
                              int32_t split_tokens, gqa::DecodeShape* s,
                              gqa::DecodeWorkspace* ws) {
  if (!q || !k_cache || !v_cache || !seq_lens || !workspace) return GQA_ERR_NULL;
  const int32_t st = make_plan(batch, hq, hkv, d, tcap, dtype, split_tokens, scale, s);
  if (st != GQA_OK) return st;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(workspace, 16) ||
      !aligned(seq_lens, 4))
    return GQA_ERR_ALIGN;
  *ws = gqa::decode_workspace_layout(*s);
  if (workspace_bytes < ws->total) return GQA_ERR_WORKSPACE;
  return GQA_OK;
}

int32_t gqa_decode_split(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* seq_lens, float* out, int32_t batch, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len,
                         float scale, int32_t dtype, int32_t split_tokens, void* workspace,
                         int64_t workspace_bytes, void* stream) {
  if (!out) return GQA_ERR_NULL;
  if (dtype == GQA_FP8_E4M3) return GQA_ERR_UNSUPPORTED;   // needs the scales: gqa_decode_fp8_split
  gqa::DecodeShape s;
  gqa::DecodeWorkspace ws;
  const int32_t st = decode_prepare(q, k_cache, v_cache, seq_lens, workspace, workspace_bytes, batch,
                                    num_q_heads, num_kv_heads, head_dim, max_seq_len, scale, dtype,
                                    split_tokens, &s, &ws);
  if (st != GQA_OK) return st;
  if (!aligned(out, 16)) return GQA_ERR_ALIGN;
  return hip_status(gqa::launch_decode_split(q, k_cache, v_cache, seq_lens, out,
                                             static_cast<char*>(workspace), s,
                                             static_cast<hipStream_t>(stream)));
}

int32_t gqa_decode_merge(const int32_t* seq_lens, float* out, int32_t batch, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len,
                         int32_t dtype, int32_t split_tokens, const void* workspace,
                         int64_t workspace_bytes, void* stream) {
  if (!seq_lens || !out || !workspace) return GQA_ERR_NULL;
  gqa::DecodeShape s;
  const int32_t st = make_plan(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, dtype,
                               split_tokens, 1.f, &s);
  if (st != GQA_OK) return st;
  if (!aligned(out, 16) || !aligned(workspace, 16) || !aligned(seq_lens, 4)) return GQA_ERR_ALIGN;
  const gqa::DecodeWorkspace ws = gqa::decode_workspace_layout(s);
  if (workspace_bytes < ws.total) return GQA_ERR_WORKSPACE;
  return hip_status(gqa::launch_decode_merge(seq_lens, out, static_cast<const char*>(workspace), s,
                                             static_cast<hipStream_t>(stream)));
}

int32_t gqa_decode(const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* seq_lens, float* out, int32_t batch, int32_t num_q_heads,
                   int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len, float scale,
                   int32_t dtype, int32_t split_tokens, void* workspace, int64_t workspace_bytes,
                   void* stream) {
  if (!out) return GQA_ERR_NULL;
  if (dtype == GQA_FP8_E4M3) return GQA_ERR_UNSUPPORTED;   // needs the scales: gqa_decode_fp8
  gqa::DecodeShape s;
  gqa::DecodeWorkspace ws;
  int32_t st = decode_prepare(q, k_cache, v_cache, seq_lens, workspace, workspace_bytes, batch,
                              num_q_heads, num_kv_heads, head_dim, max_seq_len, scale, dtype,
                              split_tokens, &s, &ws);
  if (st != GQA_OK) return st;
  if (!aligned(out, 16)) return GQA_ERR_ALIGN;
  char* base = static_cast<char*>(workspace);
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  st = hip_status(gqa::launch_decode_split(q, k_cache, v_cache, seq_lens, out, base, s, hs));
  if (st != GQA_OK) return st;
  return hip_status(gqa::launch_decode_merge(seq_lens, out, base, s, hs));
}

int32_t gqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* seq_lens, float* out, int32_t batch, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len, float scale,
                           int32_t dtype, int32_t split_tokens, void* stream) {
  if (!q || !k_cache || !v_cache || !seq_lens || !out) return GQA_ERR_NULL;
  if (dtype == GQA_FP8_E4M3) return GQA_ERR_UNSUPPORTED;   // needs the scales: gqa_decode_fp8
  gqa::DecodeShape s;
  int32_t st = make_plan(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, dtype, split_tokens, scale, &s);
  if (st != GQA_OK) return st;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(seq_lens, 4))
    return GQA_ERR_ALIGN;
  if (gqa::decode_workspace_layout(s).total > kNoAllocScratchBytes) return GQA_ERR_WORKSPACE;
  char* base = nullptr;
  st = noalloc_scratch(&base);
  if (st != GQA_OK) return st;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  st = hip_status(gqa::launch_decode_split(q, k_cache, v_cache, seq_lens, out, base, s, hs));
  if (st != GQA_OK) return st;
  return hip_status(gqa::launch_decode_merge(seq_lens, out, base, s, hs));
}

static int32_t paged_prepare(const void* q, const void* k_pages, const void* v_pages,
                             const int32_t* block_table, const int32_t* seq_lens, float* out,
                             int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t page_size, int32_t num_pages,
                             int32_t max_pages_per_seq, float scale, int32_t dtype,
                             int32_t split_tokens, void* workspace, int64_t workspace_bytes,
                             gqa::DecodeShape* s, gqa::PagedKV* pk) {
  if (!out || !block_table) return GQA_ERR_NULL;
  if (page_size < 1 || page_size > 65536 || (page_size & (page_size - 1)) != 0 || num_pages < 1 ||
      max_pages_per_seq < 1)
    return GQA_ERR_SHAPE;
  const int64_t tcap = (int64_t)max_pages_per_seq * page_size;
  if (tcap > INT32_MAX) return GQA_ERR_SHAPE;
  if (dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
  gqa::DecodeWorkspace ws;
  const int32_t st = decode_prepare(q, k_pages, v_pages, seq_lens, workspace, workspace_bytes, batch,
                                    num_q_heads, num_kv_heads, head_dim, (int32_t)tcap, scale, dtype,
                                    split_tokens, s, &ws);
  if (st != GQA_OK) return st;
  if (!aligned(out, 16) || !aligned(block_table, 4)) return GQA_ERR_ALIGN;
  int log2 = 0;
  while ((1 << log2) < page_size) ++log2;
  *pk = gqa::PagedKV{block_table, max_pages_per_seq, num_pages, log2};
  return GQA_OK;
}

int32_t gqa_decode_paged_split(const void* q, const void* k_pages, const void* v_pages,
                               const int32_t* block_table, const int32_t* seq_lens, float* out,
                               int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t page_size, int32_t num_pages,
                               int32_t max_pages_per_seq, float scale, int32_t dtype,
                               int32_t split_tokens, void* workspace, int64_t workspace_bytes,
                               void* stream) {
  gqa::DecodeShape s;
  gqa::PagedKV pk;
  const int32_t st = paged_prepare(q, k_pages, v_pages, block_table, seq_lens, out, batch, num_q_heads,
                                   num_kv_heads, head_dim, page_size, num_pages, max_pages_per_seq, scale,
                                   dtype, split_tokens, workspace, workspace_bytes, &s, &pk);
  if (st != GQA_OK) return st;
  return hip_status(gqa::launch_decode_split(q, k_pages, v_pages, seq_lens, out, static_cast<char*>(workspace),
                                             s, static_cast<hipStream_t>(stream), pk));
}

int32_t gqa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                         const int32_t* block_table, const int32_t* seq_lens, float* out,
                         int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t page_size, int32_t num_pages,
                         int32_t max_pages_per_seq, float scale, int32_t dtype,
                         int32_t split_tokens, void* workspace, int64_t workspace_bytes,
                         void* stream) {
  gqa::DecodeShape s;
  gqa::PagedKV pk;
  int32_t st = paged_prepare(q, k_pages, v_pages, block_table, seq_lens, out, batch, num_q_heads,
                             num_kv_heads, head_dim, page_size, num_pages, max_pages_per_seq, scale, dtype,
                             split_tokens, workspace, workspace_bytes, &s, &pk);
  if (st != GQA_OK) return st;
  char* base = static_cast<char*>(workspace);
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  st = hip_status(gqa::launch_decode_split(q, k_pages, v_pages, seq_lens, out, base, s, hs, pk));
  if (st != GQA_OK) return st;
  return hip_status(gqa::launch_decode_merge(seq_lens, out, base, s, hs));
}

static int32_t fp8_run(bool merge, const void* q, const void* k_cache, const void* v_cache,
                       const float* k_scale, const float* v_scale, const int32_t* seq_lens, float* out,
                       int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t max_seq_len, float scale, int32_t split_tokens, void* workspace,
                       int64_t workspace_bytes, void* stream) {
  if (!out || !k_scale || !v_scale) return GQA_ERR_NULL;
  gqa::DecodeShape s;
  gqa::DecodeWorkspace ws;
  int32_t st = decode_prepare(q, k_cache, v_cache, seq_lens, workspace, workspace_bytes, batch, num_q_heads,
                              num_kv_heads, head_dim, max_seq_len, scale, GQA_FP8_E4M3, split_tokens, &s, &ws);
  if (st != GQA_OK) return st;
  if (!aligned(out, 16) || !aligned(k_scale, 4) || !aligned(v_scale, 4)) return GQA_ERR_ALIGN;
  char* base = static_cast<char*>(workspace);
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  st = hip_status(gqa::launch_decode_split(q, k_cache, v_cache, seq_lens, out, base, s, hs,
                                           gqa::PagedKV{nullptr, 0, 0, 0}, k_scale, v_scale));
  if (st != GQA_OK || !merge) return st;
  return hip_status(gqa::launch_decode_merge(seq_lens, out, base, s, hs));
}

int32_t gqa_decode_fp8(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                       const float* v_scale, const int32_t* seq_lens, float* out, int32_t batch,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len,
                       float scale, int32_t split_tokens, void* workspace, int64_t workspace_bytes,
                       void* stream) {
  return fp8_run(true, q, k_cache, v_cache, k_scale, v_scale, seq_lens, out, batch, num_q_heads, num_kv_heads,
                 head_dim, max_seq_len, scale, split_tokens, workspace, workspace_bytes, stream);
}

int32_t gqa_decode_fp8_split(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                             const float* v_scale, const int32_t* seq_lens, float* out, int32_t batch,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t max_seq_len, float scale, int32_t split_tokens, void* workspace,
                             int64_t workspace_bytes, void* stream) {
  return fp8_run(false, q, k_cache, v_cache, k_scale, v_scale, seq_lens, out, batch, num_q_heads,
                 num_kv_heads, head_dim, max_seq_len, scale, split_tokens, workspace, workspace_bytes, stream);
}

int32_t gqa_prefill_causal(const void* q, const void* k, const void* v, float* out, float* lse,
                           int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t seq_len, int32_t head_dim, float scale, int32_t dtype,
                           void* stream) {
  if (!q || !k || !v || !out) return GQA_ERR_NULL;
  const int32_t st = check_prefill(batch, num_q_heads, num_kv_heads, seq_len, head_dim, dtype);
  if (st != GQA_OK) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      (lse && !aligned(lse, 4)))
    return GQA_ERR_ALIGN;
  gqa::PrefillShape s{batch, num_q_heads, num_kv_heads, seq_len, head_dim, scale};
  return hip_status(gqa::launch_prefill_causal(q, k, v, out, lse, s, static_cast<hipStream_t>(stream)));
}

int32_t gqa_prefill_backward_workspace(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t seq_len, int32_t head_dim, int64_t* workspace_bytes_out) {
  if (!workspace_bytes_out) return GQA_ERR_NULL;
  const int32_t st = check_prefill(batch, num_q_heads, num_kv_heads, seq_len, head_dim, GQA_BF16);
  if (st != GQA_OK) return st;
  *workspace_bytes_out = backward_workspace_bytes(batch, num_q_heads, seq_len);
  return GQA_OK;
}

int32_t gqa_prefill_causal_backward(const void* q, const void* k, const void* v, const float* out,
                                    const float* lse, const void* dout, float* dq, float* dk, float* dv,
                                    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t seq_len, int32_t head_dim, float scale, int32_t dtype,
                                    void* workspace, int64_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv || !workspace) return GQA_ERR_NULL;
  const int32_t st = check_prefill(batch, num_q_heads, num_kv_heads, seq_len, head_dim, dtype);
  if (st != GQA_OK) return st;
  if (workspace_bytes < backward_workspace_bytes(batch, num_q_heads, seq_len)) return GQA_ERR_WORKSPACE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(workspace, 16) ||
      !aligned(lse, 4))
    return GQA_ERR_ALIGN;
  gqa::PrefillShape s{batch, num_q_heads, num_kv_heads, seq_len, head_dim, scale};
  return hip_status(gqa::launch_prefill_backward(q, k, v, out, lse, dout, dq, dk, dv,
                                                 static_cast<float*>(workspace), s,
                                                 static_cast<hipStream_t>(stream)));
}

int32_t gqa_decode_wide_plan(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim_qk,
                             int32_t head_dim_v, int32_t max_seq_len, int32_t split_tokens,
                             int32_t* ranges_out, int64_t* workspace_bytes_out) {
  gqa::WideShape s;
  const int32_t st = make_wide_plan(batch, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, max_seq_len,
                                    split_tokens, 1.f, &s);
  if (st != GQA_OK) return st;
  if (ranges_out) *ranges_out = s.nranges;
  if (workspace_bytes_out) *workspace_bytes_out = gqa::wide_workspace_bytes(s);
  return GQA_OK;
}

int32_t gqa_decode_wide(const void* q, const void* kv_cache, const int32_t* seq_lens, float* out,
                        int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim_qk,
                        int32_t head_dim_v, int32_t max_seq_len, float scale, int32_t split_tokens,
                        void* workspace, int64_t workspace_bytes, void* stream) {
  if (!q || !kv_cache || !seq_lens || !out) return GQA_ERR_NULL;
  gqa::WideShape s;
  const int32_t st = make_wide_plan(batch, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, max_seq_len,
                                    split_tokens, scale, &s);
  if (st != GQA_OK) return st;
  const int64_t need = gqa::wide_workspace_bytes(s);
  if (need > 0 && !workspace) return GQA_ERR_NULL;
  if (workspace_bytes < need) return GQA_ERR_WORKSPACE;
  if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(out, 16) || !aligned(seq_lens, 4) ||
      (need > 0 && !aligned(workspace, 16)))
    return GQA_ERR_ALIGN;
  return hip_status(gqa::launch_decode_wide(q, kv_cache, seq_lens, out, static_cast<char*>(workspace), s,
                                            static_cast<hipStream_t>(stream)));
}

}  // extern "C"
