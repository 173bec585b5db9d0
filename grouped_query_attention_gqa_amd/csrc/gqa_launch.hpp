// Host-side launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

// Query heads of one MFMA column block in decode.  A decode unit covers one
// block, or, for bf16 and E4M3 caches when the group is larger than 16, two
// blocks (32 heads) at head_dim 128 and up to kMaxHeadBlocks64 blocks (80
// heads) at head_dim 64, whose accumulators take half the registers; so
// groups of up to 32 (head_dim 128) or 80 (head_dim 64) query heads share a
// single pass over their KV head.
constexpr int kDecodeHeadBlock = 16;
constexpr int kMaxHeadBlocks64 = 5;
// Decode: tokens per wavefront iteration (bf16 path) and waves per workgroup.
constexpr int kDecodeWaveTile = 32;
constexpr int kDecodeWaves = 4;
// Caller-fixed range sizes are positive multiples of this many tokens.
constexpr int kRangeQuantum = 32;
// Smallest automatic range: below this, per-range overhead dominates.
constexpr int kMinRange = 256;
// Persistent decode workgroups: 256 CUs x 2 resident 4-wave workgroups.
#ifndef GQA_DECODE_GRID
#define GQA_DECODE_GRID 512
#endif
constexpr int kPersistentWorkgroups = GQA_DECODE_GRID;

struct DecodeShape {
  int batch, hq, hkv, d, tcap;
  int hb;            // 16-head blocks per unit: 1 for fp32 caches or g <= 16, else 2 at d = 128
                     // and min(ceil(g / 16), kMaxHeadBlocks64) at d = 64
  int nhg;           // units per KV head: ceil(ceil(g / 16) / hb)
  int units;         // batch * hkv * nhg
  int q_fixed;       // tokens per range fixed by the caller, 0 = chosen on the device
  int grid;          // workgroups launched
  int64_t max_slots; // upper bound on partial slots (ranges + units)
  float scale;
  int dtype;         // gqa_dtype (GQA_FP8_E4M3: bf16 q with an E4M3 cache)
};

// Byte offsets of the workspace arrays: per-unit (first slot, segment
// count), then per-slot log2-sum-exp [slots][16 hb], then per-slot
// normalised outputs [slots][16 hb][d], each 256-byte aligned.
struct DecodeWorkspace {
  int64_t info_offset, lse_offset, o_offset, total;
};

DecodeWorkspace decode_workspace_layout(const DecodeShape& s);

// K/V held in a pool of pages [num_pages, Hkv, page_size, d]; table[b, i]
// names the page of tokens i*page_size .. (i+1)*page_size-1 of sequence b.
// A null table means the contiguous cache [batch, Hkv, tcap, d].
struct PagedKV {
  const int32_t* table;
  int max_pages, num_pages, page_log2;
};

hipError_t launch_decode_split(const void* q, const void* k, const void* v, const int32_t* lens,
                               float* out, char* workspace, const DecodeShape& s,
                               hipStream_t stream, const PagedKV& paged = PagedKV{nullptr, 0, 0, 0},
                               const float* k_scale = nullptr, const float* v_scale = nullptr);

hipError_t launch_decode_merge(const int32_t* lens, float* out, const char* workspace,
                               const DecodeShape& s, hipStream_t stream);

// Wide-row decode (absorbed-MLA shape): cached rows of kWideDK columns whose
// first kWideDV columns are the value; a workgroup serves kWideHeadBlock
// query heads of one KV head over one token range.
constexpr int kWideDK = 576;
constexpr int kWideDV = 512;
constexpr int kWideHeadBlock = 64;

struct WideShape {
  int batch, hq, hkv, tcap;
  int nhb;       // head blocks per KV head, ceil(g / kWideHeadBlock)
  int units;     // batch * hkv * nhb
  int split;     // tokens per range (a multiple of 32)
  int nranges;   // ceil(tcap / split); 1 means no workspace and no merge
  int grid;      // workgroups launched (the head blocks of a range share an XCD)
  float scale;
};

// Workspace: partial log2-sum-exp [nranges][units][kWideHeadBlock], then
// normalised partial outputs [nranges][units][kWideHeadBlock][kWideDV].
inline int64_t wide_lse_bytes(int64_t slots) { return (slots * 4 + 255) / 256 * 256; }
inline int64_t wide_workspace_bytes(const WideShape& s) {
  if (s.nranges <= 1) return 0;
  const int64_t slots = (int64_t)s.nranges * s.units * kWideHeadBlock;
  return wide_lse_bytes(slots) + slots * kWideDV * 4;
}

hipError_t launch_decode_wide(const void* q, const void* kv, const int32_t* lens, float* out,
                              char* workspace, const WideShape& s, hipStream_t stream);

struct PrefillShape {
  int batch, hq, hkv, n, d;
  float scale;
};

hipError_t launch_prefill_causal(const void* q, const void* k, const void* v, float* out,
                                 float* lse, const PrefillShape& s, hipStream_t stream);

// Backward of causal prefill: dq, then (after it, on the same stream) dk and
// dv; `row_terms` [2][batch, hq, n] receives lse * log2(e) and
// rowsum(dout * out) from the first kernel and is read by the second.
hipError_t launch_prefill_backward(const void* q, const void* k, const void* v, const float* out,
                                   const float* lse, const void* dout, float* dq, float* dk, float* dv,
                                   float* row_terms, const PrefillShape& s, hipStream_t stream);

}  // namespace gqa
