// Host-side launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

// Query heads handled by one decode workgroup: the MFMA column block.  Groups
// of up to 16 query heads share a single pass over their KV head.
constexpr int kDecodeHeadBlock = 16;
// Decode: tokens per wavefront iteration (bf16 path) and waves per workgroup.
constexpr int kDecodeWaveTile = 32;
constexpr int kDecodeWaves = 4;
// Split sizes are multiples of this many tokens.
constexpr int kSplitQuantum = 64;

struct DecodeShape {
  int batch, hq, hkv, d, tcap;
  int chunk;   // tokens per split
  int nsplit;  // split slots per sequence = ceil(tcap / chunk)
  float scale;
  int dtype;   // gqa_dtype
};

// Byte offsets of the two workspace arrays.
struct DecodeWorkspace {
  int64_t o_offset, lse_offset, total;
};

DecodeWorkspace decode_workspace_layout(const DecodeShape& s);

hipError_t launch_decode_split(const void* q, const void* k, const void* v, const int32_t* lens,
                               float* part_o, float* part_lse, const DecodeShape& s,
                               hipStream_t stream);

hipError_t launch_decode_merge(const float* part_o, const float* part_lse, const int32_t* lens,
                               float* out, const DecodeShape& s, hipStream_t stream);

struct PrefillShape {
  int batch, hq, hkv, n, d;
  float scale;
};

hipError_t launch_prefill_causal(const void* q, const void* k, const void* v, float* out,
                                 float* lse, const PrefillShape& s, hipStream_t stream);

}  // namespace gqa
