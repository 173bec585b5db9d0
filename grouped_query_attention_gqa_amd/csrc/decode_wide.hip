// Decode over wide cached rows that are both key and value: the absorbed-MLA
// shape on gfx950 bf16 matrix cores.
//
// With weight absorption, MLA decode is many query heads attending to one
// cached latent row per token, scored over the whole row (latent plus the
// shared rotary key) and averaged over the row's latent part
// (anrans.github.io, "Attention variants: MQA, GQA, MLA", section "MLA:
// multi-head latent attention": an MQA with a very large head dimension,
// 512 latent + 64 rotary = 576 cached numbers per token).  Here the row is
// d_k = 576 bf16 values, the value is its first d_v = 512, and query head h
// reads KV head h / g as everywhere in this library.
//
// At g = 128 the intensity is about 242 FLOP per cached byte, close to the
// MI355X ridge (~312), so the work sits on the matrix cores and the design
// is about registers and LDS bandwidth.  On gfx950 an MFMA whose operand
// comes from LDS runs at full rate only when two wavefronts share a SIMD
// (one wavefront does not overlap its own LDS reads with its MFMAs), so a
// wavefront must stay under 256 registers:
//  * a workgroup is 8 wavefronts serving 128 query heads of one KV head over
//    one token range; every 32-token tile of 576-column rows (36 KiB) is
//    brought into LDS once by direct global-to-LDS loads, double-buffered,
//    and read by all eight wavefronts;
//  * a wavefront owns 16 heads outright, on v_mfma_f32_16x16x32_bf16:
//    S^T[32 tok, 16 heads] = K Q^T over all 576 columns (18 steps per
//    16-token half, Q^T in 72 registers) and O^T[512, 16 heads] += V^T P^T
//    (32 column blocks, 128 accumulation registers, V^T by transposing LDS
//    reads), with no exchange between wavefronts;
//  * the weights of a range are taken against one fixed maximum, the first
//    tile's; weights up to 2^8 are harmless in bf16 and fp32, and a range
//    whose later scores exceed that (not met at ordinary score sizes) is
//    computed a second time against its true maximum, so the accumulators
//    are never rescaled;
//  * token ranges of a unit (sequence, KV head, head block) are merged by
//    their log-sum-exp, as in the narrow decode, when there is more than
//    one.
// Rows are 72 chunks of 16 bytes; in LDS the low three bits of the chunk
// index are XOR-ed with a rotation of (row / 2) mod 8, which keeps the row
// reads (16 rows, one chunk each per 16 lanes) and the transposing reads (4
// rows, 32 bytes each) free of bank conflicts although a row is not a power
// of two long.

#include "gqa_device.hpp"
#include "gqa_launch.hpp"

namespace gqa {

namespace {

constexpr int kDK = kWideDK;
constexpr int kDV = kWideDV;
constexpr int kCPR = kDK / 8;                     // 16-byte chunks per row
constexpr int kTok = 32;                          // tokens per tile
constexpr int kThreads = 512;
constexpr int kFillThreads = 256;                 // the first four wavefronts fill the tiles
constexpr int kWaveHeads = 16;                    // query heads per wavefront
constexpr int kKSteps = kDK / 32;                 // score MFMAs per 16-token half
constexpr int kVBlocks = kDV / 16;                // 16-column blocks of the value
constexpr int kTileElems = kTok * kDK;
constexpr int kLoads = kTok * kCPR / kFillThreads;   // 16-byte loads per filling thread per tile
constexpr float kLazyMax = 8.f;                   // log2 slack before a second pass
constexpr int kXcds = 8;

static_assert(kTok * kCPR % kFillThreads == 0, "tile must split evenly over the filling threads");
static_assert(kWideHeadBlock == (kThreads / 64) * kWaveHeads, "eight wavefronts of 16 heads");
static_assert(kKSteps % 2 == 0 && kVBlocks % 4 == 0, "step and block counts");

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Low-bit swizzle of row r: a rotation of (r / 2) mod 8.
__device__ __forceinline__ int wide_swz(int r) {
  const int x = (r >> 1) & 7;
  return ((x << 1) | (x >> 2)) & 7;
}

// Physical chunk of logical chunk c in row r (an involution on the low bits).
__device__ __forceinline__ int wide_phys(int r, int c) { return (c & ~7) | ((c ^ wide_swz(r)) & 7); }

__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

struct WideArgs {
  const __bf16* q;
  const __bf16* kv;
  const int32_t* lens;
  float* out;
  float* part_o;
  float* part_lse;
  int hq, hkv, g, nhb, tcap, split, nranges, units;
  float scale_log2;
};

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void decode_wide_bf16(WideArgs a) {
  __shared__ __align__(16) __bf16 t0s[kTileElems];
  __shared__ __align__(16) __bf16 t1s[kTileElems];

  // Workgroup -> (space index s = (b, kvh, range), head block hb); the nhb
  // head blocks of one s are 8 workgroups apart, i.e. on the same XCD.
  const int wg = blockIdx.x;
  const int hb = (wg / kXcds) % a.nhb;
  const int sidx = (wg / kXcds / a.nhb) * kXcds + wg % kXcds;
  const int total = a.units / a.nhb * a.nranges;
  if (sidx >= total) return;
  const int r = sidx % a.nranges;
  const int bk = sidx / a.nranges;
  const int b = bk / a.hkv;
  const int kvh = bk - b * a.hkv;
  const int unit = bk * a.nhb + hb;
  int len = a.lens[b];
  len = len < 0 ? 0 : (len > a.tcap ? a.tcap : len);
  const int t_begin = r * a.split;
  const int t_end = min(len, t_begin + a.split);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15;   // this lane's head (B / D column) and A row
  const int kg = lane >> 4;    // contraction group
  const int hl = hb * kWideHeadBlock + kWaveHeads * w + c16;   // head within the group
  const bool head_ok = hl < a.g;
  const int head = kvh * a.g + min(hl, a.g - 1);
  const size_t slot = ((size_t)r * a.units + unit) * kWideHeadBlock + kWaveHeads * w + c16;

  if (t_begin >= t_end) {   // nothing to attend in this range (uniform over the workgroup)
    if (a.nranges > 1) {
      if (kg == 0) a.part_lse[slot] = -INFINITY;
    } else if (head_ok) {
      float* o = a.out + ((size_t)b * a.hq + head) * kDV;
      for (int i = 4 * kg; i < kDV; i += 16) *reinterpret_cast<f32x4*>(o + i) = f32x4{};
    }
    return;
  }

  // Q^T as B operands: head c16, columns 32 kk + 8 kg .. +7.
  bf16x8 qb[kKSteps];
  {
    const __bf16* qrow = a.q + ((size_t)b * a.hq + head) * kDK;
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk) qb[kk] = load_bf16x8(qrow + 32 * kk + 8 * kg);
  }

  // LDS offsets.  K rows: token 16 tb + c16, chunk 4 kk + kg; the swizzle
  // depends neither on tb nor on kk beyond its parity, so two bases plus
  // 64-element steps (per two kk) and 16-row steps (per tb) cover all.  V^T:
  // rows 4 kg + 0..3 and 16 + 4 kg + 0..3, columns 16 db + ...; the swizzle
  // is the same for both row groups and repeats every four db.  The empty
  // asm hides the bases' value range so that constants fold into the
  // instructions' offset fields.
  int k_base[2], v_base[4];
  {
    const int swk = wide_swz(c16);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      k_base[p] = c16 * kDK + ((4 * p + kg) ^ swk) * 8;
      asm volatile("" : "+v"(k_base[p]));
    }
    const int L = c16;
    const int row = 4 * kg + (L >> 2);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int colv = 16 * p + 4 * (L & 3);
      v_base[p] = row * kDK + wide_phys(row, colv >> 3) * 8 + (colv & 7);
      asm volatile("" : "+v"(v_base[p]));
    }
  }
  auto k_op = [&](const __bf16* ts, int tb, int kk) {
    return load_bf16x8(ts + k_base[kk & 1] + 64 * (kk >> 1) + tb * 16 * kDK);
  };
  auto v_op = [&](const __bf16* ts, int db) {
    const int rd = v_base[db & 3] + 64 * (db >> 2);
    return concat(lds_read_tr16(ts + rd), lds_read_tr16(ts + rd + 16 * kDK));
  };

  // Tile fill: thread tid < 256 deposits physical chunks tid + 256 i (the
  // source offsets are recomputed per tile rather than held in registers).
  const __bf16* kvb = a.kv + ((size_t)b * a.hkv + kvh) * (size_t)a.tcap * kDK;
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(kvb, t_end * kDK * 2);   // rows >= t_end read as 0
  auto fill = [&](__bf16* dst, int t0) {
    if (w < kFillThreads / 64) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int p = tid + kFillThreads * i;
        const int row = p / kCPR;
        const int src = row * kDK * 2 + wide_phys(row, p - row * kCPR) * 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(dst + (w * 64 + kFillThreads * i) * 8), 16,
                                                 t0 * kDK * 2 + src, 0, 0, kCacheStream);
      }
    }
  };

  f32x4 acc[kVBlocks];
  float m_fix = -INFINITY;    // the maximum (log2 units) the weights are taken against
  float m_seen = -INFINITY;   // the largest tile maximum met so far
  float l_run = 0.f;          // this lane's share of the sum of weights

  // One tile.  Operands are read in groups of four, one group ahead of the
  // MFMAs that use them.
  auto tile = [&](const __bf16* ts, int t0) {
    // S^T for the two 16-token halves.  With two wavefronts per SIMD the
    // other wavefront covers each operand read, so the reads are not
    // prefetched into extra registers.
    f32x4 s0 = f32x4{}, s1 = f32x4{};
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk) {
      s0 = mfma16(k_op(ts, 0, kk), qb[kk], s0);
      s1 = mfma16(k_op(ts, 1, kk), qb[kk], s1);
      if (kk % 2 == 1) __builtin_amdgcn_sched_barrier(0);   // bounds how far reads are hoisted
    }
    // element e: token t0 + 16 (e / 4) + 4 kg + e % 4 of head c16
    float s[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[e] = s0[e] * a.scale_log2;
      s[4 + e] = s1[e] * a.scale_log2;
    }
    if (t0 + kTok > t_end) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = t0 + 16 * (e >> 2) + 4 * kg + (e & 3);
        s[e] = t < t_end ? s[e] : -INFINITY;
      }
    }
    float mx = max3f(max3f(s[0], s[1], s[2]), max3f(s[3], s[4], s[5]), fmaxf(s[6], s[7]));
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    m_seen = fmaxf(m_seen, mx);
    m_fix = m_fix == -INFINITY ? mx : m_fix;   // the first tile fixes it (every tile has a token)
    bf16x8 pb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = fast_exp2(s[e] - m_fix);
      l_run += p;
      pb[e] = (__bf16)p;
    }
    // O^T[512, 16 heads] += V^T[512, 32 tok] P^T[32 tok, 16 heads], 16 columns per MFMA.
#pragma unroll
    for (int db = 0; db < kVBlocks; ++db) {
      acc[db] = mfma16(v_op(ts, db), pb, acc[db]);
      if (db % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The accumulators are never rescaled inside the loop.  The first pass
  // takes the weights against the first tile's maximum; if a later tile's
  // maximum exceeded it by more than kLazyMax (weights above 2^8, which
  // scores of ordinary size never reach) the range is computed again against
  // the largest maximum, which bounds every weight by 1.
  const int ntiles = (t_end - t_begin + kTok - 1) / kTok;
  auto run = [&]() {
#pragma unroll
    for (int i = 0; i < kVBlocks; ++i) acc[i] = f32x4{};
    l_run = 0.f;
    fill(t0s, t_begin);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
      const bool odd = it & 1;
      if (it + 1 < ntiles) fill(odd ? t0s : t1s, t_begin + (it + 1) * kTok);
      tile(odd ? t1s : t0s, t_begin + it * kTok);
      __builtin_amdgcn_s_waitcnt(0);   // this thread's loads of the next tile have landed
      __syncthreads();                 // ... everyone's, and the current stage is free again
    }
  };
  run();
  // Workgroup-wide decision, so every wavefront takes part in the same
  // barriers; the second pass is a separate copy of the loop.
  if (__syncthreads_or(m_seen > m_fix + kLazyMax)) {
    m_fix = m_seen;
    run();
  }

  float l_tot = l_run + shfl_xor(l_run, 16);
  l_tot += shfl_xor(l_tot, 32);
  if (!head_ok) return;
  const float inv = 1.f / l_tot;
  // O^T block db: column 16 db + 4 kg + e of head c16
  float* o = a.nranges > 1 ? a.part_o + slot * kDV : a.out + ((size_t)b * a.hq + head) * kDV;
#pragma unroll
  for (int db = 0; db < kVBlocks; ++db) *reinterpret_cast<f32x4*>(o + 16 * db + 4 * kg) = acc[db] * inv;
  if (a.nranges > 1 && kg == 0) a.part_lse[slot] = m_fix + __log2f(l_tot);
}

// out[b, h] = sum over ranges 2^(lse_r - M) O_r / sum 2^(lse_r - M); empty
// ranges carry lse = -inf, and a sequence with no tokens gets zeros.
constexpr int kWideMergeThreads = kDV / 4;

__global__ __launch_bounds__(kWideMergeThreads)
void decode_wide_merge(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                       float* __restrict__ out, int hq, int hkv, int g, int nhb, int nranges, int units) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int kvh = h / g;
  const int hl = h - kvh * g;
  const int hb = hl / kWideHeadBlock;
  const int unit = (b * hkv + kvh) * nhb + hb;
  const int lane_slot = hl - hb * kWideHeadBlock;
  const int c4 = threadIdx.x;
  float mx = -INFINITY;
  for (int r = 0; r < nranges; ++r)
    mx = fmaxf(mx, part_lse[((size_t)r * units + unit) * kWideHeadBlock + lane_slot]);
  f32x4 acc = f32x4{};
  if (mx != -INFINITY) {
    float den = 0.f;
    for (int r = 0; r < nranges; ++r) {
      const size_t slot = ((size_t)r * units + unit) * kWideHeadBlock + lane_slot;
      const float lr = part_lse[slot];
      if (lr == -INFINITY) continue;
      const float wgt = fast_exp2(lr - mx);
      den += wgt;
      acc += wgt * *reinterpret_cast<const f32x4*>(part_o + slot * kDV + 4 * c4);
    }
    acc *= 1.f / den;
  }
  *reinterpret_cast<f32x4*>(out + ((size_t)b * hq + h) * kDV + 4 * c4) = acc;
}

}  // namespace

hipError_t launch_decode_wide(const void* q, const void* kv, const int32_t* lens, float* out,
                              char* workspace, const WideShape& s, hipStream_t stream) {
  WideArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.kv = static_cast<const __bf16*>(kv);
  a.lens = lens;
  a.out = out;
  const int64_t slots = (int64_t)s.nranges * s.units * kWideHeadBlock;
  a.part_lse = s.nranges > 1 ? reinterpret_cast<float*>(workspace) : nullptr;
  a.part_o = s.nranges > 1 ? reinterpret_cast<float*>(workspace + wide_lse_bytes(slots)) : nullptr;
  a.hq = s.hq;
  a.hkv = s.hkv;
  a.g = s.hq / s.hkv;
  a.nhb = s.nhb;
  a.tcap = s.tcap;
  a.split = s.split;
  a.nranges = s.nranges;
  a.units = s.units;
  a.scale_log2 = s.scale * kLog2e;
  hipLaunchKernelGGL(decode_wide_bf16, dim3((unsigned)s.grid), dim3(kThreads), 0, stream, a);
  if (s.nranges > 1)
    hipLaunchKernelGGL(decode_wide_merge, dim3((unsigned)s.hq, (unsigned)s.batch), dim3(kWideMergeThreads), 0,
                       stream, a.part_o, a.part_lse, out, s.hq, s.hkv, a.g, s.nhb, s.nranges, s.units);
  return hipGetLastError();
}

}  // namespace gqa
