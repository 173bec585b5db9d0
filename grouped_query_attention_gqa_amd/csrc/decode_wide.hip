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
// MI355X ridge (~312): per tile the matrix-core time and the HBM time are
// about equal, so the design is about keeping operand traffic through LDS
// and the phases of a tile overlapped.  A workgroup is 8 wavefronts (two
// per SIMD) serving a block of 64 query heads of one KV head over one token
// range; the two blocks of a 128-head group run on the same XCD and share
// the rows through L2.  32-token tiles of 576-column rows (36 KiB) go into a
// ring of three LDS stages by direct global-to-LDS loads issued two tiles
// ahead.  The wavefronts split into two roles that share each SIMD:
//  * score wavefronts 0-3 take contraction columns 144 w .. +143 of S^T[32
//    tok, 64 heads] (v_mfma_f32_32x32x16_bf16, Q^T in 72 registers, every K
//    operand feeding both 32-head blocks), publish the partial scores to
//    LDS, and issue the tile loads;
//  * value wavefronts 4-7 own output columns 128 (w - 4) .. +127 for all 64
//    heads, O^T[128, 64] += V^T[128, 32 tok] P^T[32 tok, 64] (16 MFMAs per
//    tile, 128 accumulation registers, no value column read twice), and sum
//    the four partial scores of their 16 heads and weight them (bf16
//    P[head][token] in LDS).
// In step it the score wavefronts work on tile it while the value
// wavefronts accumulate tile it - 1, so the two kinds of MFMA work overlap
// on every SIMD; two barriers per step.
// The weights of a range are taken against one fixed maximum per head, the
// first tile's, so the accumulators never need a rescale; weights up to 2^8
// are harmless in bf16 and fp32, and a range whose later scores exceed that
// (not met at ordinary score sizes) is computed a second time against its
// true maximum.  Token ranges of a unit (sequence, KV head, head block) are
// merged by their log-sum-exp, as in the narrow decode, when there is more
// than one.
// Rows are 72 chunks of 16 bytes; in LDS the low three bits of the chunk
// index are XOR-ed with a rotation of (row / 2) mod 8, which keeps the K
// operand reads (16 rows, one chunk each per 16 lanes) and the transposing
// value reads (4 rows, 4 chunks each per 32 lanes) free of bank conflicts
// although a row is not a power of two long.

#include "gqa_device.hpp"
#include "gqa_launch.hpp"

namespace gqa {

namespace {

constexpr int kDK = kWideDK;
constexpr int kDV = kWideDV;
constexpr int kCPR = kDK / 8;                     // 16-byte chunks per row
constexpr int kTok = 32;                          // tokens per tile
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kScoreWaves = 4;                    // wavefronts 0-3 score, 4-7 accumulate values
constexpr int kQDims = kDK / kScoreWaves;         // 144 contraction columns per score wavefront
constexpr int kKSteps = kQDims / 16;              // 9 MFMA steps per quarter
constexpr int kNB = kWideHeadBlock / 32;          // 32-head blocks
constexpr int kPvCols = kDV / (kWaves - kScoreWaves);   // 128 value columns per value wavefront
constexpr int kCB = kPvCols / 32;                 // 32-column blocks per value wavefront
constexpr int kRedHeads = kWideHeadBlock / (kWaves - kScoreWaves);   // heads per value wavefront in the reduction
constexpr int kChunks = kTok * kCPR;              // 16-byte chunks per tile
constexpr int kFillThreads = kScoreWaves * 64;    // the score wavefronts load the tiles
constexpr int kLoads = kChunks / kFillThreads;    // 16-byte loads per filling thread per tile
constexpr int kStages = 3;                        // tile ring: loads run two tiles ahead
// s_waitcnt immediate (gfx9 encoding) for vmcnt <= kLoads with the LDS and
// export counters left alone: after two tiles' loads have been issued, this
// waits for the older tile's.
constexpr int kWaitNewest = (kLoads & 0xF) | ((kLoads >> 4) << 14) | (0x7 << 4) | (0xF << 8);
constexpr int kXElems = kWideHeadBlock * kTok;    // one quarter's partial scores
constexpr int kPRow = kTok + 8;                   // bf16 per row of P (80 bytes: 5 chunks)
constexpr float kLazyMax = 8.f;                   // log2 slack before a second pass
constexpr int kXcds = 8;

static_assert(kWideHeadBlock == 64 && kNB == 2 && kCB == 4 && kRedHeads == 16, "64-head blocks");
static_assert(kQDims % 16 == 0, "whole MFMA steps per quarter");
static_assert(kChunks % kFillThreads == 0, "tile must split evenly over the filling threads");

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Low-bit swizzle of row r: (r / 2) mod 8 rotated right by one bit, so rows
// 4m .. 4m+3 take swizzles that differ in bit 2 between their two pairs.
__device__ __forceinline__ int wide_swz(int r) {
  const int x = (r >> 1) & 7;
  return ((x & 1) << 2) | (x >> 1);
}

// Physical chunk of logical chunk c in row r (an involution on the low bits).
__device__ __forceinline__ int wide_phys(int r, int c) { return (c & ~7) | ((c ^ wide_swz(r)) & 7); }

__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Lane exchanges inside quads on the DPP path (no LDS traffic): swap with
// lane ^ 1, then with lane ^ 2.
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2, 3, 0, 1]
__device__ __forceinline__ float max4(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  return fmaxf(x, dpp<kDppXor2>(x));
}
__device__ __forceinline__ float sum4(float x) {
  x += dpp<kDppXor1>(x);
  return x + dpp<kDppXor2>(x);
}

// Barrier over LDS traffic only: waits for this wavefront's LDS accesses,
// not for its global-to-LDS tile loads still in flight (a release fence on
// LDS would wait for those too, since they write LDS).  The memory clobber
// keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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
  // three tile stages as separate arrays, so that the compiler can tell a
  // read of one stage from the loads in flight into another
  __shared__ __align__(16) __bf16 t0s[kChunks * 8];
  __shared__ __align__(16) __bf16 t1s[kChunks * 8];
  __shared__ __align__(16) __bf16 t2s[kChunks * 8];
  __shared__ __align__(16) float xs[kScoreWaves * kXElems];    // partial scores [quarter][head][token]
  __shared__ __align__(16) __bf16 ps[kWideHeadBlock * kPRow];   // weights [head][token]
  __shared__ float lsum_s[kWideHeadBlock];

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
  const int hbase = hb * kWideHeadBlock;   // first head (within the group) of the block
  const size_t slot0 = ((size_t)r * a.units + unit) * kWideHeadBlock;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool scorer = w < kScoreWaves;
  const int l32 = lane & 31;
  const int j = lane >> 5;     // contraction group of the 32x32 operands

  if (t_begin >= t_end) {   // nothing to attend in this range (uniform over the workgroup)
    if (a.nranges > 1) {
      if (tid < kWideHeadBlock) a.part_lse[slot0 + tid] = -INFINITY;
    } else {
      for (int i = tid; i < kWideHeadBlock * (kDV / 4); i += kThreads) {
        const int hl = hbase + i / (kDV / 4);
        if (hl < a.g)
          *reinterpret_cast<f32x4*>(a.out + ((size_t)b * a.hq + kvh * a.g + hl) * kDV + 4 * (i % (kDV / 4))) =
              f32x4{};
      }
    }
    return;
  }

  // Score role (wavefront w < 4): contraction columns 144 w .. +143 for all
  // 64 heads.  Q^T B operand (hb2, kk): head 32 hb2 + l32, columns
  // 144 w + 16 kk + 8 j .. +7.  The two roles run separate loops (with the
  // same barriers), so Q^T (72 registers) and the value accumulators (128)
  // share the register file.
  bf16x8 qb[kNB][kKSteps];
  f32x16 acc[kCB][kNB];
  auto load_q = [&]() {
#pragma unroll
    for (int hb2 = 0; hb2 < kNB; ++hb2) {
      const int hl = hbase + 32 * hb2 + l32;
      const int head = kvh * a.g + min(hl, a.g - 1);
      const __bf16* qrow = a.q + ((size_t)b * a.hq + head) * kDK + kQDims * w + 8 * j;
#pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) qb[hb2][kk] = load_bf16x8(qrow + 16 * kk);
    }
  };
  // K operand of step kk: token l32, logical chunk 18 w + 2 kk + j.  Four
  // steps later the chunk is 8 further with the same low bits, so four
  // bases plus 64-element steps cover all nine.  The empty asm hides the
  // bases' value range so that constants fold into the offset fields.
  int k_base[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    k_base[p] = l32 * kDK + wide_phys(l32, 2 * (kKSteps * (w & 3) + p) + j) * 8;
    asm volatile("" : "+v"(k_base[p]));
  }
  float* const xw = xs + (w & 3) * kXElems;

  // Value role (wavefront w >= 4): columns 128 (w - 4) .. +127.  V^T operand
  // (cb, kc): lane l reads column 128 (w - 4) + 32 cb + 16 ((l / 16) % 2) +
  // ..., rows 16 kc + 8 j + 4 q + (l % 16) / 4 for q = 0, 1 (transposing
  // reads); the swizzle repeats every 16 rows, so kc is a constant offset.
  int v_base[kCB][2];
  {
    const int L = lane & 15;
    const int ch = (lane >> 4) & 1;
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int row = 8 * j + 4 * q + (L >> 2);
        const int col = kPvCols * (w & 3) + 32 * cb + 16 * ch + 4 * (L & 3);
        v_base[cb][q] = row * kDK + wide_phys(row, col >> 3) * 8 + (col & 7);
        asm volatile("" : "+v"(v_base[cb][q]));
      }
  }
  auto v_op = [&](const __bf16* ts, int cb, int kc) {
    return concat(lds_read_tr16(ts + v_base[cb][0] + 16 * kc * kDK),
                  lds_read_tr16(ts + v_base[cb][1] + 16 * kc * kDK));
  };
  // P^T operand (nb, kc): head 32 nb + l32, tokens 16 kc + 8 j .. +7.
  const int p_rd = l32 * kPRow + 8 * j;

  // Reduction role (value wavefronts): head hr = 16 (w - 4) + lane / 4,
  // tokens 8 tq .. 8 tq + 7; partial scores sit in 16-byte units XOR-ed by
  // (head / 2) mod 8.
  const int hr = kRedHeads * (w & 3) + (lane >> 2);
  const int tq = lane & 3;
  const int xr0 = hr * kTok + ((2 * tq) ^ ((hr >> 1) & 7)) * 4;
  const int xr1 = hr * kTok + ((2 * tq + 1) ^ ((hr >> 1) & 7)) * 4;

  // Tile fill (score wavefronts): thread tid deposits physical chunks
  // tid + 256 i of a tile; source offsets are computed once.  Rows past the
  // range read as zeros without a memory access.
  const __bf16* kvb = a.kv + ((size_t)b * a.hkv + kvh) * (size_t)a.tcap * kDK;
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(kvb, t_end * kDK * 2);
  int fsrc[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int p = (tid & (kFillThreads - 1)) + kFillThreads * i;
    const int row = p / kCPR;
    fsrc[i] = row * kDK * 2 + wide_phys(row, p - row * kCPR) * 16;
  }
  auto fill = [&](__bf16* dst, int t0) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(dst + ((w & 3) * 64 + kFillThreads * i) * 8), 16,
                                               t0 * kDK * 2 + fsrc[i], 0, 0, kCacheDefault);
  };

  float m_fix = -INFINITY;    // head hr: the maximum (log2 units) the weights are taken against
  float m_seen = -INFINITY;   // head hr: the largest tile maximum met so far
  float l_run = 0.f;          // head hr: this lane's share of the sum of weights

  // S^T[32 tok, 64 heads] over this wavefront's quarter of the columns,
  // published to xs.
  auto score = [&](const __bf16* ts) {
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk) {
      const bf16x8 kop = load_bf16x8(ts + k_base[kk & 3] + 64 * (kk >> 2));
      s0 = mfma32(kop, qb[0][kk], s0);
      s1 = mfma32(kop, qb[1][kk], s1);
    }
    // element rr of block hb2: token 8 (rr / 4) + 4 j + rr % 4 of head 32 hb2 + l32
    auto publish = [&](f32x16 sc, int hb2) {
      const int hw = 32 * hb2 + l32;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<f32x4*>(xw + hw * kTok + (((2 * r4 + j) ^ ((hw >> 1) & 7)) * 4)) =
            f32x4{sc[4 * r4], sc[4 * r4 + 1], sc[4 * r4 + 2], sc[4 * r4 + 3]};
    };
    publish(s0, 0);
    publish(s1, 1);
  };
  // O^T[128 cols, 64 heads] += V^T[128 cols, 32 tok] P^T[32 tok, 64 heads].
  auto values = [&](const __bf16* ts) {
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      bf16x8 va[kCB], pb[kNB];
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) va[cb] = v_op(ts, cb, kc);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) pb[nb] = load_bf16x8(ps + p_rd + 32 * nb * kPRow + 16 * kc);
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) acc[cb][nb] = mfma32(va[cb], pb[nb], acc[cb][nb]);
    }
  };
  // Sum the four quarters of head hr, tokens 8 tq .. +7, weight them and
  // publish the weights to ps.
  auto reduce = [&](int t0) {
    f32x4 a0 = *reinterpret_cast<const f32x4*>(xs + xr0);
    f32x4 a1 = *reinterpret_cast<const f32x4*>(xs + xr1);
#pragma unroll
    for (int d = 1; d < kScoreWaves; ++d) {
      a0 += *reinterpret_cast<const f32x4*>(xs + d * kXElems + xr0);
      a1 += *reinterpret_cast<const f32x4*>(xs + d * kXElems + xr1);
    }
    float s[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[e] = a0[e] * a.scale_log2;
      s[4 + e] = a1[e] * a.scale_log2;
    }
    if (t0 + kTok > t_end) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] = t0 + 8 * tq + e < t_end ? s[e] : -INFINITY;
    }
    const float mx = max4(max3f(max3f(s[0], s[1], s[2]), max3f(s[3], s[4], s[5]), fmaxf(s[6], s[7])));
    m_seen = fmaxf(m_seen, mx);
    m_fix = m_fix == -INFINITY ? mx : m_fix;   // the first tile fixes it (every tile has a token)
    bf16x8 pw;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = fast_exp2(s[e] - m_fix);
      l_run += p;
      pw[e] = (__bf16)p;
    }
    store_bf16x8(ps + hr * kPRow + 8 * tq, pw);
  };

  // Step it: the score wavefronts work on tile it (in `cur`) while the value
  // wavefronts finish tile it - 1 (in `prev`, with its weights still in ps);
  // after a barrier the score wavefronts issue the loads of tile it + 2 into
  // `prev` while the value wavefronts weight tile it.  Both roles execute
  // the same barriers.
  const int ntiles = (t_end - t_begin + kTok - 1) / kTok;
  auto finish_scores = [&](__bf16* prev, int it) {
    lds_barrier();   // partial scores published; `prev` and ps are free
    fill(prev, min(t_begin + (it + 2) * kTok, t_end));   // past the range: zeros
    __builtin_amdgcn_s_waitcnt(kWaitNewest);   // this thread's loads of tile it + 1 have landed
    lds_barrier();                             // ... everyone's; the weights are published
  };
  auto finish_values = [&](int it) {
    lds_barrier();
    reduce(t_begin + it * kTok);
    lds_barrier();
  };
  auto run_scores = [&]() {
    load_q();
    fill(t0s, t_begin);
    fill(t1s, t_begin + kTok);
    __builtin_amdgcn_s_waitcnt(kWaitNewest);
    lds_barrier();
    for (int it = 0; it < ntiles; it += kStages) {
      score(t0s);
      finish_scores(t2s, it);
      if (it + 1 >= ntiles) break;
      score(t1s);
      finish_scores(t0s, it + 1);
      if (it + 2 >= ntiles) break;
      score(t2s);
      finish_scores(t1s, it + 2);
    }
    __builtin_amdgcn_s_waitcnt(0);   // no load into a stage outlives the pass
  };
  auto run_values = [&]() {
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) acc[cb][nb] = f32x16{};
    l_run = 0.f;
    lds_barrier();        // the first tile has landed
    finish_values(0);   // step 0: no earlier tile to accumulate
    // step it accumulates tile it - 1; after the last tile only that remains
    for (int it = 1;; it += kStages) {
      values(t0s);
      if (it >= ntiles) break;
      finish_values(it);
      values(t1s);
      if (it + 1 >= ntiles) break;
      finish_values(it + 1);
      values(t2s);
      if (it + 2 >= ntiles) break;
      finish_values(it + 2);
    }
  };

  // The accumulators are never rescaled inside the loop.  The first pass
  // takes the weights against the first tile's maximum; if a later tile's
  // maximum exceeded it by more than kLazyMax (weights above 2^8, which
  // scores of ordinary size never reach) the range is computed again against
  // the largest maximum, which bounds every weight by 1.  The decision is
  // workgroup-wide, so both roles take part in the same barriers; each role
  // keeps to its own code path until the end, so that its registers are
  // never live in the other's loop.
  auto second_pass = [&]() {
    const bool redo = __syncthreads_or(m_seen > m_fix + kLazyMax);
    if (redo) m_fix = m_seen;
    return redo;
  };
  // Denominators of the block's heads, and the range's log-sum-exp.
  auto publish_sums = [&]() {
    if (!scorer) {
      const float l_tot = sum4(l_run);
      if (tq == 0) {
        lsum_s[hr] = l_tot;
        if (a.nranges > 1) a.part_lse[slot0 + hr] = m_fix + __log2f(l_tot);
      }
    }
    __syncthreads();
  };
  if (scorer) {
    run_scores();
    if (second_pass()) run_scores();
    publish_sums();
    return;
  }
  run_values();
  if (second_pass()) run_values();
  publish_sums();
  // O^T block (cb, nb): column 128 (w - 4) + 32 cb + 8 (rr / 4) + 4 j + rr % 4 of head 32 nb + l32
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const int hl = hbase + 32 * nb + l32;
    if (hl >= a.g) continue;
    const float inv = 1.f / lsum_s[32 * nb + l32];
    float* o = a.nranges > 1 ? a.part_o + (slot0 + 32 * nb + l32) * kDV
                             : a.out + ((size_t)b * a.hq + kvh * a.g + hl) * kDV;
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<f32x4*>(o + kPvCols * (w & 3) + 32 * cb + 8 * r4 + 4 * j) =
            f32x4{acc[cb][nb][4 * r4], acc[cb][nb][4 * r4 + 1], acc[cb][nb][4 * r4 + 2],
                  acc[cb][nb][4 * r4 + 3]} * inv;
  }
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
