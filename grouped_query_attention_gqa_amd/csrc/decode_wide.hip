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
// range; the head blocks of a 128-head group run on the same XCD and share
// the rows through L2.  32-token tiles of 576-column rows (36 KiB) go into a
// ring of four LDS stages by direct global-to-LDS loads, issued two tiles
// ahead by the value wavefronts at raised wavefront priority.  The
// wavefronts split into two roles that share each SIMD, each in its own
// code path so their registers never overlap:
//  * score wavefronts 0-3 own 16 heads each over all 576 columns: S^T[16
//    tok, 16 heads] per half tile on v_mfma_f32_16x16x32_bf16 (Q^T as B
//    operands in 72 registers, K operands read from LDS in groups of six,
//    one group ahead of their MFMAs), then the weights of the tile's 32
//    tokens, published as bf16 P[head][token] into one of two weight
//    buffers;
//  * value wavefronts 4-7 own output columns 128 (w - 4) .. +127 for all 64
//    heads: O^T[128, 64] += V^T[128, 32 tok] P^T[32 tok, 64] on
//    v_mfma_f32_32x32x16_bf16 (16 MFMAs per tile, 128 accumulation
//    registers, V^T through transposing LDS reads, no value column read
//    twice), and they issue the tile loads.
// In step it the score wavefronts work on tile it while the value
// wavefronts accumulate tile it - 1 from the other weight buffer, so the two
// kinds of MFMA work overlap on every SIMD; with four tile stages and two
// weight buffers one barrier per step suffices.
// The weights of a range are taken against one fixed maximum per head, the
// first tile's, so the accumulators never need a rescale.  Weights up to
// 2^32 are harmless in bf16 and fp32 (sums stay far below the fp32 range
// for any cache length the entry point accepts); a range whose later scores
// exceed the first tile's maximum by more than that (never at ordinary score
// sizes) is computed a second time against its true maximum.  The slack is
// wide on purpose: the workgroup that takes a second pass sets the time of
// the whole launch.  Token ranges of a unit (sequence, KV head, head block) are
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
constexpr int kWaveHeads = kWideHeadBlock / kScoreWaves;   // 16 heads per score wavefront
constexpr int kKSteps = kDK / 32;                 // 18 score MFMAs per 16-token half
constexpr int kNB = kWideHeadBlock / 32;          // 32-head blocks
constexpr int kPvCols = kDV / (kWaves - kScoreWaves);   // 128 value columns per value wavefront
constexpr int kCB = kPvCols / 32;                 // 32-column blocks per value wavefront
constexpr int kChunks = kTok * kCPR;              // 16-byte chunks per tile
constexpr int kFillThreads = (kWaves - kScoreWaves) * 64;   // the value wavefronts load the tiles
constexpr int kLoads = kChunks / kFillThreads;    // 16-byte loads per filling thread per tile
// s_waitcnt immediate (gfx9 encoding) for vmcnt <= kLoads with the LDS and
// export counters left alone: after two tiles' loads have been issued, this
// waits for the older tile's.
constexpr int kWaitNewest = (kLoads & 0xF) | ((kLoads >> 4) << 14) | (0x7 << 4) | (0xF << 8);
constexpr int kPRow = kTok + 8;                   // bf16 per row of P (80 bytes: 5 chunks)
constexpr int kGroup = 6;                         // K operands read one group ahead of their MFMAs
constexpr float kLazyMax = 32.f;                  // log2 slack before a second pass
constexpr int kXcds = 8;

static_assert(kWideHeadBlock == 64 && kWaveHeads == 16 && kNB == 2 && kCB == 4, "64-head blocks");
static_assert(kKSteps % 2 == 0 && 2 * kKSteps % kGroup == 0, "score steps in whole groups");
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
  // four tile stages and two weight buffers as separate arrays, so that the
  // compiler can tell a read of one stage from the loads in flight into
  // another
  __shared__ __align__(16) __bf16 t0s[kChunks * 8];
  __shared__ __align__(16) __bf16 t1s[kChunks * 8];
  __shared__ __align__(16) __bf16 t2s[kChunks * 8];
  __shared__ __align__(16) __bf16 t3s[kChunks * 8];
  __shared__ __align__(16) __bf16 p0s[kWideHeadBlock * kPRow];   // weights [head][token], even tiles
  __shared__ __align__(16) __bf16 p1s[kWideHeadBlock * kPRow];   // odd tiles
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
  const int ntiles = (t_end - t_begin + kTok - 1) / kTok;

  // The weights of a range are taken against one fixed maximum per head,
  // the first tile's, so the accumulators are never rescaled.  If a later
  // tile's maximum exceeded it by more than kLazyMax (weights above 2^32,
  // which scores of ordinary size never reach) the range is computed again
  // against the largest maximum, which bounds every weight by 1.  The
  // decision is workgroup-wide, so both roles take part in the same
  // barriers; each role keeps to its own code path to the end, so that its
  // registers are never live in the other's loop.
  float m_fix = -INFINITY;    // score lanes: the maximum (log2 units) of head c16
  float m_seen = -INFINITY;   // score lanes: the largest score met so far (this lane's, then the head's)
  float l_run = 0.f;          // score lanes: this lane's share of the sum of weights
  auto second_pass = [&]() {
    const bool redo = __syncthreads_or(m_seen > m_fix + kLazyMax);
    if (redo) m_fix = m_seen;
    return redo;
  };

  if (scorer) {
    // Score role: heads 16 w + c16 over all 576 columns on
    // v_mfma_f32_16x16x32_bf16, S^T[16 tok, 16 heads] per half tile; then
    // the weights of the 32 tokens are published as P[head][token].
    const int c16 = lane & 15;   // head within the wavefront (B / D column) and K row
    const int kg = lane >> 4;    // contraction group
    const int hw = kWaveHeads * w + c16;   // head within the block
    const int head = kvh * a.g + min(hbase + hw, a.g - 1);
    // Q^T B operands: columns 32 kk + 8 kg .. +7 of head `head`.
    bf16x8 qb[kKSteps];
    // K operand (tb, kk): token 16 tb + c16, chunk 4 kk + kg; the swizzle
    // repeats every 16 rows and, for kk two apart, every 8 chunks, so two
    // bases cover all.  The empty asm hides the bases' value range so that
    // constants fold into the offset fields.
    int k_base[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      k_base[p] = c16 * kDK + wide_phys(c16, 4 * p + kg) * 8;
      asm volatile("" : "+v"(k_base[p]));
    }
    const int p_wr = hw * kPRow + 4 * kg;   // P row of this head, tokens 4 kg (+ 16 tb)
    auto tile = [&](const __bf16* ts, __bf16* pbuf, int t0, bool first) {
      // K operands (kk, tb) in the order n = 2 kk + tb, read in groups of
      // kGroup one group ahead of the MFMAs that use them (the scheduling
      // barriers keep the compiler from moving each read next to its use).
      auto k_op = [&](int n) {
        const int kk = n >> 1, tb = n & 1;
        return load_bf16x8(ts + k_base[kk & 1] + 64 * (kk >> 1) + tb * 16 * kDK);
      };
      f32x4 sc[2] = {f32x4{}, f32x4{}};
      bf16x8 kop[2][kGroup];
#pragma unroll
      for (int i = 0; i < kGroup; ++i) kop[0][i] = k_op(i);
#pragma unroll
      for (int g = 0; g < 2 * kKSteps / kGroup; ++g) {
        if (g + 1 < 2 * kKSteps / kGroup) {
#pragma unroll
          for (int i = 0; i < kGroup; ++i) kop[(g + 1) & 1][i] = k_op(kGroup * (g + 1) + i);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
          const int n = kGroup * g + i;
          sc[n & 1] = mfma16(kop[g & 1][i], qb[n >> 1], sc[n & 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // element e of half tb: token t0 + 16 tb + 4 kg + e of head hw
      float s[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[e] = sc[0][e] * a.scale_log2;
        s[4 + e] = sc[1][e] * a.scale_log2;
      }
      if (t0 + kTok > t_end) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = t0 + 16 * (e >> 2) + 4 * kg + (e & 3) < t_end ? s[e] : -INFINITY;
      }
      // Only the first tile of a pass needs the head's maximum across lanes
      // (it fixes m_fix); later tiles only track this lane's own maximum,
      // which is combined across lanes once, at the end of the pass.
      const float mx = max3f(max3f(s[0], s[1], s[2]), max3f(s[3], s[4], s[5]), fmaxf(s[6], s[7]));
      m_seen = fmaxf(m_seen, mx);
      if (first) {
        const float mh = fmaxf(mx, shfl_xor(mx, 16));
        m_fix = fmaxf(mh, shfl_xor(mh, 32));   // finite: the first tile holds a token
      }
      bf16x4 pw[2];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = fast_exp2(s[e] - m_fix);
        l_run += p;
        pw[e >> 2][e & 3] = (__bf16)p;
      }
      *reinterpret_cast<bf16x4*>(pbuf + p_wr) = pw[0];
      *reinterpret_cast<bf16x4*>(pbuf + p_wr + 16) = pw[1];
    };
    // Step it: tile it, weights into buffer it % 2; one barrier per step.
    // fix_max: the pass takes m_fix from its first tile (the first pass);
    // the second pass keeps the true maximum found by the first.
    auto run = [&](bool fix_max) {
      {
        const __bf16* qrow = a.q + ((size_t)b * a.hq + head) * kDK + 8 * kg;
#pragma unroll
        for (int kk = 0; kk < kKSteps; ++kk) qb[kk] = load_bf16x8(qrow + 32 * kk);
      }
      l_run = 0.f;
      lds_barrier();   // the first tile has landed
      for (int it = 0;; it += 4) {
        tile(t0s, p0s, t_begin + it * kTok, fix_max && it == 0);
        lds_barrier();
        if (it + 1 >= ntiles) break;
        tile(t1s, p1s, t_begin + (it + 1) * kTok, false);
        lds_barrier();
        if (it + 2 >= ntiles) break;
        tile(t2s, p0s, t_begin + (it + 2) * kTok, false);
        lds_barrier();
        if (it + 3 >= ntiles) break;
        tile(t3s, p1s, t_begin + (it + 3) * kTok, false);
        lds_barrier();
        if (it + 4 >= ntiles) break;
      }
    };
    // m_seen of a head: the largest of its four lanes' maxima
    auto head_seen = [&]() {
      const float m = fmaxf(m_seen, shfl_xor(m_seen, 16));
      m_seen = fmaxf(m, shfl_xor(m, 32));
    };
    run(true);
    head_seen();
    if (second_pass()) run(false);
    float l_tot = l_run + shfl_xor(l_run, 16);
    l_tot += shfl_xor(l_tot, 32);
    if (kg == 0) {
      lsum_s[hw] = l_tot;
      if (a.nranges > 1) a.part_lse[slot0 + hw] = m_fix + __log2f(l_tot);
    }
    __syncthreads();
    return;
  }

  // Value role (wavefronts 4-7): output columns 128 (w - 4) .. +127 for all
  // 64 heads, O^T[128, 64] += V^T[128, 32 tok] P^T[32 tok, 64], and the tile
  // loads.
  const int wv = w - kScoreWaves;
  const int l32 = lane & 31;
  const int j = lane >> 5;   // contraction group of the 32x32 operands
  // V^T operand (cb, kc): lane l reads column 128 wv + 32 cb + 16 ((l / 16)
  // % 2) + ..., rows 16 kc + 8 j + 4 q + (l % 16) / 4 for q = 0, 1
  // (transposing reads); the swizzle repeats every 16 rows, so kc is a
  // constant offset.
  int v_base[kCB][2];
  {
    const int L = lane & 15;
    const int ch = (lane >> 4) & 1;
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int row = 8 * j + 4 * q + (L >> 2);
        const int col = kPvCols * wv + 32 * cb + 16 * ch + 4 * (L & 3);
        v_base[cb][q] = row * kDK + wide_phys(row, col >> 3) * 8 + (col & 7);
        asm volatile("" : "+v"(v_base[cb][q]));
      }
  }
  // P^T operand (nb, kc): head 32 nb + l32, tokens 16 kc + 8 j .. +7.
  const int p_rd = l32 * kPRow + 8 * j;
  f32x16 acc[kCB][kNB];
  auto values = [&](const __bf16* ts, const __bf16* pbuf) {
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      bf16x8 va[kCB], pb[kNB];
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb)
        va[cb] = concat(lds_read_tr16(ts + v_base[cb][0] + 16 * kc * kDK),
                        lds_read_tr16(ts + v_base[cb][1] + 16 * kc * kDK));
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) pb[nb] = load_bf16x8(pbuf + p_rd + 32 * nb * kPRow + 16 * kc);
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) acc[cb][nb] = mfma32(va[cb], pb[nb], acc[cb][nb]);
    }
  };
  // Tile loads: thread tid - 256 deposits physical chunks (tid - 256) +
  // 256 i of a tile; source offsets are computed once.  Rows past the range
  // read as zeros without a memory access.
  const __bf16* kvb = a.kv + ((size_t)b * a.hkv + kvh) * (size_t)a.tcap * kDK;
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(kvb, t_end * kDK * 2);
  int fsrc[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int p = (tid - kScoreWaves * 64) + kFillThreads * i;
    const int row = p / kCPR;
    fsrc[i] = row * kDK * 2 + wide_phys(row, p - row * kCPR) * 16;
  }
  // The loads issue at raised wavefront priority, ahead of the score
  // wavefront that shares the SIMD (2-5% shorter launches).
  auto fill = [&](__bf16* dst, int tile_idx) {
    const int t0 = min(t_begin + tile_idx * kTok, t_end);   // past the range: zeros
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(dst + (wv * 64 + kFillThreads * i) * 8), 16,
                                               t0 * kDK * 2 + fsrc[i], 0, 0, kCacheDefault);
    __builtin_amdgcn_s_setprio(0);
  };
  // Step it: loads of tile it + 2, then tile it - 1 (weights in buffer
  // (it - 1) % 2), then wait for tile it + 1 and the step's barrier.
  auto step_end = [&]() {
    __builtin_amdgcn_s_waitcnt(kWaitNewest);   // this thread's loads of the next tile have landed
    lds_barrier();                             // ... everyone's; the step's weights are published
  };
  auto run = [&]() {
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) acc[cb][nb] = f32x16{};
    fill(t0s, 0);
    fill(t1s, 1);
    __builtin_amdgcn_s_waitcnt(kWaitNewest);
    lds_barrier();   // the first tile has landed
    fill(t2s, 2);    // step 0: no earlier tile to accumulate
    step_end();
    for (int it = 1;; it += 4) {
      fill(t3s, it + 2);
      values(t0s, p0s);
      if (it >= ntiles) break;
      step_end();
      fill(t0s, it + 3);
      values(t1s, p1s);
      if (it + 1 >= ntiles) break;
      step_end();
      fill(t1s, it + 4);
      values(t2s, p0s);
      if (it + 2 >= ntiles) break;
      step_end();
      fill(t2s, it + 5);
      values(t3s, p1s);
      if (it + 3 >= ntiles) break;
      step_end();
    }
    __builtin_amdgcn_s_waitcnt(0);   // no load into a stage outlives the pass
  };
  run();
  if (second_pass()) run();
  __syncthreads();   // the score wavefronts publish the denominators
  // O^T block (cb, nb): column 128 wv + 32 cb + 8 (rr / 4) + 4 j + rr % 4 of head 32 nb + l32
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
        *reinterpret_cast<f32x4*>(o + kPvCols * wv + 32 * cb + 8 * r4 + 4 * j) =
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
  // Four ranges per round, each range's lse and output loaded together (one
  // round trip for up to four ranges), combined online against the running
  // maximum.  The output of an empty range is never written, so it is
  // selected away rather than multiplied by its zero weight.
  float mx = -INFINITY, den = 0.f;
  f32x4 acc = f32x4{};
  for (int r0 = 0; r0 < nranges; r0 += 4) {
    float lr[4];
    f32x4 ov[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = r0 + u;
      const size_t slot = ((size_t)min(r, nranges - 1) * units + unit) * kWideHeadBlock + lane_slot;
      lr[u] = r < nranges ? part_lse[slot] : -INFINITY;
      ov[u] = *reinterpret_cast<const f32x4*>(part_o + slot * kDV + 4 * c4);
    }
    const float mn = fmaxf(mx, fmaxf(fmaxf(lr[0], lr[1]), fmaxf(lr[2], lr[3])));
    if (mn == -INFINITY) continue;   // no tokens so far
    const float rs = fast_exp2(mx - mn);
    den *= rs;
    acc *= rs;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float wgt = fast_exp2(lr[u] - mn);
      den += wgt;
      acc += lr[u] == -INFINITY ? f32x4{} : wgt * ov[u];
    }
    mx = mn;
  }
  if (mx != -INFINITY) acc *= 1.f / den;
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
