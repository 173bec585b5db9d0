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
// is about registers and LDS bandwidth:
//  * a workgroup is 8 wavefronts serving 64 query heads of one KV head over
//    one token range; every 32-token tile of 576-column rows (36 KiB) is
//    brought into LDS once by direct global-to-LDS loads, double-buffered,
//    and read by all eight wavefronts;
//  * the four wavefronts of a quad share 32 heads.  Each computes a quarter
//    of S^T[32 tok, 32 heads] = K Q^T (9 of the 36 contraction steps of
//    v_mfma_f32_32x32x16_bf16, its quarter of Q^T in 36 registers), the quad
//    adds the quarters through LDS in one fixed order (so all four hold the
//    same scores bit for bit), and each then accumulates a quarter of
//    O^T[512, 32 heads] += V^T P^T (128 columns, 64 accumulation registers,
//    V^T by transposing LDS reads).  That keeps a wavefront under 256
//    registers, so two run on every SIMD and hide each other's LDS and
//    softmax time; a single wavefront per SIMD cannot (one wavefront alone
//    draws only about a quarter of a CU's LDS read bandwidth);
//  * the weights of a range are taken against one fixed maximum, the first
//    tile's; weights up to 2^8 are harmless in bf16 and fp32, and a range
//    whose later scores exceed that (not met at ordinary score sizes) is
//    computed a second time against its true maximum, so the accumulators
//    are never rescaled;
//  * token ranges of a unit (sequence, KV head, head block) are merged by
//    their log-sum-exp, as in the narrow decode, when there is more than
//    one; the head blocks of a (sequence, range) run on one XCD so the second
//    one finds the tile in L2.
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
constexpr int kQuad = 4;                          // wavefronts sharing 32 heads
constexpr int kKSteps = kDK / 16;                 // score MFMAs per tile and head block
constexpr int kKPart = kKSteps / kQuad;           // ... per wavefront
constexpr int kVBlocks = kDV / 32 / kQuad;        // 32-column value blocks per wavefront
constexpr int kTileElems = kTok * kDK;
constexpr int kLoads = kTok * kCPR / kFillThreads;   // 16-byte loads per filling thread per tile
constexpr float kLazyMax = 8.f;                   // log2 slack before a rescale
constexpr int kXcds = 8;

static_assert(kTok * kCPR % kFillThreads == 0, "tile must split evenly over the filling threads");
static_assert(kWideHeadBlock == 2 * 32, "two quads of 32 heads");
static_assert(kKSteps % kQuad == 0 && (kDV / 32) % kQuad == 0, "steps and columns split over a quad");

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Low-bit swizzle of row r: a rotation of (r / 2) mod 8.
__device__ __forceinline__ int wide_swz(int r) {
  const int x = (r >> 1) & 7;
  return ((x << 1) | (x >> 2)) & 7;
}

// Physical chunk of logical chunk c in row r (an involution on the low bits).
__device__ __forceinline__ int wide_phys(int r, int c) { return (c & ~7) | ((c ^ wide_swz(r)) & 7); }

// Workgroup barrier that orders LDS only: unlike __syncthreads it does not
// wait for the next tile's global-to-LDS loads still in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

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
  __shared__ __align__(16) f32x4 xch[8 * 4 * 64];   // partial scores: [wave][4 floats of 16][lane]

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
  const int quad = w >> 2;     // the quad's 32 heads
  const int part = w & 3;      // score steps and value columns of this wavefront
  const int col = lane & 31;   // this lane's query head within the quad (B / D column)
  const int j = lane >> 5;     // contraction group
  const int hl = hb * kWideHeadBlock + 32 * quad + col;   // head within the group
  const bool head_ok = hl < a.g;
  const int head = kvh * a.g + min(hl, a.g - 1);
  const size_t slot = ((size_t)r * a.units + unit) * kWideHeadBlock + 32 * quad + col;
  const int vcol0 = part * (kDV / kQuad);   // first value column of this wavefront

  if (t_begin >= t_end) {   // nothing to attend in this range (uniform over the workgroup)
    if (a.nranges > 1) {
      if (j == 0 && part == 0) a.part_lse[slot] = -INFINITY;
    } else if (head_ok) {
      float* o = a.out + ((size_t)b * a.hq + head) * kDV + vcol0;
      for (int i = 4 * j; i < kDV / kQuad; i += 8) *reinterpret_cast<f32x4*>(o + i) = f32x4{};
    }
    return;
  }

  // This wavefront's quarter of Q^T as B operands: head `col`, columns
  // 16 (kk0 + i) + 8 j .. +7 for its score steps kk0 .. kk0 + 8.
  const int kk0 = part * kKPart;
  bf16x8 qb[kKPart];
  {
    const __bf16* qrow = a.q + ((size_t)b * a.hq + head) * kDK;
#pragma unroll
    for (int i = 0; i < kKPart; ++i) qb[i] = load_bf16x8(qrow + 16 * (kk0 + i) + 8 * j);
  }

  // LDS offsets.  K rows: token `col`, chunk 2 kk + j; the swizzle repeats
  // every 4 kk, so four bases plus 64-element steps cover all steps.  V^T:
  // tokens 16 c + 4 j + 0..3 (and + 8), columns 32 db + ...; the swizzle
  // does not depend on c and repeats every two db.  The empty asm hides the
  // bases' value range so that constants fold into the instructions' offsets.
  int k_base[4], v_base[2], v_dx[2];
#pragma unroll
  for (int m = 0; m < 4; ++m) {   // step kk0 + m; step kk0 + m + 4 n is 64 n elements further
    const int c = 2 * (kk0 + m) + j;
    k_base[m] = col * kDK + ((c & ~7) | ((c ^ wide_swz(col)) & 7)) * 8;
    asm volatile("" : "+v"(k_base[m]));
  }
  {
    const int L = lane & 15;
    const int row = 4 * j + (L >> 2);
    const int hcol = 16 * ((lane >> 4) & 1);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int colv = 32 * p + hcol + 4 * (L & 3);
      const int ch = colv >> 3;
      v_base[p] = row * kDK + wide_phys(row, ch) * 8 + (colv & 7);
      v_dx[p] = (wide_phys(row + 8, ch) - wide_phys(row, ch)) * 8;
      asm volatile("" : "+v"(v_base[p]));
    }
  }
  // K operand of this wavefront's score step kk0 + i
  auto k_op = [&](const __bf16* ts, int i) { return load_bf16x8(ts + k_base[i & 3] + 64 * (i >> 2)); };
  // value block db (32 columns, counted from column 0) of 16-token half c
  auto v_op = [&](const __bf16* ts, int c, int db) {
    const int rd = v_base[db & 1] + c * 16 * kDK + 64 * (db >> 1);
    return concat(lds_read_tr16(ts + rd), lds_read_tr16(ts + rd + 8 * kDK + v_dx[db & 1]));
  };

  // Tile fill: thread tid < 256 deposits physical chunks tid + 256 i.
  int src_off[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int p = (tid & (kFillThreads - 1)) + kFillThreads * i;
    const int row = p / kCPR;
    const int ph = p - row * kCPR;
    src_off[i] = row * kDK * 2 + wide_phys(row, ph) * 16;
  }
  const __bf16* kvb = a.kv + ((size_t)b * a.hkv + kvh) * (size_t)a.tcap * kDK;
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(kvb, t_end * kDK * 2);   // rows >= t_end read as 0
  auto fill = [&](__bf16* dst, int t0) {
    if (w < kFillThreads / 64) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(dst + (w * 64 + kFillThreads * i) * 8), 16,
                                                 t0 * kDK * 2 + src_off[i], 0, 0, kCacheStream);
    }
  };

  f32x16 acc[kVBlocks];
  float m_fix = -INFINITY;    // the maximum (log2 units) the weights are taken against
  float m_seen = -INFINITY;   // the largest tile maximum met so far
  float l_run = 0.f;          // this lane's share of the sum of weights
  f32x4* xmine = xch + (w * 4) * 64 + lane;
  const f32x4* xquad = xch + (quad * kQuad * 4) * 64 + lane;   // the quad's four partials

  // One tile.  Operands are read in groups of four, one group ahead of the
  // MFMAs that use them.
  auto tile = [&](const __bf16* ts, int t0) {
    constexpr int G = 4;
    f32x16 s0 = f32x16{}, s1 = f32x16{};
    bf16x8 op[2][G];
    constexpr int NGK = (kKPart + G - 1) / G;
#pragma unroll
    for (int i = 0; i < G; ++i) op[0][i] = k_op(ts, i);
#pragma unroll
    for (int grp = 0; grp < NGK; ++grp) {
      if (grp + 1 < NGK) {
#pragma unroll
        for (int i = 0; i < G; ++i)
          if (G * (grp + 1) + i < kKPart) op[(grp + 1) & 1][i] = k_op(ts, G * (grp + 1) + i);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const int kk = G * grp + i;
        if (kk < kKPart) {
          if (i & 1) s1 = mfma32(op[grp & 1][i], qb[kk], s1);
          else s0 = mfma32(op[grp & 1][i], qb[kk], s0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // The quad adds its quarters: publish this one, then add all four in
    // quad order (the same operations in every wavefront of the quad).
    const f32x16 sh = s0 + s1;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) xmine[q4 * 64] = f32x4{sh[4 * q4], sh[4 * q4 + 1], sh[4 * q4 + 2], sh[4 * q4 + 3]};
    lds_barrier();
    // element e: token t0 + 8 (e/4) + 4 j + e%4 of head `col`
    float s[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      f32x4 sum = xquad[(0 * 4 + q4) * 64];
#pragma unroll
      for (int p = 1; p < kQuad; ++p) sum += xquad[(p * 4 + q4) * 64];
#pragma unroll
      for (int e = 0; e < 4; ++e) s[4 * q4 + e] = sum[e] * a.scale_log2;
    }
    // The first value operands load while the softmax runs.
#pragma unroll
    for (int i = 0; i < G; ++i) op[0][i] = v_op(ts, 0, part * kVBlocks + i);
    if (t0 + kTok > t_end) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = t0 + 8 * (e >> 2) + 4 * j + (e & 3);
        s[e] = t < t_end ? s[e] : -INFINITY;
      }
    }
    float mx = max3f(s[0], s[1], s[2]);
#pragma unroll
    for (int e = 3; e < 15; e += 2) mx = max3f(mx, s[e], s[e + 1]);
    mx = fmaxf(mx, s[15]);
    mx = fmaxf(mx, shfl_xor(mx, 32));
    m_seen = fmaxf(m_seen, mx);
    m_fix = m_fix == -INFINITY ? mx : m_fix;   // the first tile fixes it (every tile has a token)
    bf16x8 pb[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = fast_exp2(s[e] - m_fix);
      l_run += p;
      pb[e >> 3][e & 7] = (__bf16)p;
    }
    __builtin_amdgcn_sched_barrier(0);
    // O^T[128 cols, 32 heads] += V^T[128, 16 tok] P^T[16 tok, 32 heads] for
    // the two 16-token halves; group n covers the four blocks of half n / PER.
    constexpr int PER = kVBlocks / G;
    constexpr int NG = 2 * PER;
#pragma unroll
    for (int n = 0; n < NG; ++n) {
      if (n + 1 < NG) {
#pragma unroll
        for (int i = 0; i < G; ++i)
          op[(n + 1) & 1][i] = v_op(ts, (n + 1) / PER, part * kVBlocks + G * ((n + 1) % PER) + i);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const int db = G * (n % PER) + i;
        acc[db] = mfma32(op[n & 1][i], pb[n / PER], acc[db]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The accumulators are never rescaled inside the loop (a conditional
  // rescale of 128 accumulation registers costs the loop 128 register moves
  // per tile).  The first pass takes the weights against the first tile's
  // maximum; if a later tile's maximum exceeded it by more than kLazyMax
  // (weights above 2^8, which scores of ordinary size never reach) the range
  // is computed again against the largest maximum, which bounds every weight
  // by 1.
  const int ntiles = (t_end - t_begin + kTok - 1) / kTok;
  auto run = [&]() {
#pragma unroll
    for (int i = 0; i < kVBlocks; ++i) acc[i] = f32x16{};
    l_run = 0.f;
    fill(t0s, t_begin);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int it = 0; it < ntiles; it += 2) {
      if (it + 1 < ntiles) fill(t1s, t_begin + (it + 1) * kTok);
      tile(t0s, t_begin + it * kTok);
      __builtin_amdgcn_s_waitcnt(0);   // this thread's loads of the next tile have landed
      __syncthreads();                 // ... everyone's; stage 0 and the exchange are free again
      if (it + 1 >= ntiles) break;
      if (it + 2 < ntiles) fill(t0s, t_begin + (it + 2) * kTok);
      tile(t1s, t_begin + (it + 1) * kTok);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  };
  run();
  // Workgroup-wide decision, so every wavefront takes part in the same
  // barriers; the second pass is a separate copy of the loop so that the
  // accumulators are carried by one simple loop at a time.
  if (__syncthreads_or(m_seen > m_fix + kLazyMax)) {
    m_fix = m_seen;
    run();
  }

  const float l_tot = l_run + shfl_xor(l_run, 32);
  if (!head_ok) return;
  const float inv = 1.f / l_tot;
  float* o = (a.nranges > 1 ? a.part_o + slot * kDV : a.out + ((size_t)b * a.hq + head) * kDV) + vcol0;
#pragma unroll
  for (int db = 0; db < kVBlocks; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = acc[db][4 * r4 + e] * inv;
      *reinterpret_cast<f32x4*>(o + 32 * db + 8 * r4 + 4 * j) = o4;
    }
  if (a.nranges > 1 && j == 0 && part == 0) a.part_lse[slot] = m_fix + __log2f(l_tot);
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
