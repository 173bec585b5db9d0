// Causal GQA prefill (flash attention forward) on gfx950 bf16 matrix cores.
//
// Row i of query head h attends to keys 0..i of KV head h/g (lower-triangular
// mask broadcast over the group; anrans.github.io, "Attention variants: MQA,
// GQA, MLA", section "Kernels do not need to copy the KV heads", whose
// grouped form stacks the g query heads of a group as extra query rows
// against the one shared K/V).  Prefill is a dense contraction, so QK^T and
// PV run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation; the score
// matrix lives only in registers and never reaches HBM.
//
// Workgroup = 4 wavefronts = 128 query rows of ONE KV head: Gw query heads
// of the group x Mq = 128/Gw consecutive positions (Gw = 4, 2 or 1, the
// largest dividing g).  Each 64-key K/V tile is loaded into LDS once and used
// by all Gw heads.  Wavefront w owns 32 rows (one head, 32 positions) and
// keeps:
//   Q^T      as MFMA B operands in registers (loaded once),
//   S^T      [64 keys, 32 rows] = K Q^T in registers,
//   O^T      [d, 32 rows] fp32 accumulators.
// The online softmax keeps a per-row reference point m for the weights
// exp2(s*scale*log2e - m) and moves it only when a tile's maximum exceeds it
// by more than 2^8 in weight, so the accumulators are rescaled on few tiles
// (softmax is shift-invariant, so the result is the same).
// The tile loop is software-pipelined within each wavefront: step it issues
// the score MFMAs of tile it + 1 and computes the weights of tile it between
// them (a branch-free block whose groups are fenced so that the compiler
// keeps the interleave), so the softmax arithmetic runs while the matrix
// core works; then tile it is accumulated.  K and V have two LDS stages
// each, filled by direct global-to-LDS buffer loads (no register staging):
// step it reads K(it + 1) and V(it) and loads K(it + 2) and V(it + 1) into
// the stages the previous step finished with, so one barrier per step
// suffices.  The stages are separate LDS arrays and the loop is unrolled by
// two, so the compiler can see that reading one stage does not alias the
// loads in flight into another.  Tiles are stored in 16-byte
// chunks with the chunk index XOR-ed by a rotation of the key index, which
// keeps both the K reads (ds_read_b128, 16 keys x one chunk per 16 lanes)
// and the transposing V reads (ds_read_b64_tr_b16, 4 keys x 2 chunks per 16
// lanes) free of bank conflicts.  Key tiles above a wavefront's diagonal are
// skipped and the mask is applied only where a tile crosses it.  Workgroups
// are issued heaviest-first and, when the (sequence, KV head) count allows,
// all q-tiles of one KV head land on the same XCD so its K/V stays in one L2.

#include "gqa_device.hpp"
#include "gqa_launch.hpp"
#include "prefill_tiles.hpp"

namespace gqa {

namespace {

constexpr int kRows = 128;   // query rows per workgroup
constexpr int kBN = tiles::kRows;   // keys per tile
constexpr int kXcds = 8;
constexpr int kPrefillThreads = tiles::kThreads;

// Per-lane constants of a wavefront: its Q operands and the LDS element
// offsets of its K and V operands within a tile.  The tile swizzle repeats
// every 16 rows, so key block kb (32 rows) and 16-key chunk c are constant
// offsets (32 kb D and 16 c D) from the bases kept here.
template <int D>
struct Lane {
  static constexpr int KSTEPS = D / 16;
  static constexpr int DB = D / 32;
  bf16x8 qb[KSTEPS];   // Q^T B operands: q[pos][16kk + 8j .. +7]
  int k_rd[KSTEPS];    // K: key row (of key block 0), logical chunk 2kk + j
  int v_rd[DB];        // V (transposed), chunk 0: key 4j + L/4, column 32db + dlo + 4(L%4)
  int v_dx[DB];        // offset correction of the same column 8 keys later
};

// Online-softmax state of a wavefront's 32 query rows: weights are
// 2^(s * scale * log2 e - r) for a per-row reference point r (log2 domain).
template <int D>
struct RowState {
  float r, lsum;              // reference point and this lane's share of the sum
  f32x16 acc[D / 32];         // O^T[d, rows]
};

// S^T[64 keys, 32 rows] = K Q^T of one tile, as two 32-key blocks.
template <int D>
__device__ __forceinline__ void scores(const __bf16* ks, const Lane<D>& ln, f32x16 (&sc)[2]) {
  constexpr int KSTEPS = Lane<D>::KSTEPS;
  sc[0] = f32x16{};
  sc[1] = f32x16{};
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sc[kb] = mfma32(load_bf16x8(ks + ln.k_rd[kk] + 32 * kb * D), ln.qb[kk], sc[kb]);
}

// Keys after the row (and past the end) become -inf, by a select, in a tile
// that crosses the diagonal.  sc[kb][r] is the score of key t0 + 32kb +
// 8(r/4) + 4j + r%4 for query row `pos`.
__device__ __forceinline__ void mask_scores(f32x16 (&sc)[2], int t0, int pos, int n, int j) {
  const int lim = min(pos, n - 1);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = t0 + 32 * kb + 8 * (r >> 2) + 4 * j + (r & 3);
      sc[kb][r] = t <= lim ? sc[kb][r] : -INFINITY;
    }
}

// One pipelined step's arithmetic in one branch-free block: the scores of
// the next tile (K reads and MFMAs into sn) and the weights of this one
// (2^(sc * mult - r) -> bf16 P^T as four B operands: key chunk c holds keys
// 16c + 4j + 0..3, then 16c + 8 + 4j + 0..3) with this lane's share of
// their sum.  It is written as KSTEPS groups fenced by scheduling barriers:
// group kk issues the K reads of step kk + 1, the two MFMAs of step kk and
// four of the weights, so the weights are computed while the matrix core
// runs.  No row maximum is taken here: the weights are relative to the
// reference point, and the caller checks afterwards that none of them grew
// past 2^8.  mult > 0 multiplies raw scores into the log2 domain (scale *
// log2 e, folded into the weight's FMA); the caller passes scores already
// scaled and mult = 1 for a zero or negative scale.
template <int D>
__device__ __forceinline__ void scores_and_weights(const __bf16* kn, const Lane<D>& ln, f32x16 (&sn)[2],
                                                   const f32x16 (&sc)[2], float mult, float r, bf16x8 (&pb)[4],
                                                   float& ps) {
  constexpr int KSTEPS = Lane<D>::KSTEPS;
  constexpr int kPerGroup = 32 / KSTEPS;   // weights per group
  static_assert(kPerGroup % 2 == 0, "weights pair up for the row sums");
  sn[0] = f32x16{};
  sn[1] = f32x16{};
  bf16x8 kop[2][2];
  kop[0][0] = load_bf16x8(kn + ln.k_rd[0]);
  kop[0][1] = load_bf16x8(kn + ln.k_rd[0] + 32 * D);
  ps = 0.f;
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    if (kk + 1 < KSTEPS) {
      kop[(kk + 1) & 1][0] = load_bf16x8(kn + ln.k_rd[kk + 1]);
      kop[(kk + 1) & 1][1] = load_bf16x8(kn + ln.k_rd[kk + 1] + 32 * D);
    }
    sn[0] = mfma32(kop[kk & 1][0], ln.qb[kk], sn[0]);
    sn[1] = mfma32(kop[kk & 1][1], ln.qb[kk], sn[1]);
    // weights e0 .. e0 + kPerGroup - 1 of the 32 (element e: block e / 16, register e % 16)
    const int e0 = kk * kPerGroup;
#pragma unroll
    for (int e = e0; e < e0 + kPerGroup; ++e) {
      float pe = fast_exp2(__builtin_fmaf(sc[e >> 4][e & 15], mult, -r));
      asm volatile("" : "+v"(pe));   // keeps the weight in this group (not sunk to its use)
      pb[e >> 3][e & 7] = (__bf16)pe;
    }
    // the denominator sums exactly the bf16 weights PV uses (2 per dot)
#pragma unroll
    for (int e = e0; e < e0 + kPerGroup; e += 2)
      ps = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[e >> 3][e & 7], pb[e >> 3][(e & 7) + 1]}, ones, ps, false);
    asm volatile("" : "+v"(ps));
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The rare path of a step, taken when some weight of the tile may exceed
// 2^8 (a lane's partial sum above 2^8, which includes overflow to infinity)
// or on a wavefront's first tile (forced: r then becomes the first tile's
// row maximum).  A row whose tile maximum exceeds r + 8 moves its reference
// point up to that maximum: its weights are recomputed and its accumulators
// and sum so far are rescaled by 2^(r_old - r_new).
template <int D>
__device__ __forceinline__ void rebase_rows(RowState<D>& st, const f32x16 (&sc)[2], float mult, bf16x8 (&pb)[4],
                                            float& ps, bool first) {
  constexpr float kSlack = 8.f;   // log2 of the largest weight kept without a rebase
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
  // rows pair lanes l and l + 32; a positive mult keeps the maximum the maximum
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * mult;
  // every row's first tile holds key 0, so mx is finite there
  const float r_new = (first || mx > st.r + kSlack) ? mx : st.r;
  if (__builtin_amdgcn_ballot_w64(r_new != st.r) == 0) return;   // the weights stand
  if (!first) {   // (on the first tile the sum and accumulators are still zero)
    const float alpha = fast_exp2(st.r - r_new);
    st.lsum *= alpha;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) st.acc[i] *= alpha;
  }
  st.r = r_new;
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
  ps = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) pb[e >> 3][e & 7] = (__bf16)fast_exp2(__builtin_fmaf(sc[e >> 4][e & 15], mult, -r_new));
#pragma unroll
  for (int e = 0; e < 32; e += 2)
    ps = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[e >> 3][e & 7], pb[e >> 3][(e & 7) + 1]}, ones, ps, false);
}

// O^T[d, rows] += V^T[d, 16 keys] P^T[16 keys, rows] over the tile's four
// key chunks; the V operands of the next chunk load during this chunk's
// MFMAs.
template <int D>
__device__ __forceinline__ void accumulate(const __bf16* vs, const Lane<D>& ln, const bf16x8 (&pb)[4],
                                           RowState<D>& st) {
  constexpr int DB = D / 32;
  bf16x8 va[2][DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) va[0][db] = tiles::read_tr<D>(vs, ln.v_rd[db], ln.v_dx[db]);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (c + 1 < 4) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
        va[(c + 1) & 1][db] = tiles::read_tr<D>(vs + 16 * (c + 1) * D, ln.v_rd[db], ln.v_dx[db]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < DB; ++db) st.acc[db] = mfma32(va[c & 1][db], pb[c], st.acc[db]);
  }
}

template <int D>
__global__ __launch_bounds__(kPrefillThreads) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_causal_bf16(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                         const __bf16* __restrict__ v, float* __restrict__ out,
                         float* __restrict__ lse, int hq, int hkv, int n, int g, int gw,
                         int n_qtiles, int units, float scale_log2) {
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = kBN * D;         // bf16 elements per K or V tile
  __shared__ __align__(16) __bf16 k0s[TILE];
  __shared__ __align__(16) __bf16 k1s[TILE];
  __shared__ __align__(16) __bf16 v0s[TILE];
  __shared__ __align__(16) __bf16 v1s[TILE];

  // Workgroup -> (unit = (b, kvh, head block), q-tile), heaviest tiles first.
  int unit, qt;
  {
    const int wg = blockIdx.x;
    if (units % kXcds == 0) {
      const int xcd = wg % kXcds, slot = wg / kXcds, per = units / kXcds;
      unit = xcd * per + slot % per;
      qt = n_qtiles - 1 - slot / per;
    } else {
      unit = wg % units;
      qt = n_qtiles - 1 - wg / units;
    }
  }
  const int nhb = g / gw;
  const int b = unit / (hkv * nhb);
  const int rem = unit - b * hkv * nhb;
  const int kvh = rem / nhb;
  const int hb = rem - kvh * nhb;
  const int mq = kRows / gw;
  const int q0 = qt * mq;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS addresses stay scalar
  const int row = lane & 31;   // query row within the wave (B/D column)
  const int j = lane >> 5;     // contraction group
  const int head = kvh * g + hb * gw + (32 * w) / mq;
  const int pos0 = q0 + (32 * w) % mq;
  const int pos = pos0 + row;

  Lane<D> ln;
  {
    const __bf16* qrow = q + (((size_t)b * hq + head) * n + min(pos, n - 1)) * D;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) ln.qb[kk] = load_bf16x8(qrow + 16 * kk + 8 * j);
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      ln.k_rd[kk] = tiles::row_offset<D>(row, 2 * kk + j);
      asm volatile("" : "+v"(ln.k_rd[kk]));
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      tiles::tr_offsets<D>(lane, 0, db, ln.v_rd[db], ln.v_dx[db]);
      asm volatile("" : "+v"(ln.v_rd[db]));
    }
  }

  // K/V of this (sequence, KV head); rows >= n read as zeros.
  const size_t kv_off = ((size_t)b * hkv + kvh) * (size_t)n * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + kv_off, n * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + kv_off, n * D * 2);
  const tiles::TileFill<D> fill(tid);

  RowState<D> st;
  st.r = 0.f;
  st.lsum = 0.f;
#pragma unroll
  for (int i = 0; i < DB; ++i) st.acc[i] = f32x16{};

  const int kv_hi = min(n, q0 + mq);       // keys any row of the workgroup needs
  const int wave_hi = min(n, pos0 + 32);   // keys this wavefront needs
  const int ntiles = (kv_hi + kBN - 1) / kBN;
  const int nt_w = (wave_hi + kBN - 1) / kBN;   // tiles this wavefront needs (a prefix, at least one)

  // Software pipeline over the tiles: in step it the scores of tile it + 1
  // are issued on the matrix cores first, and the weights of tile it (whose
  // scores the previous step produced) are computed while those MFMAs run;
  // then tile it is accumulated.  K and V have two LDS stages each: step it
  // reads K(it + 1) and V(it) and loads K(it + 2) and V(it + 1) into the
  // stages that step it - 1 finished with, so one barrier per step suffices.
  fill.issue(k0s, rk, w, 0);
  fill.issue(v0s, rv, w, 0);
  if (ntiles > 1) fill.issue(k1s, rk, w, kBN);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 sc[2];
  scores<D>(k0s, ln, sc);   // tile 0: every row needs key 0
  __syncthreads();          // k0s is free for K(2)

  // One step; kn/vc hold K(it + 1)/V(it), kf/vf receive K(it + 2)/V(it + 1).
  // The tile loads and the end-of-step wait run at raised wavefront priority,
  // so that they do not queue behind the other wavefront's arithmetic on the
  // SIMD.
  auto step = [&](const __bf16* kn, const __bf16* vc, __bf16* kf, __bf16* vf, int it) {
    __builtin_amdgcn_s_setprio(2);
    if (it + 2 < ntiles) fill.issue(kf, rk, w, (it + 2) * kBN);
    if (it + 1 < ntiles) fill.issue(vf, rv, w, (it + 1) * kBN);
    __builtin_amdgcn_s_setprio(0);
    f32x16 sn[2];
    if (it < nt_w) {
      const int t0 = it * kBN;
      if (t0 + kBN > pos0 || t0 + kBN > n) mask_scores(sc, t0, pos, n, j);
      if (scale_log2 <= 0.f) {
        // zero or negative scale: scale first, keeping masked keys at -inf
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[kb][r] = sc[kb][r] == -INFINITY ? -INFINITY : sc[kb][r] * scale_log2;
      }
      const float mult = scale_log2 > 0.f ? scale_log2 : 1.f;
      // (after the wavefront's last tile the scores of the next are computed
      // but never used: reading a stage that holds no tile is harmless)
      bf16x8 pb[4];
      float ps;
      scores_and_weights<D>(kn, ln, sn, sc, mult, st.r, pb, ps);
      if (__builtin_amdgcn_ballot_w64(it == 0 || !(ps <= 256.f)) != 0) rebase_rows<D>(st, sc, mult, pb, ps, it == 0);
      st.lsum += ps;
      accumulate<D>(vc, ln, pb, st);
    }
    sc[0] = sn[0];
    sc[1] = sn[1];
    __builtin_amdgcn_s_setprio(2);
    __builtin_amdgcn_s_waitcnt(0);   // this thread's loads for the next step have landed
    __syncthreads();                 // ... everyone's, and the stages read here are free again
    __builtin_amdgcn_s_setprio(0);
  };
  for (int it = 0; it < ntiles; it += 2) {
    step(k1s, v0s, k0s, v1s, it);
    if (it + 1 >= ntiles) break;
    step(k0s, v1s, k1s, v0s, it + 1);
  }

  const float lsum = st.lsum + shfl_xor(st.lsum, 32);
  if (pos < n) {
    const float inv = 1.f / lsum;
    float* orow = out + (((size_t)b * hq + head) * n + pos) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 o4;
#pragma unroll
        for (int r = 0; r < 4; ++r) o4[r] = st.acc[db][4 * r4 + r] * inv;
        *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * r4 + 4 * j) = o4;
      }
    if (lse != nullptr && j == 0) lse[((size_t)b * hq + head) * n + pos] = (st.r + __log2f(lsum)) * kLn2;
  }
}

}  // namespace

hipError_t launch_prefill_causal(const void* q, const void* k, const void* v, float* out,
                                 float* lse, const PrefillShape& s, hipStream_t stream) {
  const int g = s.hq / s.hkv;
  const int gw = (g % 4 == 0) ? 4 : (g % 2 == 0 ? 2 : 1);
  const int mq = kRows / gw;
  const int n_qtiles = (s.n + mq - 1) / mq;
  const int units = s.batch * s.hkv * (g / gw);
  const dim3 grid((unsigned)units * (unsigned)n_qtiles);
  const float sl2 = s.scale * kLog2e;
  auto qp = static_cast<const __bf16*>(q);
  auto kp = static_cast<const __bf16*>(k);
  auto vp = static_cast<const __bf16*>(v);
  if (s.d == 128)
    hipLaunchKernelGGL(prefill_causal_bf16<128>, grid, dim3(kPrefillThreads), 0, stream, qp, kp, vp,
                       out, lse, s.hq, s.hkv, s.n, g, gw, n_qtiles, units, sl2);
  else
    hipLaunchKernelGGL(prefill_causal_bf16<64>, grid, dim3(kPrefillThreads), 0, stream, qp, kp, vp,
                       out, lse, s.hq, s.hkv, s.n, g, gw, n_qtiles, units, sl2);
  return hipGetLastError();
}

}  // namespace gqa
