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
// K/V tiles are double-buffered in LDS and filled by direct global-to-LDS
// buffer loads (no register staging) while the previous tile is computed;
// one barrier per tile.  The two stages are separate LDS arrays and the loop
// is unrolled by two, so the compiler can see that reading one stage does not
// alias the loads in flight into the other.  Tiles are stored in 16-byte
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
constexpr float kSlack = 8.f;   // log2 of the largest weight before a rescale

// Per-lane constants of a wavefront: its Q operands and the LDS element
// offsets of its K and V operands within a tile.
template <int D>
struct Lane {
  static constexpr int KSTEPS = D / 16;
  static constexpr int DB = D / 32;
  bf16x8 qb[KSTEPS];     // Q^T B operands: q[pos][16kk + 8j .. +7]
  int k_rd[2][KSTEPS];   // K: key 32*kb + row, logical chunk 2kk + j
  int v_rd[4][DB];       // V (transposed): key 16c + 4j + L/4, column 32db + dlo + 4(L%4)
  int v_dx[4][DB];       // offset correction of the same column 8 keys later
};

// Online-softmax state of a wavefront's 32 query rows.
template <int D>
struct RowState {
  float m, lsum;              // running max (log2 domain) and this lane's share of the sum
  f32x16 acc[D / 32];         // O^T[d, rows]
};

template <int D>
__device__ __forceinline__ void attend_tile(const __bf16* ks, const __bf16* vs, const Lane<D>& ln,
                                            RowState<D>& st, int t0, int pos0, int pos, int n,
                                            int j, float scale_log2) {
  constexpr int KSTEPS = Lane<D>::KSTEPS;
  constexpr int DB = Lane<D>::DB;
  // All K operands of the tile are read before the first MFMA so the LDS
  // latency is paid once, not once per step.
  bf16x8 ka[KSTEPS][2];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) ka[kk][kb] = load_bf16x8(ks + ln.k_rd[kb][kk]);
  __builtin_amdgcn_sched_barrier(0);
  f32x16 sc[2] = {f32x16{}, f32x16{}};
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sc[kb] = mfma32(ka[kk][kb], ln.qb[kk], sc[kb]);
  // The first V operands load while the softmax runs.
  bf16x8 va[2][DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
    va[0][db] = tiles::read_tr<D>(vs, ln.v_rd[0][db], ln.v_dx[0][db]);
  __builtin_amdgcn_sched_barrier(0);

  // sc[kb][r] = raw score of key t0 + 32*kb + 8*(r/4) + 4*j + r%4, query row
  // `pos`.  Keys after the row (and past the end) become -inf, by a select,
  // only in tiles that cross the diagonal.
  if (t0 + kBN > pos0 || t0 + kBN > n) {
    const int lim = min(pos, n - 1);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t0 + 32 * kb + 8 * (r >> 2) + 4 * j + (r & 3);
        sc[kb][r] = t <= lim ? sc[kb][r] : -INFINITY;
      }
  }
  // Row maximum of the tile in the log2 domain (scale * log2 e folded in).
  float mx = -INFINITY;
  if (scale_log2 > 0.f) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
    mx = fmaxf(mx, shfl_xor(mx, 32)) * scale_log2;
  } else {
    // zero or negative scale: scale first, then mask-preserving max
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sc[kb][r] = sc[kb][r] == -INFINITY ? -INFINITY : sc[kb][r] * scale_log2;
        mx = fmaxf(mx, sc[kb][r]);
      }
    mx = fmaxf(mx, shfl_xor(mx, 32));
  }
  // The reference point st.m of the weights moves only when a row's tile
  // maximum exceeds it by more than kSlack, so weights stay below 2^kSlack
  // and the O^T accumulators are rescaled only on such (rare) tiles.  Every
  // row's first tile holds key 0, so st.m is finite from then on.
  const bool grow = mx > st.m + kSlack;
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
    const float m_new = grow ? mx : st.m;
    const float alpha = fast_exp2(st.m - m_new);
    st.m = m_new;
    st.lsum *= alpha;
#pragma unroll
    for (int i = 0; i < DB; ++i) st.acc[i] *= alpha;
  }
  bf16x8 pb[4];
  if (scale_log2 > 0.f) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        pb[2 * kb + (r >> 3)][r & 7] = (__bf16)fast_exp2(__builtin_fmaf(sc[kb][r], scale_log2, -st.m));
  } else {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) pb[2 * kb + (r >> 3)][r & 7] = (__bf16)fast_exp2(sc[kb][r] - st.m);
  }
  // the denominator sums exactly the bf16 weights PV uses (2 per dot)
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
  float ps = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      ps = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[c][2 * e], pb[c][2 * e + 1]}, ones, ps, false);
  st.lsum += ps;

  // O^T[d, rows] += V^T[d, 16 keys] P^T[16 keys, rows], four times.  B slots
  // of pb[c]: keys 16c + 4j + (0..3) then 16c + 8 + 4j + (0..3); the V
  // operands of the next key chunk load during this chunk's MFMAs.
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (c + 1 < 4) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
        va[(c + 1) & 1][db] = tiles::read_tr<D>(vs, ln.v_rd[c + 1][db], ln.v_dx[c + 1][db]);
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
  __shared__ __align__(16) __bf16 v0s[TILE];
  __shared__ __align__(16) __bf16 k1s[TILE];
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
  const int w = tid >> 6;
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
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) ln.k_rd[kb][kk] = tiles::row_offset<D>(32 * kb + row, 2 * kk + j);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int db = 0; db < DB; ++db) tiles::tr_offsets<D>(lane, c, db, ln.v_rd[c][db], ln.v_dx[c][db]);
  }

  // K/V of this (sequence, KV head); rows >= n read as zeros.
  const size_t kv_off = ((size_t)b * hkv + kvh) * (size_t)n * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + kv_off, n * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + kv_off, n * D * 2);
  const tiles::TileFill<D> fill(tid);

  RowState<D> st;
  st.m = -INFINITY;
  st.lsum = 0.f;
#pragma unroll
  for (int i = 0; i < DB; ++i) st.acc[i] = f32x16{};

  const int kv_hi = min(n, q0 + mq);       // keys any row of the workgroup needs
  const int wave_hi = min(n, pos0 + 32);   // keys this wavefront needs
  const int ntiles = (kv_hi + kBN - 1) / kBN;

  fill.issue2(k0s, rk, v0s, rv, w, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < ntiles; it += 2) {
    // stage 0 holds tile it
    if (it + 1 < ntiles) fill.issue2(k1s, rk, v1s, rv, w, (it + 1) * kBN);
    if (it * kBN < wave_hi) attend_tile<D>(k0s, v0s, ln, st, it * kBN, pos0, pos, n, j, scale_log2);
    __builtin_amdgcn_s_waitcnt(0);   // this thread's loads of the next tile have landed
    __syncthreads();                 // ... everyone's, and everyone is done with stage 0
    if (it + 1 >= ntiles) break;
    // stage 1 holds tile it + 1
    if (it + 2 < ntiles) fill.issue2(k0s, rk, v0s, rv, w, (it + 2) * kBN);
    if ((it + 1) * kBN < wave_hi)
      attend_tile<D>(k1s, v1s, ln, st, (it + 1) * kBN, pos0, pos, n, j, scale_log2);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
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
    if (lse != nullptr && j == 0) lse[((size_t)b * hq + head) * n + pos] = (st.m + __log2f(lsum)) * kLn2;
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
