// Causal GQA prefill backward on gfx950 bf16 matrix cores.
//
// Gradients of out_h = softmax(scale Q_h K^T, causal) V for every query head
// h, with K and V shared by the g consecutive query heads of a group: a
// shared K or V row collects gradient from every query head of its group
// (study.greatitself.com, "Grouped-Query and Multi-Query Attention", section
// "Share keys and values without confusing query-head identity", training
// paragraph).  P is recomputed tile by tile from the forward's log-sum-exp,
// P = exp(scale q.k - lse), and with the row term D_i = rowsum(dO_i * O_i)
// (equal to rowsum(P_i * dP_i), the correction of the softmax Jacobian):
//
//   dV[kv] = sum over the group's heads of P^T dO
//   dS     = P * (dO V^T - D)
//   dQ     = scale dS K
//   dK[kv] = scale * sum over the group's heads of dS^T Q
//
// Two kernels, no atomics, bitwise deterministic:
//  * prefill_bwd_dq: a workgroup owns 128 query rows of one KV head's group
//    (the forward's partition: Gw heads x 128/Gw positions), streams the K/V
//    tiles of keys up to its diagonal through LDS and accumulates dQ^T in
//    registers.  Its prologue forms D for its rows from out and dO and
//    stores it, with lse in the log2 domain, for the second kernel.
//  * prefill_bwd_dkdv: a workgroup owns two 128-key tiles of one KV head,
//    p and the mirror tile from the end (32 keys per wavefront, with K and
//    V held in registers as MFMA operands), one after the other.  For each
//    it streams, through double-buffered LDS, the Q/dO tiles of every query
//    head of the group at every position from the tile's first key on.  dK
//    and dV of the KV head are summed over the g heads in registers:
//    per-head gradients never reach memory and the shared K/V rows are
//    never copied.  The two tiles of a pair cover the same number of Q
//    tiles whatever p, so one round of equal workgroups (one per CU, at
//    512 registers per lane) covers the sequence; the first tile is swept
//    from the last Q tile down and the second from its diagonal up, so all
//    workgroups of one KV head, placed on one XCD when the KV-head count
//    allows, read the same one or two Q tiles at any time and share them
//    in L2.
//
// Layouts: q, dout, out [B, Hq, N, d]; k, v [B, Hkv, N, d]; lse [B, Hq, N];
// row_terms [2][B, Hq, N] (lse * log2 e, then D); dq [B, Hq, N, d]; dk, dv
// [B, Hkv, N, d].  MFMA operand
// layouts are the ones listed in gqa_device.hpp; LDS tiles are those of
// prefill_tiles.hpp.

#include <type_traits>

#include "gqa_device.hpp"
#include "gqa_launch.hpp"
#include "prefill_tiles.hpp"

namespace gqa {

namespace {

constexpr int kThreads = tiles::kThreads;
constexpr int kTile = tiles::kRows;   // rows per LDS tile (keys, or query positions)
constexpr int kDqRows = 128;          // query rows per dQ workgroup
constexpr int kKeys = 128;            // keys per dK/dV workgroup (32 per wavefront)
constexpr int kXcds = 8;

// Workgroup -> (unit, tile) with the tile holding the most work first and,
// when units divide evenly, all tiles of a unit on one XCD (workgroup w runs
// on XCD w % 8).
__device__ __forceinline__ void unit_and_tile(int wg, int units, int& unit, int& slot_tile) {
  if (units % kXcds == 0) {
    const int xcd = wg % kXcds, slot = wg / kXcds, per = units / kXcds;
    unit = xcd * per + slot % per;
    slot_tile = slot / per;
  } else {
    unit = wg % units;
    slot_tile = wg / units;
  }
}

// ---------------------------------------------------------------------------
// dQ (and D)
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_bwd_dq(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                    const __bf16* __restrict__ v, const float* __restrict__ out,
                    const float* __restrict__ lse, const __bf16* __restrict__ dout,
                    float* __restrict__ dq, float* __restrict__ row_terms, size_t rows, int hq, int hkv,
                    int n, int g, int gw, int n_qtiles, int units, float scale_log2, float scale) {
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = kTile * D;
  __shared__ __align__(16) __bf16 k0s[TILE];
  __shared__ __align__(16) __bf16 v0s[TILE];
  __shared__ __align__(16) __bf16 k1s[TILE];
  __shared__ __align__(16) __bf16 v1s[TILE];

  int unit, back;
  unit_and_tile(blockIdx.x, units, unit, back);
  const int qt = n_qtiles - 1 - back;
  const int nhb = g / gw;
  const int b = unit / (hkv * nhb);
  const int rem = unit - b * hkv * nhb;
  const int kvh = rem / nhb;
  const int hb = rem - kvh * nhb;
  const int mq = kDqRows / gw;
  const int q0 = qt * mq;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int row = lane & 31;   // query row within the wave (B/D column)
  const int j = lane >> 5;     // contraction group
  const int head = kvh * g + hb * gw + (32 * w) / mq;
  const int pos0 = q0 + (32 * w) % mq;
  const int pos = pos0 + row;
  const size_t row_idx = ((size_t)b * hq + head) * n + min(pos, n - 1);

  // Q^T and dO^T as B operands (8 consecutive columns per contraction
  // group), and this row's D from the same dO values and out.
  bf16x8 qb[KSTEPS], ob[KSTEPS];
  float dpart = 0.f;
  {
    const __bf16* qrow = q + row_idx * D;
    const __bf16* orow = dout + row_idx * D;
    const float* frow = out + row_idx * D;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      qb[kk] = load_bf16x8(qrow + 16 * kk + 8 * j);
      ob[kk] = load_bf16x8(orow + 16 * kk + 8 * j);
      const f32x4 f0 = *reinterpret_cast<const f32x4*>(frow + 16 * kk + 8 * j);
      const f32x4 f1 = *reinterpret_cast<const f32x4*>(frow + 16 * kk + 8 * j + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dpart = __builtin_fmaf((float)ob[kk][e], f0[e], dpart);
        dpart = __builtin_fmaf((float)ob[kk][4 + e], f1[e], dpart);
      }
    }
  }
  const float drow = dpart + shfl_xor(dpart, 32);
  const float lse2 = lse[row_idx] * kLog2e;
  // row_terms[0] = lse * log2(e), row_terms[1] = D, each [B, Hq, N]
  if (pos < n) row_terms[(size_t)j * rows + row_idx] = j == 0 ? lse2 : drow;

  // LDS operand offsets.  The tile swizzle repeats every 16 rows, so key
  // block kb (32 rows) and 16-key chunk c are the constant offsets 32 kb D
  // and 16 c D from the offsets kept here.
  int a_rd[KSTEPS];            // K / V rows: key row (of block 0), chunk 2 kk + j
  int t_rd[DB], t_dx[DB];      // K^T: keys of 16-key chunk 0, columns of block db
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    a_rd[kk] = tiles::row_offset<D>(row, 2 * kk + j);
    asm volatile("" : "+v"(a_rd[kk]));
  }
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    tiles::tr_offsets<D>(lane, 0, db, t_rd[db], t_dx[db]);
    asm volatile("" : "+v"(t_rd[db]));
  }

  const size_t kv_off = ((size_t)b * hkv + kvh) * (size_t)n * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + kv_off, n * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + kv_off, n * D * 2);
  const tiles::TileFill<D> fill(tid);

  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};

  const int lim = min(pos, n - 1);           // last key this row sees
  const int wave_hi = min(n, pos0 + 32);     // keys this wavefront needs
  const int ntiles = (min(n, q0 + mq) + kTile - 1) / kTile;

  // dS of element r of block kb (P recomputed from lse) into its B-operand
  // slot: element r of block kb is key t0 + 32 kb + 8 (r/4) + 4 j + r%4.
  auto grad = [&](const f32x16 (&sc)[2], const f32x16 (&dp)[2], bf16x8 (&dsb)[4], int kb, int r) {
    float ds = fast_exp2(__builtin_fmaf(sc[kb][r], scale_log2, -lse2)) * (dp[kb][r] - drow);
    asm volatile("" : "+v"(ds));   // keeps it in its group (not sunk to its use)
    dsb[2 * kb + (r >> 3)][r & 7] = (__bf16)ds;
  };

  // A tile that crosses the diagonal (or the end): the keys past each row
  // get P = 0.  The products run one after the other.
  auto tile_edge = [&](const __bf16* ks, const __bf16* vs, int t0) {
    // S^T and dP^T [64 keys, 32 rows] = K Q^T and V dO^T
    f32x16 sc[2] = {f32x16{}, f32x16{}};
    f32x16 dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sc[kb] = mfma32(load_bf16x8(ks + a_rd[kk] + 32 * kb * D), qb[kk], sc[kb]);
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) dp[kb] = mfma32(load_bf16x8(vs + a_rd[kk] + 32 * kb * D), ob[kk], dp[kb]);
    bf16x8 dsb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(__builtin_fmaf(sc[kb][r], scale_log2, -lse2));
        const int t = t0 + 32 * kb + 8 * (r >> 2) + 4 * j + (r & 3);
        p = t <= lim ? p : 0.f;
        dsb[2 * kb + (r >> 3)][r & 7] = (__bf16)(p * (dp[kb][r] - drow));
      }
    // dQ^T [d, rows] += K^T [d, 16 keys] dS^T [16 keys, rows]
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        acc[db] = mfma32(tiles::read_tr<D>(ks + 16 * c * D, t_rd[db], t_dx[db]), dsb[c], acc[db]);
  };

  // A tile below the diagonal: the same arithmetic, with the dS of each key
  // block computed between independent MFMAs of this wavefront, in groups
  // fenced by scheduling barriers: dS of block 0 while the S^T and dP^T
  // products of block 1 run, the first half of block 1's dS while the dQ^T
  // products of block 0's dS run, and its second half beside those of the
  // first half.  The products accumulate in the same order as in tile_edge.
  auto tile_inner = [&](const __bf16* ks, const __bf16* vs) {
    constexpr int kPerB = 8 / KSTEPS;   // dS elements per S^T / dP^T product of block 1
    constexpr int kPerC = 4 / DB;       // ... per dQ^T product of chunks 0 and 1
    constexpr int kPerD = 8 / DB;       // ... per dQ^T product of chunk 2
    f32x16 sc[2] = {f32x16{}, f32x16{}};
    f32x16 dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) sc[0] = mfma32(load_bf16x8(ks + a_rd[kk]), qb[kk], sc[0]);
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) dp[0] = mfma32(load_bf16x8(vs + a_rd[kk]), ob[kk], dp[0]);
    bf16x8 dsb[4];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 2 * KSTEPS; ++i) {   // S^T of block 1, then its dP^T
      const int kk = i % KSTEPS;
      if (i < KSTEPS)
        sc[1] = mfma32(load_bf16x8(ks + a_rd[kk] + 32 * D), qb[kk], sc[1]);
      else
        dp[1] = mfma32(load_bf16x8(vs + a_rd[kk] + 32 * D), ob[kk], dp[1]);
#pragma unroll
      for (int r = i * kPerB; r < (i + 1) * kPerB; ++r) grad(sc, dp, dsb, 0, r);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < 4 * DB; ++i) {   // product i: key chunk i / DB, column block i % DB
      acc[i % DB] = mfma32(tiles::read_tr<D>(ks + 16 * (i / DB) * D, t_rd[i % DB], t_dx[i % DB]), dsb[i / DB],
                           acc[i % DB]);
      if (i < 2 * DB) {
#pragma unroll
        for (int r = i * kPerC; r < (i + 1) * kPerC; ++r) grad(sc, dp, dsb, 1, r);
      } else if (i < 3 * DB) {
#pragma unroll
        for (int r = 8 + (i - 2 * DB) * kPerD; r < 8 + (i - 2 * DB + 1) * kPerD; ++r) grad(sc, dp, dsb, 1, r);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto tile = [&](const __bf16* ks, const __bf16* vs, int t0) {
    if (t0 + kTile > pos0 || t0 + kTile > n)
      tile_edge(ks, vs, t0);
    else
      tile_inner(ks, vs);
  };

  fill.issue2(k0s, rk, v0s, rv, w, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < ntiles; it += 2) {
    if (it + 1 < ntiles) fill.issue2(k1s, rk, v1s, rv, w, (it + 1) * kTile);
    if (it * kTile < wave_hi) tile(k0s, v0s, it * kTile);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (it + 1 >= ntiles) break;
    if (it + 2 < ntiles) fill.issue2(k0s, rk, v0s, rv, w, (it + 2) * kTile);
    if ((it + 1) * kTile < wave_hi) tile(k1s, v1s, (it + 1) * kTile);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if (pos < n) {
    float* drow_out = dq + row_idx * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 o4;
#pragma unroll
        for (int r = 0; r < 4; ++r) o4[r] = acc[db][4 * r4 + r] * scale;
        *reinterpret_cast<f32x4*>(drow_out + 32 * db + 8 * r4 + 4 * j) = o4;
      }
  }
}

// ---------------------------------------------------------------------------
// dK, dV (summed over the group's query heads)
// ---------------------------------------------------------------------------

// Start the loads of query rows row0 .. row0+63 of one head: its q and dout
// rows into LDS tiles, and (waves 0 and 1 only) 64 floats of `scalars`
// (lse or D) into rs[64 w ..].  A plain function rather than a lambda: the
// host pass cannot form buffer resources, and a kernel whose lambda builds
// one silently loses its host launch stub.
template <int D>
__device__ __forceinline__ void issue_rows(const tiles::TileFill<D>& fill, const __bf16* qh,
                                           const __bf16* oh, const float* scalars, __bf16* qs, __bf16* os,
                                           float* rs, int n, int w, int row0) {
  fill.issue2(qs, make_rsrc(qh, n * D * 2), os, make_rsrc(oh, n * D * 2), w, row0);
  if (w < 2) {
    // the lane index is recomputed here rather than kept live across the
    // step (under the step's register pressure it would be spilled)
    int lane;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
    tiles::load_floats_lds(rs + w * kTile, make_rsrc(scalars, n * 4), (row0 + lane) * 4);
  }
}

// P^T and dS^T of one 32-row block as bf16 A operands (lane = key, k-group
// j = rows 16 c + 4 j + 0..3 and 16 c + 8 + 4 j + 0..3 for chunk c), from
// S and dP (element r: row 8 (r/4) + 4 j + r%4 of the block).  With MASK,
// `rel` is the lane's key minus the block's first row: rows before the key
// get P = 0.
template <bool MASK>
__device__ __forceinline__ void softmax_grad_block(const f32x16& sc, const f32x16& dp, const float* rs_lse,
                                                   const float* rs_d, float scale_log2, int j, int rel,
                                                   bf16x8 (&pa)[2], bf16x8 (&da)[2]) {
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const f32x4 l4 = *reinterpret_cast<const f32x4*>(rs_lse + 8 * r4 + 4 * j);
    const f32x4 d4 = *reinterpret_cast<const f32x4*>(rs_d + 8 * r4 + 4 * j);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * r4 + e;
      float p = fast_exp2(__builtin_fmaf(sc[r], scale_log2, -l4[e]));
      if (MASK) p = (8 * r4 + 4 * j + e >= rel) ? p : 0.f;
      pa[r >> 3][r & 7] = (__bf16)p;
      da[r >> 3][r & 7] = (__bf16)(p * (dp[r] - d4[e]));
    }
  }
}

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x2;
constexpr int kSchedMfma = 0x8;
constexpr int kSchedDsRead = 0x100;

// Transposed LDS operands of 16-row chunk c: dO^T and Q^T for all column blocks.
template <int D>
__device__ __forceinline__ void read_chunk_tr(const __bf16* qs, const __bf16* os, const int (&t_rd)[4][D / 32],
                                              const int (&t_dx)[4][D / 32], int c, bf16x8 (&ot)[D / 32],
                                              bf16x8 (&qt)[D / 32]) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    ot[db] = tiles::read_tr<D>(os, t_rd[c][db], t_dx[c][db]);
    qt[db] = tiles::read_tr<D>(qs, t_rd[c][db], t_dx[c][db]);
  }
}

// One 64-row Q/dO tile against the wavefront's 32 keys: S and dP for the
// two 32-row blocks, then dV += P^T dO and dK += dS^T Q chunk by chunk.
// With one wavefront per SIMD nothing else hides LDS latency, so the code is
// software-pipelined by hand: the LDS operands of each group of MFMAs are
// read while the previous group runs, and the softmax arithmetic of a block
// is interleaved with MFMAs that do not depend on it.
template <int D, bool MASK>
__device__ __forceinline__ void dkdv_step(const __bf16* qs, const __bf16* os, const float* rs,
                                          const bf16x8 (&kb)[D / 16], const bf16x8 (&vb)[D / 16],
                                          const int (&a_rd)[2][D / 16], const int (&t_rd)[4][D / 32],
                                          const int (&t_dx)[4][D / 32], f32x16 (&dka)[D / 32],
                                          f32x16 (&dva)[D / 32], float scale_log2, int j, int rel) {
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  f32x16 sc0 = f32x16{}, dp0 = f32x16{}, sc1 = f32x16{}, dp1 = f32x16{};
  bf16x8 qa[KSTEPS], oa[KSTEPS], qa1[KSTEPS], oa1[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    qa[kk] = load_bf16x8(qs + a_rd[0][kk]);
    oa[kk] = load_bf16x8(os + a_rd[0][kk]);
  }
  __builtin_amdgcn_sched_barrier(0);
  // S, dP of rows 0..31; the row operands of rows 32..63 load meanwhile.
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    sc0 = mfma32(qa[kk], kb[kk], sc0);
    dp0 = mfma32(oa[kk], vb[kk], dp0);
  }
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    qa1[kk] = load_bf16x8(qs + a_rd[1][kk]);
    oa1[kk] = load_bf16x8(os + a_rd[1][kk]);
  }
#pragma unroll
  for (int i = 0; i < KSTEPS; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  // S, dP of rows 32..63; the transposed operands of chunk 0 load meanwhile.
  bf16x8 ot[2][DB], qt[2][DB];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    sc1 = mfma32(qa1[kk], kb[kk], sc1);
    dp1 = mfma32(oa1[kk], vb[kk], dp1);
  }
  read_chunk_tr<D>(qs, os, t_rd, t_dx, 0, ot[0], qt[0]);
#pragma unroll
  for (int i = 0; i < 2 * KSTEPS; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 1);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 1);
  }
  __builtin_amdgcn_sched_barrier(0);
  bf16x8 pa0[2], da0[2], pa1[2], da1[2];
  softmax_grad_block<MASK>(sc0, dp0, rs, rs + kTile, scale_log2, j, rel, pa0, da0);
  __builtin_amdgcn_sched_barrier(0);
  // Chunks 0 and 1 (rows 0..31) while the operands of the next chunk load;
  // the softmax of rows 32..63 is spread over chunk 1's MFMAs.
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dva[db] = mfma32(pa0[0], ot[0][db], dva[db]);
    dka[db] = mfma32(da0[0], qt[0][db], dka[db]);
  }
  read_chunk_tr<D>(qs, os, t_rd, t_dx, 1, ot[1], qt[1]);
#pragma unroll
  for (int i = 0; i < 2 * DB; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 2);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 2);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dva[db] = mfma32(pa0[1], ot[1][db], dva[db]);
    dka[db] = mfma32(da0[1], qt[1][db], dka[db]);
  }
  read_chunk_tr<D>(qs, os, t_rd, t_dx, 2, ot[0], qt[0]);
  softmax_grad_block<MASK>(sc1, dp1, rs + 32, rs + kTile + 32, scale_log2, j, rel - 32, pa1, da1);
#pragma unroll
  for (int i = 0; i < 2 * DB; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 3);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 3);
    __builtin_amdgcn_sched_group_barrier(kSchedValu, 12, 3);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dva[db] = mfma32(pa1[0], ot[0][db], dva[db]);
    dka[db] = mfma32(da1[0], qt[0][db], dka[db]);
  }
  read_chunk_tr<D>(qs, os, t_rd, t_dx, 3, ot[1], qt[1]);
#pragma unroll
  for (int i = 0; i < 2 * DB; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 4);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 4);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dva[db] = mfma32(pa1[1], ot[1][db], dva[db]);
    dka[db] = mfma32(da1[1], qt[1][db], dka[db]);
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1)))
void prefill_bwd_dkdv(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                      const __bf16* __restrict__ v, const __bf16* __restrict__ dout,
                      const float* __restrict__ row_terms, size_t rows, float* __restrict__ dk,
                      float* __restrict__ dv, int hq, int hkv, int n, int g, int units, float scale_log2,
                      float scale) {
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = kTile * D;
  __shared__ __align__(16) __bf16 q0s[TILE];
  __shared__ __align__(16) __bf16 o0s[TILE];
  __shared__ __align__(16) __bf16 q1s[TILE];
  __shared__ __align__(16) __bf16 o1s[TILE];
  __shared__ __align__(16) float r0s[2 * kTile];   // lse, then D, of the stage's rows
  __shared__ __align__(16) float r1s[2 * kTile];

  int unit, pair;
  unit_and_tile(blockIdx.x, units, unit, pair);
  const int b = unit / hkv;
  const int kvh = unit - b * hkv;
  const int n_ktiles = (n + kKeys - 1) / kKeys;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;   // this lane's key within the wave (A row / D row index)
  const int j = lane >> 5;     // contraction group

  // K and V rows of key kw + col as B operands of S = Q K^T and dP = dO V^T.
  const size_t kv_off = ((size_t)b * hkv + kvh) * (size_t)n * D;
  bf16x8 kb[KSTEPS], vb[KSTEPS];
  auto load_kv = [&](int kw) {
    const int key = kw + col;
    const __bf16* krow = k + kv_off + (size_t)min(key, n - 1) * D;
    const __bf16* vrow = v + kv_off + (size_t)min(key, n - 1) * D;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      kb[kk] = load_bf16x8(krow + 16 * kk + 8 * j);
      vb[kk] = load_bf16x8(vrow + 16 * kk + 8 * j);
      if (key >= n) kb[kk] = vb[kk] = bf16x8{};
    }
  };

  int a_rd[2][KSTEPS];           // Q / dO rows 32 rb + col, chunk 2 kk + j
  int t_rd[4][DB], t_dx[4][DB];  // Q^T / dO^T: rows of 16-row chunk c, columns of block db
  // The swizzle depends on the row modulo 16, so the offsets of row blocks
  // 32 rb and chunks 16 c are those of block 0 plus a constant.  The empty
  // asm hides the base offsets' value range from the compiler, which then
  // adds stage and block constants through the LDS instructions' offset
  // field instead of spending a VALU op per read on an OR.
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    int base = tiles::row_offset<D>(col, 2 * kk + j);
    asm volatile("" : "+v"(base));
    a_rd[0][kk] = base;
    a_rd[1][kk] = base + 32 * D;
  }
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    int base, dx;
    tiles::tr_offsets<D>(lane, 0, db, base, dx);
    asm volatile("" : "+v"(base));
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      t_rd[c][db] = base + 16 * D * c;
      t_dx[c][db] = dx;
    }
  }

  f32x16 dka[DB], dva[DB];
  const int qt_last = (n - 1) / kTile;
  const tiles::TileFill<D> fill(tid);

  // Loads of step s of a sweep into one stage: the Q and dO tiles of q-tile
  // qt, and one float per lane from waves 0 (lse) and 1 (D), zeros past n.
  auto issue = [&](int s, int qt, __bf16* qs, __bf16* os, float* rs) {
    const size_t hrow = ((size_t)b * hq + kvh * g + s % g) * n;
    issue_rows<D>(fill, q + hrow * D, dout + hrow * D, row_terms + (w == 1 ? rows : 0) + hrow, qs, os, rs, n, w,
                  qt * kTile);
  };
  auto sync = [&]() {
    __builtin_amdgcn_s_waitcnt(0);   // this thread's loads of the next step have landed
    __syncthreads();                 // ... everyone's, and everyone is done with the current stage
  };
  float* dk_b = dk + kv_off;
  float* dv_b = dv + kv_off;

  // One key tile: the q-tiles from the one holding its first key to the
  // last, each for the g query heads of the group, visited downward
  // (UP false) or upward.  Only the two q-tiles at the diagonal (2 g steps:
  // the last of a downward sweep, the first of an upward one) reach below a
  // key of the workgroup and need the causal mask; every other step runs the
  // mask-free body, in a loop of its own so that the accumulators never
  // cross a branch.  Rows past n need no mask either: their q, dout, lse and
  // D arrive as zeros, so their P = 1 meets zero dout and zero dS.  Stage 0
  // holds even steps, stage 1 odd ones.
  auto sweep = [&](int kt, auto upward) {
    constexpr bool UP = decltype(upward)::value;
    const int kw = kt * kKeys + 32 * w;   // the wave's first key
    const int qt_first = kt * kKeys / kTile;
    const int nsteps = (qt_last - qt_first + 1) * g;
    auto qt_of = [&](int s) { return UP ? qt_first + s / g : qt_last - s / g; };
    auto plain = [&](const __bf16* qs, const __bf16* os, const float* rs) {
      dkdv_step<D, false>(qs, os, rs, kb, vb, a_rd, t_rd, t_dx, dka, dva, scale_log2, j, 0);
    };
    auto masked = [&](int s, const __bf16* qs, const __bf16* os, const float* rs) {
      const int i0 = qt_of(s) * kTile;
      if (i0 + kTile - 1 < kw) return;   // every row of the tile precedes the wave's keys
      dkdv_step<D, true>(qs, os, rs, kb, vb, a_rd, t_rd, t_dx, dka, dva, scale_log2, j, kw + col - i0);
    };
    auto masked_steps = [&](int& s, int end) {
      for (; s < end; ++s) {
        if (s & 1) {
          if (s + 1 < nsteps) issue(s + 1, qt_of(s + 1), q0s, o0s, r0s);
          masked(s, q1s, o1s, r1s);
        } else {
          if (s + 1 < nsteps) issue(s + 1, qt_of(s + 1), q1s, o1s, r1s);
          masked(s, q0s, o0s, r0s);
        }
        sync();
      }
    };
    // the same for an even s on entry and an even count, two steps per trip
    auto masked_pairs = [&](int& s, int end) {
      for (; s + 1 < end; s += 2) {
        issue(s + 1, qt_of(s + 1), q1s, o1s, r1s);
        masked(s, q0s, o0s, r0s);
        sync();
        if (s + 2 < nsteps) issue(s + 2, qt_of(s + 2), q0s, o0s, r0s);
        masked(s + 1, q1s, o1s, r1s);
        sync();
      }
    };
    // plain steps s .. end - 1, s even on entry
    auto plain_steps = [&](int& s, int end) {
      for (; s + 1 < end; s += 2) {
        issue(s + 1, qt_of(s + 1), q1s, o1s, r1s);
        plain(q0s, o0s, r0s);
        sync();
        if (s + 2 < nsteps) issue(s + 2, qt_of(s + 2), q0s, o0s, r0s);
        plain(q1s, o1s, r1s);
        sync();
      }
      if (s < end) {
        if (s + 1 < nsteps) issue(s + 1, qt_of(s + 1), q1s, o1s, r1s);
        plain(q0s, o0s, r0s);
        sync();
        ++s;
      }
    };

    __builtin_amdgcn_sched_barrier(0);   // the previous sweep's stores go first
    issue(0, qt_of(0), q0s, o0s, r0s);
    load_kv(kw);
#pragma unroll
    for (int i = 0; i < DB; ++i) dka[i] = dva[i] = f32x16{};
    sync();
    const int n_mask = min(nsteps, 2 * g);   // even whenever plain steps follow it
    int s = 0;
    if (UP) {
      masked_pairs(s, n_mask);
      if (s < n_mask) {   // an odd count: the sweep's one q-tile with g odd, s even here
        if (s + 1 < nsteps) issue(s + 1, qt_of(s + 1), q1s, o1s, r1s);
        masked(s, q0s, o0s, r0s);
        sync();
        ++s;
      }
      plain_steps(s, nsteps);
    } else {
      plain_steps(s, nsteps - n_mask);
      masked_steps(s, nsteps);
    }

    // D rows of dK/dV: key kw + 8 (r/4) + 4 j + r%4, column 32 db + col.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kw + 8 * (r >> 2) + 4 * j + (r & 3);
      if (key < n) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dk_b[(size_t)key * D + 32 * db + col] = dka[db][r] * scale;
          dv_b[(size_t)key * D + 32 * db + col] = dva[db][r];
        }
      }
    }
  };

  // A workgroup owns key tiles `pair` and n_ktiles - 1 - `pair`, whose sweeps
  // hold n_ktiles + 1 q-tiles between them whatever the pair (for 128-key
  // tiles and 64-row q-tiles), so one round of workgroups covers the
  // sequence with equal work each.  The first sweep runs downward from the
  // last q-tile and the second upward from its diagonal: every down-sweep
  // reads q-tile qt_last - t at its t-th q-tile and every up-sweep, which
  // starts as its workgroup's down-sweep ends, reads q-tile t - 2 then, so
  // the workgroups of one KV head read the same one or two q-tiles at a time
  // and share them in L2.
  sweep(pair, std::integral_constant<bool, false>{});
  const int kt2 = n_ktiles - 1 - pair;
  if (kt2 > pair) sweep(kt2, std::integral_constant<bool, true>{});
}

}  // namespace

hipError_t launch_prefill_backward(const void* q, const void* k, const void* v, const float* out,
                                   const float* lse, const void* dout, float* dq, float* dk, float* dv,
                                   float* row_terms, const PrefillShape& s, hipStream_t stream) {
  const int g = s.hq / s.hkv;
  const int gw = (g % 4 == 0) ? 4 : (g % 2 == 0 ? 2 : 1);
  const int mq = kDqRows / gw;
  const int n_qtiles = (s.n + mq - 1) / mq;
  const int dq_units = s.batch * s.hkv * (g / gw);
  const int kv_units = s.batch * s.hkv;
  const int n_ktiles = (s.n + kKeys - 1) / kKeys;
  const int n_pairs = (n_ktiles + 1) / 2;   // key tiles p and n_ktiles - 1 - p per workgroup
  const size_t rows = (size_t)s.batch * s.hq * s.n;
  const float sl2 = s.scale * kLog2e;
  auto qp = static_cast<const __bf16*>(q);
  auto kp = static_cast<const __bf16*>(k);
  auto vp = static_cast<const __bf16*>(v);
  auto op = static_cast<const __bf16*>(dout);
  const dim3 block(kThreads);
  const dim3 grid_dq((unsigned)dq_units * (unsigned)n_qtiles);
  const dim3 grid_kv((unsigned)kv_units * (unsigned)n_pairs);
  if (s.d == 128) {
    hipLaunchKernelGGL(prefill_bwd_dq<128>, grid_dq, block, 0, stream, qp, kp, vp, out, lse, op, dq, row_terms,
                       rows, s.hq, s.hkv, s.n, g, gw, n_qtiles, dq_units, sl2, s.scale);
    hipLaunchKernelGGL(prefill_bwd_dkdv<128>, grid_kv, block, 0, stream, qp, kp, vp, op, row_terms, rows, dk,
                       dv, s.hq, s.hkv, s.n, g, kv_units, sl2, s.scale);
  } else {
    hipLaunchKernelGGL(prefill_bwd_dq<64>, grid_dq, block, 0, stream, qp, kp, vp, out, lse, op, dq, row_terms,
                       rows, s.hq, s.hkv, s.n, g, gw, n_qtiles, dq_units, sl2, s.scale);
    hipLaunchKernelGGL(prefill_bwd_dkdv<64>, grid_kv, block, 0, stream, qp, kp, vp, op, row_terms, rows, dk,
                       dv, s.hq, s.hkv, s.n, g, kv_units, sl2, s.scale);
  }
  return hipGetLastError();
}

}  // namespace gqa
