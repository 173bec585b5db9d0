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
// largest dividing g).  Each K/V tile is loaded into LDS once and used by all
// Gw heads.  Wavefront w owns 32 rows (one head, 32 positions) and keeps:
//   Q^T      as MFMA B operands in registers (loaded once),
//   S^T      [32 keys, 32 rows] = K Q^T in registers,
//   O^T      [d, 32 rows] fp32 accumulators, rescaled by the online softmax.
// K tiles feed the A operand with plain 16-byte LDS reads; V tiles feed the
// A operand of O^T += V^T P^T through the transposing ds_read_b64_tr_b16.
// Key tiles strictly above a wavefront's diagonal are skipped, and the mask
// is applied only where a tile crosses it.  Workgroups are issued
// heaviest-first and, when the (sequence, KV head) count allows, all
// q-tiles of one KV head land on the same XCD so its K/V stays in one L2.

#include "gqa_device.hpp"
#include "gqa_launch.hpp"

namespace gqa {

namespace {

constexpr int kRows = 128;   // query rows per workgroup
constexpr int kBN = 32;      // keys per tile
constexpr int kXcds = 8;

template <int D>
__global__ __launch_bounds__(256)
void prefill_causal_bf16(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                         const __bf16* __restrict__ v, float* __restrict__ out,
                         float* __restrict__ lse, int hq, int hkv, int n, int g, int gw,
                         int n_qtiles, int units, float scale_log2) {
  constexpr int KSTEPS = D / 16;   // MFMA steps over the head dim for QK^T
  constexpr int DB = D / 32;       // O^T row blocks
  constexpr int PITCH = D + 8;     // bf16 elements per LDS row (16-byte pad)
  constexpr int CPR = D / 8;       // 16-byte chunks per row
  __shared__ __align__(16) __bf16 ks[kBN * PITCH];
  __shared__ __align__(16) __bf16 vs[kBN * PITCH];

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

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int row = lane & 31;   // query row within the wave (B/D column)
  const int j = lane >> 5;     // contraction group
  const int head = kvh * g + hb * gw + (32 * w) / mq;
  const int pos0 = q0 + (32 * w) % mq;
  const int pos = pos0 + row;

  bf16x8 qb[KSTEPS];
  {
    const __bf16* qrow = q + (((size_t)b * hq + head) * n + min(pos, n - 1)) * D;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) qb[kk] = load_bf16x8(qrow + 16 * kk + 8 * j);
  }

  float m = -INFINITY, lsum = 0.f;
  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};

  const size_t kv_off = ((size_t)b * hkv + kvh) * (size_t)n * D;
  const int kv_hi = min(n, q0 + mq);       // keys any row of the workgroup needs
  const int wave_hi = min(n, pos0 + 32);   // keys this wavefront needs

  for (int t0 = 0; t0 < kv_hi; t0 += kBN) {
    __syncthreads();
    for (int i = threadIdx.x; i < kBN * CPR; i += 256) {
      const int r = i / CPR, c = i - (i / CPR) * CPR;
      const size_t src = kv_off + (size_t)min(t0 + r, n - 1) * D + 8 * c;
      store_bf16x8(ks + r * PITCH + 8 * c, load_bf16x8(k + src));
      store_bf16x8(vs + r * PITCH + 8 * c, load_bf16x8(v + src));
    }
    __syncthreads();
    if (t0 >= wave_hi) continue;   // whole tile above this wave's diagonal

    f32x16 sc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
      sc = mfma32(load_bf16x8(ks + row * PITCH + 16 * kk + 8 * j), qb[kk], sc);
    // sc[r] = score of key t0 + 8*(r/4) + 4*j + r%4 for query row `row`.
    const bool diag = t0 + kBN > pos0 || t0 + kBN > n;
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = sc[r] * scale_log2;
      if (diag) {
        const int t = t0 + 8 * (r >> 2) + 4 * j + (r & 3);
        if (t > pos || t >= n) s = -INFINITY;
      }
      sc[r] = s;
      mx = fmaxf(mx, s);
    }
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);   // finite: key 0 is in every row's first tile
    const float alpha = fast_exp2(m - m_new);
    bf16x8 pb[2];
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const __bf16 p = (__bf16)fast_exp2(sc[r] - m_new);
      pb[r >> 3][r & 7] = p;
      ps += (float)p;
    }
    lsum = lsum * alpha + ps;
    m = m_new;
#pragma unroll
    for (int i = 0; i < DB; ++i) acc[i] *= alpha;

    // O^T[d, rows] += V^T[d, 16 keys] P^T[16 keys, rows] twice.  B slots of
    // pb[q2]: keys 16*q2 + 4*j + (0..3) then 16*q2 + 8 + 4*j + (0..3).
    const int L = lane & 15;
    const int dlo = 16 * ((lane >> 4) & 1);   // which 16 of the 32 A rows
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const __bf16* base = vs + (16 * q2 + 4 * j + (L >> 2)) * PITCH + 32 * db + dlo + 4 * (L & 3);
        const bf16x8 va = concat(lds_read_tr16(base), lds_read_tr16(base + 8 * PITCH));
        acc[db] = mfma32(va, pb[q2], acc[db]);
      }
    }
  }

  lsum += shfl_xor(lsum, 32);
  if (pos < n) {
    const float inv = 1.f / lsum;
    float* orow = out + (((size_t)b * hq + head) * n + pos) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 o4;
#pragma unroll
        for (int r = 0; r < 4; ++r) o4[r] = acc[db][4 * r4 + r] * inv;
        *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * r4 + 4 * j) = o4;
      }
    if (lse != nullptr && j == 0) lse[((size_t)b * hq + head) * n + pos] = (m + __log2f(lsum)) * kLn2;
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
    hipLaunchKernelGGL(prefill_causal_bf16<128>, grid, dim3(256), 0, stream, qp, kp, vp, out, lse,
                       s.hq, s.hkv, s.n, g, gw, n_qtiles, units, sl2);
  else
    hipLaunchKernelGGL(prefill_causal_bf16<64>, grid, dim3(256), 0, stream, qp, kp, vp, out, lse,
                       s.hq, s.hkv, s.n, g, gw, n_qtiles, units, sl2);
  return hipGetLastError();
}

}  // namespace gqa
