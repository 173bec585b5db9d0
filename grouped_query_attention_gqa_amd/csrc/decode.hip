// Split-K GQA decode for gfx950.
//
// One decode step re-reads the whole KV cache, so the kernel is bound by HBM
// bandwidth: FLOPs per cache byte equal the group size g = Hq/Hkv
// (deepconcepts.dev, "Grouped-Query Attention", section "Three numbers that
// people expect to move together"), far below the MI355X ridge point.  The
// design therefore reads every K/V element exactly once per group: a
// workgroup owns one (sequence, KV head, token chunk) and computes all g <= 16
// query heads of the group against each K/V row it loads (anrans.github.io,
// "Attention variants: MQA, GQA, MLA", section "Kernels do not need to copy
// the KV heads": the group's query heads act as extra query rows).
//
// bf16 path (one wavefront = 32 tokens per iteration):
//   S^T[32 tok, 16 heads] = K[32, d] Q^T[d, 16]      v_mfma_f32_16x16x32_bf16
//   online softmax per head (column) with wavefront shuffles, log2 domain
//   O^T[d, 16 heads]    += V^T[d, 32] P^T[32, 16]    (V^T via ds_read_b64_tr_b16)
// K goes straight from HBM into MFMA operand registers (16-byte loads of 64
// contiguous bytes per row); V goes through a per-wave LDS tile because the
// PV contraction runs over tokens, which are strided in memory.
//
// fp32 path: a plain VALU kernel (no fp32 matrix-core shape is worth it at
// d <= 128), K/V tiles staged once per workgroup in LDS, one query head per
// wavefront pass.
//
// Both write per-chunk partials (O_c normalised, lse_c in log2 units) to the
// workspace; decode_merge combines them by log-sum-exp.  Chunk c of sequence b
// covers tokens [c*chunk, min((c+1)*chunk, T_b)); empty chunks exit at once.

#include "gqa_device.hpp"
#include "gqa_launch.hpp"

namespace gqa {

namespace {

__device__ __forceinline__ int clamp_len(const int32_t* lens, int b, int tcap) {
  int t = lens[b];
  return t < 0 ? 0 : (t > tcap ? tcap : t);
}

// ---------------------------------------------------------------------------
// bf16 split kernel
// ---------------------------------------------------------------------------
template <int D>
struct DecodeBf16Smem {
  static constexpr int kPitch = D + 8;  // bf16 elements per LDS row (16-byte pad)
  static constexpr int kVTile = kDecodeWaves * kDecodeWaveTile * kPitch * 2;
  static constexpr int kComb = (2 * kDecodeWaves * kDecodeHeadBlock +
                                kDecodeWaves * kDecodeHeadBlock * (D + 4)) * 4;
  static constexpr int kBytes = kVTile > kComb ? kVTile : kComb;
};

template <int D>
__global__ __launch_bounds__(kDecodeWaves * 64)
void decode_split_bf16(const __bf16* __restrict__ q, const __bf16* __restrict__ kc,
                       const __bf16* __restrict__ vc, const int32_t* __restrict__ lens,
                       float* __restrict__ part_o, float* __restrict__ part_lse,
                       int hq, int hkv, int g, int nhb, int tcap, int chunk, int nsplit,
                       float scale_log2) {
  constexpr int KSTEPS = D / 32;          // QK^T MFMA steps over the head dim
  constexpr int DBLK = D / 16;            // PV MFMA blocks over the head dim
  constexpr int PITCH = DecodeBf16Smem<D>::kPitch;
  constexpr int LPR = D / 8;              // lanes per V row (16 B each)
  constexpr int RPI = 64 / LPR;           // V rows per wave load
  constexpr int VLOADS = kDecodeWaveTile / RPI;
  __shared__ __align__(16) char smem[DecodeBf16Smem<D>::kBytes];

  const int split = blockIdx.x;
  const int kvh = blockIdx.y / nhb;
  const int hb = blockIdx.y - kvh * nhb;
  const int b = blockIdx.z;
  const int T = clamp_len(lens, b, tcap);
  const int t_begin = split * chunk;
  if (t_begin >= T) return;
  const int t_end = min(t_begin + chunk, T);

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n = lane & 15;   // token row of A / head column of B and D
  const int j = lane >> 4;   // contraction group
  const int h_first = kvh * g + hb * kDecodeHeadBlock;
  const int nh = min(kDecodeHeadBlock, g - hb * kDecodeHeadBlock);

  // Q^T as the B operand: lane holds q[h_first+n][8j + 32kk .. +7].
  bf16x8 qb[KSTEPS];
  {
    const __bf16* qrow = q + ((size_t)b * hq + h_first + min(n, nh - 1)) * D;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      qb[kk] = load_bf16x8(qrow + 8 * j + 32 * kk);
      if (n >= nh) qb[kk] = bf16x8{};
    }
  }

  const size_t kv_off = ((size_t)b * hkv + kvh) * (size_t)tcap * D;
  const __bf16* kbase = kc + kv_off;
  const __bf16* vbase = vc + kv_off;
  __bf16* vt = reinterpret_cast<__bf16*>(smem) + w * kDecodeWaveTile * PITCH;

  float m = -INFINITY;   // running max of head n (log2 domain), same in all 4 lane groups
  float lsum = 0.f;      // this lane's share of the running denominator of head n
  f32x4 acc[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int t0 = t_begin + w * kDecodeWaveTile; t0 < t_end; t0 += kDecodeWaves * kDecodeWaveTile) {
    // K rows t0 + 16*bi + n as A operands; rows past the end re-read the
    // last valid row (its scores are masked), never the padding.
    bf16x8 ka[2][KSTEPS];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
      const int t = min(t0 + 16 * bi + n, t_end - 1);
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) ka[bi][kk] = load_bf16x8(kbase + (size_t)t * D + 8 * j + 32 * kk);
    }
    bf16x8 vr[VLOADS];
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int t = min(t0 + i * RPI + lane / LPR, t_end - 1);
      vr[i] = load_bf16x8(vbase + (size_t)t * D + 8 * (lane % LPR));
    }

    f32x4 sc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      sc[0] = mfma16(ka[0][kk], qb[kk], sc[0]);
      sc[1] = mfma16(ka[1][kk], qb[kk], sc[1]);
    }
    // sc[bi][r] = score of token t0 + 16*bi + 4*j + r for head n.
    float s2[8];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = t0 + 16 * (e >> 2) + 4 * j + (e & 3);
      s2[e] = t < t_end ? sc[e >> 2][e & 3] * scale_log2 : -INFINITY;
      mx = fmaxf(mx, s2[e]);
    }
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);       // finite: every tile holds a valid token
    const float alpha = fast_exp2(m - m_new);
    bf16x8 pb;
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const __bf16 p = (__bf16)fast_exp2(s2[e] - m_new);
      pb[e] = p;
      ps += (float)p;   // the denominator sums exactly the weights PV uses
    }
    lsum = lsum * alpha + ps;
    m = m_new;
#pragma unroll
    for (int i = 0; i < DBLK; ++i) acc[i] *= alpha;

    wave_sync();   // previous iteration's transposed reads are done
#pragma unroll
    for (int i = 0; i < VLOADS; ++i)
      store_bf16x8(vt + (i * RPI + lane / LPR) * PITCH + 8 * (lane % LPR), vr[i]);
    wave_sync();
    // V^T as the A operand: k-slots 0..3 are tokens 4j..4j+3 and slots 4..7
    // are tokens 16+4j..16+4j+3, matching the P^T slots in pb.
    const int L = lane & 15;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const __bf16* base = vt + (4 * j + (L >> 2)) * PITCH + 16 * db + 4 * (L & 3);
      const bf16x8 va = concat(lds_read_tr16(base), lds_read_tr16(base + 16 * PITCH));
      acc[db] = mfma16(va, pb, acc[db]);
    }
  }

  // Combine the four wavefronts' partial softmax states through LDS.
  lsum += shfl_xor(lsum, 16);
  lsum += shfl_xor(lsum, 32);
  __syncthreads();
  float* cm = reinterpret_cast<float*>(smem);
  float* cl = cm + kDecodeWaves * kDecodeHeadBlock;
  float* co = cl + kDecodeWaves * kDecodeHeadBlock;
  constexpr int OP = D + 4;
  if (j == 0) {
    cm[w * kDecodeHeadBlock + n] = m;
    cl[w * kDecodeHeadBlock + n] = lsum;
  }
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) co[(w * kDecodeHeadBlock + n) * OP + 16 * db + 4 * j + r] = acc[db][r];
  __syncthreads();
  for (int idx = threadIdx.x; idx < nh * D; idx += kDecodeWaves * 64) {
    const int h = idx / D;
    const int dd = idx - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kDecodeWaves; ++ww) M = fmaxf(M, cm[ww * kDecodeHeadBlock + h]);
    float Ls = 0.f, Os = 0.f;
#pragma unroll
    for (int ww = 0; ww < kDecodeWaves; ++ww) {
      const float wt = fast_exp2(cm[ww * kDecodeHeadBlock + h] - M);   // 0 for idle waves
      Ls += cl[ww * kDecodeHeadBlock + h] * wt;
      Os += co[(ww * kDecodeHeadBlock + h) * OP + dd] * wt;
    }
    const size_t row = ((size_t)b * hq + h_first + h) * nsplit + split;
    part_o[row * D + dd] = Os / Ls;
    if (dd == 0) part_lse[row] = M + __log2f(Ls);
  }
}

// ---------------------------------------------------------------------------
// fp32 split kernel
// ---------------------------------------------------------------------------
constexpr int kF32Tile = 64;        // tokens per workgroup iteration
constexpr int kF32HeadsPerWave = kDecodeHeadBlock / kDecodeWaves;

template <int D>
__global__ __launch_bounds__(kDecodeWaves * 64)
void decode_split_f32(const float* __restrict__ q, const float* __restrict__ kc,
                      const float* __restrict__ vc, const int32_t* __restrict__ lens,
                      float* __restrict__ part_o, float* __restrict__ part_lse,
                      int hq, int hkv, int g, int nhb, int tcap, int chunk, int nsplit,
                      float scale_log2) {
  constexpr int P = D + 1;          // odd pitch: column reads are conflict-free
  constexpr int CPL = D / 64;       // output columns per lane
  __shared__ float ks[kF32Tile * P];
  __shared__ float vs[kF32Tile * P];
  __shared__ float qs[kDecodeHeadBlock * D];
  __shared__ float pw[kDecodeWaves][kF32Tile];

  const int split = blockIdx.x;
  const int kvh = blockIdx.y / nhb;
  const int hb = blockIdx.y - kvh * nhb;
  const int b = blockIdx.z;
  const int T = clamp_len(lens, b, tcap);
  const int t_begin = split * chunk;
  if (t_begin >= T) return;
  const int t_end = min(t_begin + chunk, T);
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int h_first = kvh * g + hb * kDecodeHeadBlock;
  const int nh = min(kDecodeHeadBlock, g - hb * kDecodeHeadBlock);

  for (int i = threadIdx.x; i < nh * D; i += blockDim.x)
    qs[i] = q[((size_t)b * hq + h_first) * D + i];

  float m[kF32HeadsPerWave], l[kF32HeadsPerWave], o[kF32HeadsPerWave][CPL];
#pragma unroll
  for (int s = 0; s < kF32HeadsPerWave; ++s) {
    m[s] = -INFINITY;
    l[s] = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[s][c] = 0.f;
  }
  const size_t kv_off = ((size_t)b * hkv + kvh) * (size_t)tcap * D;

  for (int t0 = t_begin; t0 < t_end; t0 += kF32Tile) {
    __syncthreads();
    for (int i = threadIdx.x; i < kF32Tile * D; i += blockDim.x) {
      const int r = i / D, c = i - (i / D) * D;
      const int t = min(t0 + r, t_end - 1);
      ks[r * P + c] = kc[kv_off + (size_t)t * D + c];
      vs[r * P + c] = vc[kv_off + (size_t)t * D + c];
    }
    __syncthreads();
    const bool valid = t0 + lane < t_end;
#pragma unroll 1
    for (int s = 0; s < kF32HeadsPerWave; ++s) {
      const int hl = w + kDecodeWaves * s;
      if (hl >= nh) break;
      float dot = 0.f;
#pragma unroll 8
      for (int c = 0; c < D; ++c) dot = fmaf(qs[hl * D + c], ks[lane * P + c], dot);
      const float s2 = valid ? dot * scale_log2 : -INFINITY;
      const float m_new = fmaxf(m[s], wave_max(s2));
      const float alpha = fast_exp2(m[s] - m_new);
      const float p = fast_exp2(s2 - m_new);
      l[s] = l[s] * alpha + wave_sum(p);
      m[s] = m_new;
      pw[w][lane] = p;
      wave_sync();
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        float acc = o[s][c] * alpha;
#pragma unroll 8
        for (int t = 0; t < kF32Tile; ++t) acc = fmaf(pw[w][t], vs[t * P + lane + 64 * c], acc);
        o[s][c] = acc;
      }
      wave_sync();
    }
  }
#pragma unroll
  for (int s = 0; s < kF32HeadsPerWave; ++s) {
    const int hl = w + kDecodeWaves * s;
    if (hl >= nh) break;
    const size_t row = ((size_t)b * hq + h_first + hl) * nsplit + split;
#pragma unroll
    for (int c = 0; c < CPL; ++c) part_o[row * D + lane + 64 * c] = o[s][c] / l[s];
    if (lane == 0) part_lse[row] = m[s] + __log2f(l[s]);
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the chunk partials: one workgroup per (query head,
// sequence), one thread per head coordinate.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128)
void decode_merge(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                  const int32_t* __restrict__ lens, float* __restrict__ out, int hq, int d,
                  int tcap, int chunk, int nsplit) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int dd = threadIdx.x;
  if (dd >= d) return;
  const int T = clamp_len(lens, b, tcap);
  const int ns = (T + chunk - 1) / chunk;
  const size_t row0 = ((size_t)b * hq + h) * nsplit;
  float* o = out + ((size_t)b * hq + h) * d + dd;
  if (ns == 0) {   // empty sequence: all-zero output
    *o = 0.f;
    return;
  }
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, part_lse[row0 + s]);
  float L = 0.f, acc = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float wt = fast_exp2(part_lse[row0 + s] - M);
    L += wt;
    acc = fmaf(wt, part_o[(row0 + s) * d + dd], acc);
  }
  *o = acc / L;
}

}  // namespace

DecodeWorkspace decode_workspace_layout(const DecodeShape& s) {
  const int64_t rows = (int64_t)s.batch * s.hq * s.nsplit;
  DecodeWorkspace w;
  w.o_offset = 0;
  w.lse_offset = ((rows * s.d * 4 + 255) / 256) * 256;
  w.total = w.lse_offset + ((rows * 4 + 255) / 256) * 256;
  return w;
}

hipError_t launch_decode_split(const void* q, const void* k, const void* v, const int32_t* lens,
                               float* part_o, float* part_lse, const DecodeShape& s,
                               hipStream_t stream) {
  const int g = s.hq / s.hkv;
  const int nhb = (g + kDecodeHeadBlock - 1) / kDecodeHeadBlock;
  const dim3 grid(s.nsplit, s.hkv * nhb, s.batch);
  const dim3 block(kDecodeWaves * 64);
  const float sl2 = s.scale * kLog2e;
  if (s.dtype == 1) {
    auto qp = static_cast<const __bf16*>(q);
    auto kp = static_cast<const __bf16*>(k);
    auto vp = static_cast<const __bf16*>(v);
    if (s.d == 128)
      hipLaunchKernelGGL(decode_split_bf16<128>, grid, block, 0, stream, qp, kp, vp, lens, part_o,
                         part_lse, s.hq, s.hkv, g, nhb, s.tcap, s.chunk, s.nsplit, sl2);
    else
      hipLaunchKernelGGL(decode_split_bf16<64>, grid, block, 0, stream, qp, kp, vp, lens, part_o,
                         part_lse, s.hq, s.hkv, g, nhb, s.tcap, s.chunk, s.nsplit, sl2);
  } else {
    auto qp = static_cast<const float*>(q);
    auto kp = static_cast<const float*>(k);
    auto vp = static_cast<const float*>(v);
    if (s.d == 128)
      hipLaunchKernelGGL(decode_split_f32<128>, grid, block, 0, stream, qp, kp, vp, lens, part_o,
                         part_lse, s.hq, s.hkv, g, nhb, s.tcap, s.chunk, s.nsplit, sl2);
    else
      hipLaunchKernelGGL(decode_split_f32<64>, grid, block, 0, stream, qp, kp, vp, lens, part_o,
                         part_lse, s.hq, s.hkv, g, nhb, s.tcap, s.chunk, s.nsplit, sl2);
  }
  return hipGetLastError();
}

hipError_t launch_decode_merge(const float* part_o, const float* part_lse, const int32_t* lens,
                               float* out, const DecodeShape& s, hipStream_t stream) {
  const dim3 grid(s.hq, s.batch);
  hipLaunchKernelGGL(decode_merge, grid, dim3(128), 0, stream, part_o, part_lse, lens, out, s.hq,
                     s.d, s.tcap, s.chunk, s.nsplit);
  return hipGetLastError();
}

}  // namespace gqa
