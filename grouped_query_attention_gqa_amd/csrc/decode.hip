// Split-K GQA decode for gfx950.
//
// One decode step re-reads the whole KV cache, so the kernel is bound by HBM
// bandwidth: FLOPs per cache byte equal the group size g = Hq/Hkv
// (deepconcepts.dev, "Grouped-Query Attention", section "Three numbers that
// people expect to move together"), far below the MI355X ridge point.  The
// design therefore reads every K/V element exactly once per group: a
// workgroup attends a run of tokens of one KV head for all g <= 16 query
// heads of the group at once (anrans.github.io, "Attention variants: MQA,
// GQA, MLA", section "Kernels do not need to copy the KV heads": the group's
// query heads act as extra query rows against the shared K/V).
//
// Work partition (balanced "stream" split).  A unit is one (sequence, KV
// head, block of 16 query heads, or for bf16 and E4M3 caches when the group
// is wider, two blocks at head_dim 128 and up to five at head_dim 64); its
// work is the sequence's T_b cached tokens.  The units' tokens are laid end
// to end into one stream of W token-units, and range r of the stream is
// [r*Q, (r+1)*Q): every range has the same size no matter how ragged the
// lengths are, and about one range runs per resident workgroup, so no
// workgroup idles at the tail.  Q is
// chosen on the device from the actual lengths (Q = ceil(W / workgroups),
// at least kMinRange) unless the caller fixes it.  The piece of a range that
// falls inside one unit is a segment; a unit split over n > 1 segments gets
// n partial results (normalised O and log2-sum-exp) that decode_merge
// combines, and a unit covered by a single segment is written straight to
// the output.  Every workgroup derives the geometry itself before its first
// load, so this prologue is kept short: up to 64 sequences, each wavefront
// scans the lengths with wavefront shuffles (no barrier), and the floor
// divisions by Q go through a double reciprocal with one exact correction
// instead of 64-bit integer division.
//
// bf16 path, per wavefront and 32-token tile:
//   S^T[32 tok, 16 heads] = K[32, d] Q^T[d, 16]      v_mfma_f32_16x16x32_bf16
//   online softmax per head (column) with wavefront shuffles, log2 domain
//   O^T[d, 16 heads]    += V^T[d, 32] P^T[32, 16]    (V^T via ds_read_b64_tr_b16)
// K goes straight from HBM into MFMA operand registers (16-byte non-temporal
// buffer loads, 64 contiguous bytes per row); V goes through a per-wave LDS
// tile because the PV contraction runs over tokens, which are strided in
// memory.  The four wavefronts of a workgroup take interleaved tiles of a
// segment and are combined through LDS at the segment's end.
//
// fp32 path: a plain VALU kernel (no fp32 matrix-core shape is worth it at
// d <= 128) with the same partition, K/V tiles staged once per workgroup in
// LDS, one query head per wavefront pass.

#include "gqa_device.hpp"
#include "gqa_launch.hpp"

namespace gqa {

namespace {

constexpr int kThreads = kDecodeWaves * 64;

__device__ __forceinline__ int clamp_len(const int32_t* lens, int b, int tcap) {
  int t = lens[b];
  return t < 0 ? 0 : (t > tcap ? tcap : t);
}

// Stream geometry shared by every workgroup of a launch.
struct Stream {
  long long w;        // total token-units
  long long q;        // tokens per range
  long long ranges;   // number of ranges
  double qinv;        // 1 / q, for the floor divisions by q
};

// floor(x / q) for 0 <= x < W: the plan keeps the range count (about W / q)
// below 2^27, so the double quotient is within one of the true one and the
// remainder's sign fixes it.
__device__ __forceinline__ long long range_div(long long x, const Stream& st) {
  long long d = (long long)((double)x * st.qinv);
  const long long r = x - d * st.q;
  d += (r >= st.q) - (r < 0);
  return d;
}

// floor(a / b) for a >= 0, b >= 1 through a double quotient, instead of the
// long sequence of a 64-bit integer division.  The quotients taken here are
// below 2^45 (W < 2^54 by the plan's bounds, divided by 512 workgroups when
// W is large; range counts below 2^27; unit indices), so the double quotient
// is within one of the true one and the remainder fixes it.
__device__ __forceinline__ long long floor_div(long long a, long long b) {
  long long d = (long long)((double)a / (double)b);
  const long long r = a - d * b;
  d += (r >= b) - (r < 0);
  return d;
}

// Segments of a unit occupying stream positions [s, s + t).
__device__ __forceinline__ int unit_segments(long long s, int t, const Stream& st) {
  return t == 0 ? 0 : (int)(range_div(s + t - 1, st) - range_div(s, st) + 1);
}

// A unit of the stream: sequence b, unit j within the sequence (kvh * nhb +
// head block), its length t, first stream position s and first slot base.
struct Unit {
  int b, j, t, base;
  long long s;
};


// Every workgroup scans the lengths (two block-wide scans over the batch)
// so that any stream position maps to its unit and partial-slot index.
struct ScanSmem {
  long long tok[kThreads];   // per-thread token base
  int seg[kThreads];         // per-thread segment base
  Unit found;
  int per_unit;              // segments of every unit when all lengths are equal and Q divides them, else 0
};

// Block-wide exclusive scan of one value per thread; returns the total.
template <typename T>
__device__ T block_exclusive_scan(T* buf, T v) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const T add = tid >= off ? buf[tid - off] : T(0);
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  const T total = buf[kThreads - 1];
  const T excl = buf[tid] - v;
  __syncthreads();
  buf[tid] = excl;
  __syncthreads();
  return total;
}

// Thread t owns sequences [t*per, min(B, (t+1)*per)).
__device__ __forceinline__ void seq_block(int batch, int& b0, int& b1) {
  const int per = (batch + kThreads - 1) / kThreads;
  b0 = min(batch, (int)threadIdx.x * per);
  b1 = min(batch, b0 + per);
}

__device__ __forceinline__ long long readlane64(long long v, int l) {
  const int lo = __builtin_amdgcn_readlane((int)(unsigned)(unsigned long long)v, l);
  const int hi = __builtin_amdgcn_readlane((int)((unsigned long long)v >> 32), l);
  return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

__device__ __forceinline__ long long uniform64(long long v) {
  const int lo = __builtin_amdgcn_readfirstlane((int)(unsigned)(unsigned long long)v);
  const int hi = __builtin_amdgcn_readfirstlane((int)((unsigned long long)v >> 32));
  return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

// The geometry and units are the same in every lane; saying so keeps them in
// scalar registers (buffer resources built from them stay scalar).
__device__ __forceinline__ Stream uniform_stream(Stream st) {
  st.w = uniform64(st.w);
  st.q = uniform64(st.q);
  st.ranges = uniform64(st.ranges);
  st.qinv = __longlong_as_double(uniform64(__double_as_longlong(st.qinv)));
  return st;
}
__device__ __forceinline__ Unit uniform_unit(Unit u) {
  u.b = __builtin_amdgcn_readfirstlane(u.b);
  u.j = __builtin_amdgcn_readfirstlane(u.j);
  u.t = __builtin_amdgcn_readfirstlane(u.t);
  u.base = __builtin_amdgcn_readfirstlane(u.base);
  u.s = uniform64(u.s);
  return u;
}

template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const T o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

// Up to 64 sequences: every wavefront computes the geometry by itself with
// wavefront scans (lane b owns sequence b), so no barrier is needed.  Each
// wavefront keeps its lanes' sequence start, slot base and length in LDS
// (the same values from every wavefront) for stream_locate.
__device__ Stream stream_setup_wave(ScanSmem& sm, const int32_t* lens, int batch, int upb, int tcap,
                                    int q_fixed) {
  const int lane = threadIdx.x & 63;
  const int t = lane < batch ? clamp_len(lens, lane, tcap) : 0;
  const long long span = (long long)t * upb;
  const long long incl = wave_inclusive_scan(span);
  Stream st;
  st.w = readlane64(incl, 63);
  if (q_fixed > 0) {
    st.q = q_fixed;
  } else {
    st.q = floor_div(st.w + gridDim.x - 1, gridDim.x);
    if (st.q < kMinRange) st.q = kMinRange;
  }
  st.ranges = floor_div(st.w + st.q - 1, st.q);
  st.qinv = 1.0 / (double)st.q;
  // Equal lengths T that Q divides (the usual case of a batch decoded in
  // step): every unit starts on a range boundary and holds T / Q segments,
  // so the slot bases follow without dividing per unit.
  const int t_first = __builtin_amdgcn_readfirstlane(t);
  const bool equal = __builtin_amdgcn_ballot_w64(lane < batch && t != t_first) == 0 && t_first > 0;
  const long long per = equal ? range_div(t_first, st) : 0;
  sm.tok[lane] = incl - span;
  sm.tok[64 + lane] = t;
  if (equal && per * st.q == t_first) {
    sm.seg[lane] = lane * upb * (int)per;
    if (lane == 0) sm.per_unit = (int)per;
    return st;
  }
  long long s = incl - span;
  int segs = 0;
  for (int j = 0; j < upb; ++j, s += t) segs += unit_segments(s, t, st);
  const int sincl = wave_inclusive_scan(segs);
  sm.seg[lane] = sincl - segs;
  if (lane == 0) sm.per_unit = 0;
  return st;
}

__device__ Unit stream_locate_wave(ScanSmem& sm, int upb, const Stream& st, long long x) {
  const int lane = threadIdx.x & 63;
  const long long s_b = sm.tok[lane];
  const int t = (int)sm.tok[64 + lane];
  const int base_b = sm.seg[lane];
  const unsigned long long hit = __ballot(t > 0 && x >= s_b && x < s_b + (long long)t * upb);
  const int l = __builtin_amdgcn_readfirstlane(__ffsll((long long)hit) - 1);   // one lane holds x
  const long long s = readlane64(s_b, l);
  const int tb = __builtin_amdgcn_readlane(t, l);
  int base = __builtin_amdgcn_readlane(base_b, l);
  const int j = (int)floor_div(x - s, tb);
  const int per = __builtin_amdgcn_readfirstlane(sm.per_unit);
  if (per > 0)
    base += j * per;
  else
    for (int jj = 0; jj < j; ++jj) base += unit_segments(s + (long long)jj * tb, tb, st);
  return Unit{l, j, tb, base, s + (long long)j * tb};
}

__device__ Stream stream_setup(ScanSmem& sm, const int32_t* lens, int batch, int upb, int tcap,
                               int q_fixed) {
  if (batch <= 64) return uniform_stream(stream_setup_wave(sm, lens, batch, upb, tcap, q_fixed));
  int b0, b1;
  seq_block(batch, b0, b1);
  long long mine = 0;
  for (int b = b0; b < b1; ++b) mine += (long long)clamp_len(lens, b, tcap) * upb;
  Stream st;
  st.w = block_exclusive_scan(sm.tok, mine);
  if (q_fixed > 0) {
    st.q = q_fixed;
  } else {
    st.q = (st.w + gridDim.x - 1) / gridDim.x;
    if (st.q < kMinRange) st.q = kMinRange;
  }
  st.ranges = (st.w + st.q - 1) / st.q;
  st.qinv = 1.0 / (double)st.q;
  // segment counts, now that every unit's first position is known
  long long s = sm.tok[threadIdx.x];
  int segs = 0;
  for (int b = b0; b < b1; ++b) {
    const int t = clamp_len(lens, b, tcap);
    for (int j = 0; j < upb; ++j, s += t) segs += unit_segments(s, t, st);
  }
  block_exclusive_scan(sm.seg, segs);
  return uniform_stream(st);
}

// The non-empty unit holding stream position x (0 <= x < w).
__device__ Unit stream_locate(ScanSmem& sm, const int32_t* lens, int batch, int upb, int tcap,
                              const Stream& st, long long x) {
  if (batch <= 64) return uniform_unit(stream_locate_wave(sm, upb, st, x));
  int b0, b1;
  seq_block(batch, b0, b1);
  long long s = sm.tok[threadIdx.x];
  int base = sm.seg[threadIdx.x];
  for (int b = b0; b < b1; ++b) {
    const int t = clamp_len(lens, b, tcap);
    if (t > 0 && x >= s && x < s + (long long)t * upb) {   // x lies in sequence b
      const int j = (int)((x - s) / t);
      for (int jj = 0; jj < j; ++jj) base += unit_segments(s + (long long)jj * t, t, st);
      sm.found = Unit{b, j, t, base, s + (long long)j * t};
      break;
    }
    for (int jj = 0; jj < upb; ++jj) base += unit_segments(s + (long long)jj * t, t, st);
    s += (long long)t * upb;
  }
  __syncthreads();
  const Unit u = sm.found;
  __syncthreads();
  return uniform_unit(u);
}

// The next non-empty unit after u (the caller knows one exists).
__device__ __forceinline__ Unit stream_next(const Unit& u, const int32_t* lens, int upb, int tcap,
                                            const Stream& st) {
  Unit n = u;
  n.base = u.base + unit_segments(u.s, u.t, st);
  n.s = u.s + u.t;
  if (u.j + 1 < upb) {
    n.j = u.j + 1;
    return n;
  }
  n.j = 0;
  n.b = u.b + 1;
  n.t = clamp_len(lens, n.b, tcap);
  while (n.t == 0) n.t = clamp_len(lens, ++n.b, tcap);
  return uniform_unit(n);
}

// Records where the merge finds a unit's partials (written by the
// workgroup that holds the unit's first segment).
__device__ __forceinline__ void publish_unit(int* unit_info, const Unit& u, int upb, int nseg,
                                             int kseg) {
  if (kseg == 0 && threadIdx.x == 0) {
    const size_t i = (size_t)u.b * upb + u.j;
    unit_info[2 * i] = u.base;
    unit_info[2 * i + 1] = nseg;
  }
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

// One wavefront's 32-token tile in registers: K as MFMA A operands and the
// V rows as loaded (destined for the wave's LDS tile).
template <int D>
struct DecodeTile {
  bf16x8 k[2][D / 32];
  bf16x8 v[kDecodeWaveTile * D / 8 / 64];
};

// Byte offsets are relative to the segment start; rows at or past the
// segment end lie outside the buffer resource and load as zeros.  The whole
// offset goes in the per-lane operand: the uniform (SGPR) offset of a buffer
// access is not covered by the range check.
template <int D>
__device__ __forceinline__ void load_tile(DecodeTile<D>& t, __amdgpu_buffer_rsrc_t rk,
                                          __amdgpu_buffer_rsrc_t rv, int k_off, int v_off,
                                          int tile_bytes) {
  constexpr int ROW = D * 2;
  constexpr int RPI = 512 / D;
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      t.k[bi][kk] = buffer_load_bf16x8<kCacheStream>(rk, tile_bytes + k_off + bi * 16 * ROW + 64 * kk, 0);
#pragma unroll
  for (int i = 0; i < kDecodeWaveTile * D / 8 / 64; ++i)
    t.v[i] = buffer_load_bf16x8<kCacheStream>(rv, tile_bytes + v_off + i * RPI * ROW, 0);
}

// The same tile from a paged cache: every row the lane loads is looked up in
// the block table.  Rows past the segment end are clamped to its last token
// (their scores are masked, and their values are finite cache contents), and
// page indices are clamped into the pool, so no access leaves the K/V pools
// whatever the table holds.
template <int D>
__device__ __forceinline__ const __bf16* paged_row(const __bf16* pool, const PagedKV& pk, int b, int kvh,
                                                   int hkv, int tok, int tok_last) {
  const int t = min(tok, tok_last);
  int pid = pk.table[(size_t)b * pk.max_pages + (t >> pk.page_log2)];
  pid = min(max(pid, 0), pk.num_pages - 1);
  const size_t row = ((((size_t)pid * hkv + kvh) << pk.page_log2) | (size_t)(t & ((1 << pk.page_log2) - 1)));
  return pool + row * D;
}

template <int D>
__device__ __forceinline__ void load_tile_paged(DecodeTile<D>& t, const __bf16* kpool, const __bf16* vpool,
                                                const PagedKV& pk, int b, int kvh, int hkv, int tok0,
                                                int tok_last, int lane) {
  constexpr int LPR = D / 8;
  constexpr int RPI = 64 / LPR;
  const int n = lane & 15, j = lane >> 4;
#pragma unroll
  for (int bi = 0; bi < 2; ++bi) {
    const bf16x8* row = reinterpret_cast<const bf16x8*>(
        paged_row<D>(kpool, pk, b, kvh, hkv, tok0 + n + 16 * bi, tok_last) + 8 * j);
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) t.k[bi][kk] = __builtin_nontemporal_load(row + 4 * kk);
  }
#pragma unroll
  for (int i = 0; i < kDecodeWaveTile * D / 8 / 64; ++i)
    t.v[i] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(
        paged_row<D>(vpool, pk, b, kvh, hkv, tok0 + lane / LPR + RPI * i, tok_last) + 8 * (lane % LPR)));
}

// FP8 (OCP E4M3) cache: 8 codes (two dwords, code i in byte i) to 8 bf16,
// exactly (every E4M3 value is a bf16 value).  Each conversion result is used
// as a whole 32-bit word: element extraction from the packed result is not
// relied on.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(unsigned w0, unsigned w1) {
  const u32x4 r = {__builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, false)),
                   __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, true)),
                   __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, false)),
                   __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, true))};
  return __builtin_bit_cast(bf16x8, r);
}

// One wavefront's 32-token tile of an E4M3 cache, as loaded (16-byte chunks).
// K: lane (row n, group j) holds the D/4 contiguous codes of rows n and n+16
// starting at column j*D/4, so its MFMA k-slots for step kk are columns
// j*D/4 + 8kk .. +7 (q is laid out the same way).  V: lane holds 16 codes of
// row i*RPI8 + lane/LPR8 starting at column 16*(lane%LPR8).
template <int D>
struct DecodeTileF8 {
  static constexpr int KCH = D / 64;          // 16-byte chunks per lane per K row
  static constexpr int LPR8 = D / 16;         // lanes per V row
  static constexpr int RPI8 = 64 / LPR8;      // V rows per load
  static constexpr int VLOADS8 = kDecodeWaveTile / RPI8;
  u32x4 k[2][KCH];
  u32x4 v[VLOADS8];
};

template <int D>
__device__ __forceinline__ void load_tile_f8(DecodeTileF8<D>& t, __amdgpu_buffer_rsrc_t rk,
                                             __amdgpu_buffer_rsrc_t rv, int lane, int tile_bytes) {
  using T = DecodeTileF8<D>;
  const int n = lane & 15, j = lane >> 4;
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int c = 0; c < T::KCH; ++c)
      t.k[bi][c] = __builtin_bit_cast(u32x4, buffer_load_bf16x8<kCacheStream>(
          rk, tile_bytes + (n + 16 * bi) * D + j * (D / 4) + 16 * c, 0));
#pragma unroll
  for (int i = 0; i < T::VLOADS8; ++i)
    t.v[i] = __builtin_bit_cast(u32x4, buffer_load_bf16x8<kCacheStream>(
        rv, tile_bytes + (i * T::RPI8 + lane / T::LPR8) * D + 16 * (lane % T::LPR8), 0));
}

#ifndef GQA_DECODE_WAVES_PER_EU
#define GQA_DECODE_WAVES_PER_EU 3
#endif

// kPaged: K/V in a page pool addressed through a block table.  kFp8: K/V
// stored as E4M3 codes with one float scale per KV head (k_scale folds into
// the softmax scale, v_scale multiplies the normalised output).  HB: 16-head
// blocks per unit; with HB > 1 a unit covers 16 * HB query heads of one KV
// head, every block scored from the same K registers and accumulated from
// the same V tile, so the group reads its K/V once (two waves per SIMD, as
// launched, leave a wavefront 256 registers: room for the accumulators and
// query operands of two blocks at head_dim 128, of five at head_dim 64).
template <int D, bool kPaged, bool kFp8, int HB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(HB == 1 ? GQA_DECODE_WAVES_PER_EU : 2)))
void decode_split_bf16(const __bf16* __restrict__ q, const void* __restrict__ kcv,
                       const void* __restrict__ vcv, const int32_t* __restrict__ lens,
                       float* __restrict__ out, float* __restrict__ part_o,
                       float* __restrict__ part_lse, int* __restrict__ unit_info, int batch,
                       int hq, int hkv, int g, int nhg, int tcap, int q_fixed, float scale_log2,
                       PagedKV pk, const float* __restrict__ k_scale, const float* __restrict__ v_scale) {
  static_assert(!(kPaged && kFp8), "paged FP8 caches are not supported");
  const __bf16* kc = static_cast<const __bf16*>(kcv);
  const __bf16* vc = static_cast<const __bf16*>(vcv);
  constexpr int ELEM = kFp8 ? 1 : 2;      // bytes per cached element
  constexpr int KSTEPS = D / 32;          // QK^T MFMA steps over the head dim
  constexpr int DBLK = D / 16;            // PV MFMA blocks over the head dim
  constexpr int PITCH = DecodeBf16Smem<D>::kPitch;
  constexpr int LPR = D / 8;              // lanes per V row (16 B each)
  constexpr int RPI = 64 / LPR;           // V rows per wave load
  constexpr int VLOADS = kDecodeWaveTile / RPI;
  constexpr int STRIDE = kDecodeWaves * kDecodeWaveTile;   // tokens between a wave's tiles
  constexpr int OP = D + 4;
  __shared__ __align__(16) char smem[DecodeBf16Smem<D>::kBytes];
  __shared__ ScanSmem scan;

  constexpr int UH = kDecodeHeadBlock * HB;   // query heads per unit (partial row width)
  const int upb = hkv * nhg;
  const Stream st = stream_setup(scan, lens, batch, upb, tcap, q_fixed);

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n = lane & 15;   // token row of A / head column of B and D
  const int j = lane >> 4;   // contraction group
  const int k_off = n * D * 2 + 16 * j;                       // + 16*bi rows, + 64*kk bytes
  const int v_off = (lane / LPR) * D * 2 + 16 * (lane % LPR);  // + RPI*i rows
  __bf16* vt = reinterpret_cast<__bf16*>(smem) + w * kDecodeWaveTile * PITCH;
  float* cm = reinterpret_cast<float*>(smem);
  float* cl = cm + kDecodeWaves * kDecodeHeadBlock;
  float* co = cl + kDecodeWaves * kDecodeHeadBlock;

  for (long long r = blockIdx.x; r < st.ranges; r += gridDim.x) {
    long long lo = r * st.q;
    const long long hi = min(lo + st.q, st.w);
    Unit u = stream_locate(scan, lens, batch, upb, tcap, st, lo);
    while (true) {
      const int t0 = (int)(lo - u.s);                      // first token of the segment
      const int nt = (int)(min(hi, u.s + u.t) - lo);       // tokens in the segment
      const int kvh = u.j / nhg;
      const int hg = u.j - kvh * nhg;
      const int h_first = kvh * g + hg * UH;
      const int nh_unit = min(UH, g - hg * UH);   // heads of this unit (at least one)

      // Q^T as the B operand of block bk: lane holds q[h_first+16bk+n][8j + 32kk .. +7]
      // (for an E4M3 cache: q[..][j*D/4 + 8kk .. +7], the K slot order);
      // heads past the unit's last are zero.
      bf16x8 qb[HB][KSTEPS];
#pragma unroll
      for (int bk = 0; bk < HB; ++bk) {
        const int nh = nh_unit - kDecodeHeadBlock * bk;
        const __bf16* qrow = q + ((size_t)u.b * hq + h_first + kDecodeHeadBlock * bk + max(0, min(n, nh - 1))) * D;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          qb[bk][kk] = nh > 0 ? load_bf16x8(qrow + (kFp8 ? j * (D / 4) + 8 * kk : 8 * j + 32 * kk)) : bf16x8{};
          if (n >= nh) qb[bk][kk] = bf16x8{};
        }
      }
      const size_t seg_off = kPaged ? 0 : (((size_t)u.b * hkv + kvh) * (size_t)tcap + t0) * D * ELEM;
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(reinterpret_cast<const char*>(kcv) + seg_off, nt * D * ELEM);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(reinterpret_cast<const char*>(vcv) + seg_off, nt * D * ELEM);
      const float sl2 = kFp8 ? scale_log2 * k_scale[kvh] : scale_log2;
      const float vsc = kFp8 ? v_scale[kvh] : 1.f;

      float m[HB];      // running max of head n of each block (log2 domain), same in all 4 lane groups
      float lsum[HB];   // this lane's share of the running denominator of head n
      f32x4 acc[HB][DBLK];
#pragma unroll
      for (int bk = 0; bk < HB; ++bk) {
        m[bk] = -INFINITY;
        lsum[bk] = 0.f;
#pragma unroll
        for (int i = 0; i < DBLK; ++i) acc[bk][i] = f32x4{0.f, 0.f, 0.f, 0.f};
      }

      for (int tok = w * kDecodeWaveTile; tok < nt; tok += STRIDE) {
        DecodeTile<D> tl;
        DecodeTileF8<D> tf;
        if (kFp8) {
          load_tile_f8<D>(tf, rk, rv, lane, tok * D);
#pragma unroll
          for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk)
              tl.k[bi][kk] = e4m3x8_to_bf16(tf.k[bi][kk >> 1][2 * (kk & 1)], tf.k[bi][kk >> 1][2 * (kk & 1) + 1]);
        } else if (kPaged) {
          load_tile_paged<D>(tl, kc, vc, pk, u.b, kvh, hkv, t0 + tok, t0 + nt - 1, lane);
        } else {
          load_tile<D>(tl, rk, rv, k_off, v_off, tok * D * 2);
        }
        bf16x8 pb[HB];
#pragma unroll
        for (int bk = 0; bk < HB; ++bk) {
          f32x4 sc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
          for (int kk = 0; kk < KSTEPS; ++kk) {
            sc[0] = mfma16(tl.k[0][kk], qb[bk][kk], sc[0]);
            sc[1] = mfma16(tl.k[1][kk], qb[bk][kk], sc[1]);
          }
          // sc[bi][r] = score of token tok + 16*bi + 4*j + r for head n.
          float s2[8];
          float mx = -INFINITY;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int tt = tok + 16 * (e >> 2) + 4 * j + (e & 3);
            s2[e] = tt < nt ? sc[e >> 2][e & 3] * sl2 : -INFINITY;
            mx = fmaxf(mx, s2[e]);
          }
          mx = fmaxf(mx, shfl_xor(mx, 16));
          mx = fmaxf(mx, shfl_xor(mx, 32));
          const float m_new = fmaxf(m[bk], mx);   // finite: every tile holds a valid token
          const float alpha = fast_exp2(m[bk] - m_new);
          float ps = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const __bf16 p = (__bf16)fast_exp2(s2[e] - m_new);
            pb[bk][e] = p;
            ps += (float)p;   // the denominator sums exactly the weights PV uses
          }
          lsum[bk] = lsum[bk] * alpha + ps;
          m[bk] = m_new;
#pragma unroll
          for (int i = 0; i < DBLK; ++i) acc[bk][i] *= alpha;
        }

        wave_sync();   // the previous tile's transposed reads are done
        if (kFp8) {
          using TF = DecodeTileF8<D>;
#pragma unroll
          for (int i = 0; i < TF::VLOADS8; ++i) {
            __bf16* dst = vt + (i * TF::RPI8 + lane / TF::LPR8) * PITCH + 16 * (lane % TF::LPR8);
            store_bf16x8(dst, e4m3x8_to_bf16(tf.v[i][0], tf.v[i][1]));
            store_bf16x8(dst + 8, e4m3x8_to_bf16(tf.v[i][2], tf.v[i][3]));
          }
        } else {
#pragma unroll
          for (int i = 0; i < VLOADS; ++i)
            store_bf16x8(vt + (i * RPI + lane / LPR) * PITCH + 8 * (lane % LPR), tl.v[i]);
        }
        wave_sync();
        // V^T as the A operand: k-slots 0..3 are tokens 4j..4j+3 and slots
        // 4..7 are tokens 16+4j..16+4j+3, matching the P^T slots in pb.
        const int L = lane & 15;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
          const __bf16* base = vt + (4 * j + (L >> 2)) * PITCH + 16 * db + 4 * (L & 3);
          const bf16x8 va = concat(lds_read_tr16(base), lds_read_tr16(base + 16 * PITCH));
#pragma unroll
          for (int bk = 0; bk < HB; ++bk) acc[bk][db] = mfma16(va, pb[bk], acc[bk][db]);
        }
      }

      // Combine the four wavefronts' softmax states through LDS, one block
      // of 16 heads at a time.
      const int nseg = unit_segments(u.s, u.t, st);
      const int kseg = (int)(r - range_div(u.s, st));
      const size_t slot = (size_t)u.base + kseg;
#pragma unroll
      for (int bk = 0; bk < HB; ++bk) {
        const int nh = nh_unit - kDecodeHeadBlock * bk;
        if (nh <= 0) break;   // uniform: the unit has fewer heads than HB blocks
        const float lsb = lsum[bk] + shfl_xor(lsum[bk], 16);
        const float lsw = lsb + shfl_xor(lsb, 32);
        __syncthreads();   // every wave is done with its V tile (or the previous block's combine)
        if (j == 0) {
          cm[w * kDecodeHeadBlock + n] = m[bk];
          cl[w * kDecodeHeadBlock + n] = lsw;
        }
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            co[(w * kDecodeHeadBlock + n) * OP + 16 * db + 4 * j + rr] = acc[bk][db][rr];
        __syncthreads();
        for (int idx = threadIdx.x; idx < min(nh, kDecodeHeadBlock) * D; idx += kThreads) {
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
          const int hu = kDecodeHeadBlock * bk + h;   // head within the unit
          if (nseg == 1) {
            out[((size_t)u.b * hq + h_first + hu) * D + dd] = Os / Ls * vsc;
          } else {
            part_o[(slot * UH + hu) * D + dd] = Os / Ls * vsc;
            if (dd == 0) part_lse[slot * UH + hu] = M + __log2f(Ls);
          }
        }
      }
      publish_unit(unit_info, u, upb, nseg, kseg);
      lo += nt;
      if (lo >= hi) break;
      __syncthreads();   // the combine buffers are read before the next segment's tiles
      u = stream_next(u, lens, upb, tcap, st);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// fp32 split kernel
// ---------------------------------------------------------------------------
constexpr int kF32Tile = 64;        // tokens per workgroup iteration
constexpr int kF32HeadsPerWave = kDecodeHeadBlock / kDecodeWaves;

template <int D>
__global__ __launch_bounds__(kThreads)
void decode_split_f32(const float* __restrict__ q, const float* __restrict__ kc,
                      const float* __restrict__ vc, const int32_t* __restrict__ lens,
                      float* __restrict__ out, float* __restrict__ part_o,
                      float* __restrict__ part_lse, int* __restrict__ unit_info, int batch,
                      int hq, int hkv, int g, int nhb, int tcap, int q_fixed, float scale_log2) {
  // (one 16-head block per unit on this path: nhb is the unit count per KV head)
  constexpr int P = D + 1;          // odd pitch: column reads are conflict-free
  constexpr int CPL = D / 64;       // output columns per lane
  __shared__ float ks[kF32Tile * P];
  __shared__ float vs[kF32Tile * P];
  __shared__ float qs[kDecodeHeadBlock * D];
  __shared__ float pw[kDecodeWaves][kF32Tile];
  __shared__ ScanSmem scan;

  const int upb = hkv * nhb;
  const Stream st = stream_setup(scan, lens, batch, upb, tcap, q_fixed);
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;

  for (long long r = blockIdx.x; r < st.ranges; r += gridDim.x) {
    long long lo = r * st.q;
    const long long hi = min(lo + st.q, st.w);
    Unit u = stream_locate(scan, lens, batch, upb, tcap, st, lo);
    while (true) {
      const int t0 = (int)(lo - u.s);
      const int nt = (int)(min(hi, u.s + u.t) - lo);
      const int kvh = u.j / nhb;
      const int hb = u.j - kvh * nhb;
      const int h_first = kvh * g + hb * kDecodeHeadBlock;
      const int nh = min(kDecodeHeadBlock, g - hb * kDecodeHeadBlock);

      for (int i = threadIdx.x; i < nh * D; i += kThreads)
        qs[i] = q[((size_t)u.b * hq + h_first) * D + i];

      float m[kF32HeadsPerWave], l[kF32HeadsPerWave], o[kF32HeadsPerWave][CPL];
#pragma unroll
      for (int s = 0; s < kF32HeadsPerWave; ++s) {
        m[s] = -INFINITY;
        l[s] = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) o[s][c] = 0.f;
      }
      const size_t kv_off = (((size_t)u.b * hkv + kvh) * (size_t)tcap + t0) * D;

      for (int tt0 = 0; tt0 < nt; tt0 += kF32Tile) {
        __syncthreads();
        for (int i = threadIdx.x; i < kF32Tile * D; i += kThreads) {
          const int rr = i / D, c = i - (i / D) * D;
          const int t = min(tt0 + rr, nt - 1);   // rows past the end repeat the last valid row
          ks[rr * P + c] = kc[kv_off + (size_t)t * D + c];
          vs[rr * P + c] = vc[kv_off + (size_t)t * D + c];
        }
        __syncthreads();
        const bool valid = tt0 + lane < nt;
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
            float a = o[s][c] * alpha;
#pragma unroll 8
            for (int t = 0; t < kF32Tile; ++t) a = fmaf(pw[w][t], vs[t * P + lane + 64 * c], a);
            o[s][c] = a;
          }
          wave_sync();
        }
      }
      const int nseg = unit_segments(u.s, u.t, st);
      const int kseg = (int)(r - range_div(u.s, st));
      const size_t slot = (size_t)u.base + kseg;
#pragma unroll
      for (int s = 0; s < kF32HeadsPerWave; ++s) {
        const int hl = w + kDecodeWaves * s;
        if (hl >= nh) break;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const float val = o[s][c] / l[s];
          if (nseg == 1)
            out[((size_t)u.b * hq + h_first + hl) * D + lane + 64 * c] = val;
          else
            part_o[(slot * kDecodeHeadBlock + hl) * D + lane + 64 * c] = val;
        }
        if (nseg != 1 && lane == 0) part_lse[slot * kDecodeHeadBlock + hl] = m[s] + __log2f(l[s]);
      }
      publish_unit(unit_info, u, upb, nseg, kseg);
      lo += nt;
      if (lo >= hi) break;
      u = stream_next(u, lens, upb, tcap, st);
      __syncthreads();   // qs is rewritten for the next unit
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the segment partials: one workgroup per (query head,
// sequence).  Threads hold 4 head coordinates each; D/4 threads cover one
// partial row, so the 256 threads form 1024/D row groups.  A round loads up
// to eight rows per thread, each row's lse and output together, so one round
// trip to memory serves up to 8192/D segments.  Every row group keeps its
// own running maximum (online softmax over the partials); the groups are
// then combined through LDS against the largest.  Units written directly by
// a single segment are skipped; empty sequences get zeros.
// ---------------------------------------------------------------------------
constexpr int kMergeThreads = 256;

template <int D>
__global__ __launch_bounds__(kMergeThreads)
void decode_merge(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                  const int* __restrict__ unit_info, const int32_t* __restrict__ lens,
                  float* __restrict__ out, int hq, int hkv, int g, int nhg, int uh, int tcap) {
  constexpr int C4 = D / 4;                  // float4 columns per row
  constexpr int ROWS = kMergeThreads / C4;   // row groups
  constexpr int U = 8;                       // rows per thread per round
  __shared__ f32x4 racc[ROWS][C4];
  __shared__ float rl[ROWS];
  __shared__ float rm[ROWS];
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  float* o = out + ((size_t)b * hq + h) * D;
  if (clamp_len(lens, b, tcap) == 0) {   // empty sequence: all-zero output
    for (int i = tid; i < D; i += kMergeThreads) o[i] = 0.f;
    return;
  }
  const int kvh = h / g;
  const int hg = (h - kvh * g) / uh;         // unit of uh consecutive heads
  const int hl = (h - kvh * g) - hg * uh;    // head within the unit
  const size_t unit = ((size_t)b * hkv + kvh) * nhg + hg;
  const int base = unit_info[2 * unit];
  const int ns = unit_info[2 * unit + 1];
  if (ns <= 1) return;   // written directly by its only segment

  // Row group sr: segments sr, sr + ROWS, ...  Every segment holds at least
  // one token, so its lse is finite; rows past ns are padding with lse -inf
  // (weight 0) and a zero output, and are not loaded.
  const int c4 = tid % C4;
  const int sr = tid / C4;
  float m = -INFINITY, L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = sr; s0 < ns; s0 += U * ROWS) {
    float lr[U];
    f32x4 ov[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * ROWS;
      const size_t row = ((size_t)base + s) * uh + hl;
      lr[u] = -INFINITY;
      ov[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (s < ns) {   // padding rows load nothing
        lr[u] = part_lse[row];
        ov[u] = reinterpret_cast<const f32x4*>(part_o + row * D)[c4];
      }
    }
    float mn = m;
#pragma unroll
    for (int u = 0; u < U; ++u) mn = fmaxf(mn, lr[u]);   // finite: lr[0] is
    const float rs = fast_exp2(m - mn);
    L *= rs;
    acc *= rs;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float wt = fast_exp2(lr[u] - mn);
      L += wt;
      acc += wt * ov[u];
    }
    m = mn;
  }
  racc[sr][c4] = acc;
  if (c4 == 0) {
    rl[sr] = L;
    rm[sr] = m;   // -inf for a group with no rows: weight 0 below
  }
  __syncthreads();
  if (sr == 0) {
    float M = rm[0];
#pragma unroll
    for (int rr = 1; rr < ROWS; ++rr) M = fmaxf(M, rm[rr]);
    float Lt = 0.f;
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rr = 0; rr < ROWS; ++rr) {
      const float wt = fast_exp2(rm[rr] - M);
      Lt += wt * rl[rr];
      a += wt * racc[rr][c4];
    }
    reinterpret_cast<f32x4*>(o)[c4] = a / Lt;
  }
}

}  // namespace

DecodeWorkspace decode_workspace_layout(const DecodeShape& s) {
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  DecodeWorkspace w;
  w.info_offset = 0;
  w.lse_offset = up((int64_t)s.units * 2 * 4);
  const int64_t uh = (int64_t)kDecodeHeadBlock * s.hb;   // heads per unit: the width of a partial row
  w.o_offset = w.lse_offset + up(s.max_slots * uh * 4);
  w.total = w.o_offset + up(s.max_slots * uh * (int64_t)s.d * 4);
  return w;
}

hipError_t launch_decode_split(const void* q, const void* k, const void* v, const int32_t* lens,
                               float* out, char* workspace, const DecodeShape& s,
                               hipStream_t stream, const PagedKV& paged, const float* k_scale,
                               const float* v_scale) {
  const int g = s.hq / s.hkv;
  const DecodeWorkspace wl = decode_workspace_layout(s);
  int* info = reinterpret_cast<int*>(workspace + wl.info_offset);
  float* plse = reinterpret_cast<float*>(workspace + wl.lse_offset);
  float* po = reinterpret_cast<float*>(workspace + wl.o_offset);
  const dim3 grid(s.grid);
  const dim3 block(kThreads);
  const float sl2 = s.scale * kLog2e;
  if (s.dtype == 1 || s.dtype == 2) {
    auto qp = static_cast<const __bf16*>(q);
#define GQA_SPLIT2(DD, PG, F8, HB)                                                                       \
  hipLaunchKernelGGL((decode_split_bf16<DD, PG, F8, HB>), grid, block, 0, stream, qp, k, v, lens, out, po, plse, \
                     info, s.batch, s.hq, s.hkv, g, s.nhg, s.tcap, s.q_fixed, sl2, paged, k_scale, v_scale)
#define GQA_SPLIT(DD, PG, F8)        \
  if (s.hb == 2) {                   \
    GQA_SPLIT2(DD, PG, F8, 2);       \
  } else {                           \
    GQA_SPLIT2(DD, PG, F8, 1);       \
  }
#define GQA_SPLIT64(PG, F8)          \
  if (s.hb == 5) {                   \
    GQA_SPLIT2(64, PG, F8, 5);       \
  } else if (s.hb == 4) {            \
    GQA_SPLIT2(64, PG, F8, 4);       \
  } else if (s.hb == 3) {            \
    GQA_SPLIT2(64, PG, F8, 3);       \
  } else {                           \
    GQA_SPLIT(64, PG, F8)            \
  }
    if (s.dtype == 2) {
      if (s.d == 128) { GQA_SPLIT(128, false, true) }
      else { GQA_SPLIT64(false, true) }
    } else if (paged.table != nullptr) {
      if (s.d == 128) { GQA_SPLIT(128, true, false) }
      else { GQA_SPLIT64(true, false) }
    } else {
      if (s.d == 128) { GQA_SPLIT(128, false, false) }
      else { GQA_SPLIT64(false, false) }
    }
#undef GQA_SPLIT64
#undef GQA_SPLIT
#undef GQA_SPLIT2
  } else {
    auto qp = static_cast<const float*>(q);
    auto kp = static_cast<const float*>(k);
    auto vp = static_cast<const float*>(v);
    if (s.d == 128)
      hipLaunchKernelGGL(decode_split_f32<128>, grid, block, 0, stream, qp, kp, vp, lens, out, po,
                         plse, info, s.batch, s.hq, s.hkv, g, s.nhg, s.tcap, s.q_fixed, sl2);
    else
      hipLaunchKernelGGL(decode_split_f32<64>, grid, block, 0, stream, qp, kp, vp, lens, out, po,
                         plse, info, s.batch, s.hq, s.hkv, g, s.nhg, s.tcap, s.q_fixed, sl2);
  }
  return hipGetLastError();
}

hipError_t launch_decode_merge(const int32_t* lens, float* out, const char* workspace,
                               const DecodeShape& s, hipStream_t stream) {
  const int g = s.hq / s.hkv;
  const DecodeWorkspace wl = decode_workspace_layout(s);
  const int* info = reinterpret_cast<const int*>(workspace + wl.info_offset);
  const float* plse = reinterpret_cast<const float*>(workspace + wl.lse_offset);
  const float* po = reinterpret_cast<const float*>(workspace + wl.o_offset);
  const dim3 grid(s.hq, s.batch);
  if (s.d == 128)
    hipLaunchKernelGGL(decode_merge<128>, grid, dim3(kMergeThreads), 0, stream, po, plse, info, lens,
                       out, s.hq, s.hkv, g, s.nhg, kDecodeHeadBlock * s.hb, s.tcap);
  else
    hipLaunchKernelGGL(decode_merge<64>, grid, dim3(kMergeThreads), 0, stream, po, plse, info, lens,
                       out, s.hq, s.hkv, g, s.nhg, kDecodeHeadBlock * s.hb, s.tcap);
  return hipGetLastError();
}

}  // namespace gqa
