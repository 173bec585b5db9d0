"""Seeded synthetic inputs for grouped-query attention over a KV cache.

This module is shared by the tests, the bench and the smoke check. It draws
random numbers and fixes storage formats; it contains none of the attention
arithmetic (no scores, no softmax, no head mapping), so both the float64
oracle and the GPU path can consume its arrays without sharing method code.

Workloads (the five shapes the library is measured and checked on):

  tiny-f32    tiny decode, fp32: B=1, Hq=8, Hkv=2, d=64, 256 cached tokens
  llama3-8b   Llama-3-8B-shaped decode, bf16: B=32, Hq=32, Hkv=8, d=128, 8192 tokens
  wide-group  wide-group decode, bf16: B=64, Hq=32, Hkv=2, d=128, ragged lengths
      drawn uniformly from [1024, 32768] (inclusive), cache capacity 32768
  mqa-128k    MQA long-context decode, bf16: B=4, Hq=16, Hkv=1, d=128, 131072 tokens
  prefill-4k  causal prefill, bf16: B=2, Hq=32, Hkv=8, d=128, N=4096
  mla-decode  (WIDE_CONFIGS) decode in the absorbed-MLA shape, bf16: B=64,
      Hq=128 query heads over one cached 576-column row per token (512 latent
      + 64 rotary), value = the first 512 columns, 4096 tokens, seed 1006
  group-32    32 query heads on one KV head, bf16: B=32, d=128, 8192 tokens, seed 1007
  group-71    71 query heads on one KV head (the Falcon-7B head count), bf16:
      B=16, d=64, 8192 tokens, seed 1008

Recipe: seeds 1001..1005 in the order listed above; ``SeedSequence(seed).spawn(4)`` gives
independent PCG64 streams for (lengths, Q, K, V) in that order; values are
i.i.d. standard normal drawn as float32 and, for bf16 workloads, rounded to
bfloat16 with round-to-nearest-even.  Cache slots past a sequence's length
are filled with NaN so that any kernel reading them is caught.  The
backward pass of a prefill workload also draws an upstream output gradient
from a fifth child stream (``make_dout``).

Head-major layouts: q ``[B, Hq, d]`` (decode) or ``[B, Hq, N, d]`` (prefill);
k/v ``[B, Hkv, T_cap, d]`` (decode cache) or ``[B, Hkv, N, d]`` (prefill).
bf16 tensors are held as ``uint16`` bit patterns; ``bf16_bits_to_f32``
widens them exactly.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BF16_NAN_BITS = np.uint16(0x7FC0)


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    dtype: str            # "f32" or "bf16": storage type of q, k, v
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    max_seq_len: int      # cache capacity T_cap
    min_len: int          # lengths uniform in [min_len, max_len]
    max_len: int
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def ragged(self) -> bool:
        return self.min_len != self.max_len


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    name: str
    dtype: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    seq_len: int
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


CONFIGS = {
    "tiny-f32": DecodeConfig("tiny-decode-fp32", "f32", 1, 8, 2, 64, 256, 256, 256, 1001),
    "llama3-8b": DecodeConfig("llama3-8b-decode-bf16", "bf16", 32, 32, 8, 128, 8192, 8192, 8192, 1002),
    "wide-group": DecodeConfig("wide-group-ragged-decode-bf16", "bf16", 64, 32, 2, 128, 32768, 1024, 32768, 1003),
    "mqa-128k": DecodeConfig("mqa-long-decode-bf16", "bf16", 4, 16, 1, 128, 131072, 131072, 131072, 1004),
    "prefill-4k": PrefillConfig("causal-prefill-bf16", "bf16", 2, 32, 8, 128, 4096, 1005),
    # groups wider than one 16-head block (traffic of the shared K/V read)
    "group-32": DecodeConfig("group-32-decode-bf16", "bf16", 32, 32, 1, 128, 8192, 8192, 8192, 1007),
    "group-71": DecodeConfig("group-71-decode-bf16", "bf16", 16, 71, 1, 64, 8192, 8192, 8192, 1008),
}


@dataclasses.dataclass(frozen=True)
class WideConfig:
    """Decode in the absorbed-MLA shape: Hq query heads over Hkv cached rows
    of d_k columns, the first d_v of which are also the value."""
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    d_k: int
    d_v: int
    max_seq_len: int
    min_len: int
    max_len: int
    seed: int
    scale_dim: int        # scores are divided by sqrt(scale_dim)
    dtype: str = "bf16"

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.scale_dim)

    @property
    def ragged(self) -> bool:
        return self.min_len != self.max_len


# The MLA decode shape: 128 query heads sharing one 512-column latent row plus
# a 64-column rotary key (576 cached numbers per token); scores divided by
# sqrt(128 + 64), the per-head query/key width before absorption.
WIDE_CONFIGS = {
    "mla-decode": WideConfig("mla-absorbed-decode-bf16", 64, 128, 1, 576, 512, 4096, 4096, 4096, 1006, 192),
}


def describe(cfg) -> str:
    """One-line workload description used in bench output and test ids."""
    if isinstance(cfg, WideConfig):
        lens = (f"T={cfg.max_len}" if not cfg.ragged
                else f"T~U[{cfg.min_len},{cfg.max_len}] cap={cfg.max_seq_len}")
        return (f"wide decode {cfg.dtype} B={cfg.batch} Hq={cfg.num_q_heads} Hkv={cfg.num_kv_heads} "
                f"d_k={cfg.d_k} d_v={cfg.d_v} {lens}")
    if isinstance(cfg, DecodeConfig):
        lens = (f"T={cfg.max_len}" if not cfg.ragged
                else f"T~U[{cfg.min_len},{cfg.max_len}] cap={cfg.max_seq_len}")
        return (f"decode {cfg.dtype} B={cfg.batch} Hq={cfg.num_q_heads} "
                f"Hkv={cfg.num_kv_heads} d={cfg.head_dim} {lens}")
    return (f"causal prefill {cfg.dtype} B={cfg.batch} Hq={cfg.num_q_heads} "
            f"Hkv={cfg.num_kv_heads} d={cfg.head_dim} N={cfg.seq_len}")


# ---------------------------------------------------------------------------
# bfloat16 storage helpers (IEEE bit manipulation only)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return uint16 bits.

    Inputs must be finite (the generator only rounds normal draws)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of stored values (fp32 arrays or bf16 bit arrays)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _normals(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def _streams(seed: int):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(4)]


# ---------------------------------------------------------------------------
# Generators
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class DecodeInputs:
    cfg: DecodeConfig
    q: np.ndarray          # [B, Hq, d]          (float32 or uint16 bf16 bits)
    k_cache: np.ndarray    # [B, Hkv, T_cap, d]
    v_cache: np.ndarray    # [B, Hkv, T_cap, d]
    seq_lens: np.ndarray   # [B] int32


@dataclasses.dataclass
class PrefillInputs:
    cfg: PrefillConfig
    q: np.ndarray          # [B, Hq, N, d]  (uint16 bf16 bits)
    k: np.ndarray          # [B, Hkv, N, d]
    v: np.ndarray          # [B, Hkv, N, d]


def make_seq_lens(cfg: DecodeConfig, rng: Optional[np.random.Generator] = None) -> np.ndarray:
    if rng is None:
        rng = _streams(cfg.seed)[0]
    if not cfg.ragged:
        return np.full(cfg.batch, cfg.max_len, dtype=np.int32)
    return rng.integers(cfg.min_len, cfg.max_len, endpoint=True,
                        size=cfg.batch).astype(np.int32)


def make_decode(cfg: DecodeConfig, poison_padding: bool = True) -> DecodeInputs:
    """Deterministic decode inputs for ``cfg`` (see module docstring)."""
    r_len, r_q, r_k, r_v = _streams(cfg.seed)
    seq_lens = make_seq_lens(cfg, r_len)
    B, Hq, Hkv, d, T = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.max_seq_len
    q = _normals(r_q, (B, Hq, d), cfg.dtype)
    store = np.uint16 if cfg.dtype == "bf16" else np.float32
    k = np.empty((B, Hkv, T, d), dtype=store)
    v = np.empty((B, Hkv, T, d), dtype=store)
    for b in range(B):   # per sequence keeps the float32 temporaries small
        k[b] = _normals(r_k, (Hkv, T, d), cfg.dtype)
        v[b] = _normals(r_v, (Hkv, T, d), cfg.dtype)
    if poison_padding:
        poison_past_lengths(k, seq_lens, cfg.dtype)
        poison_past_lengths(v, seq_lens, cfg.dtype)
    return DecodeInputs(cfg, q, k, v, seq_lens)


def poison_past_lengths(cache: np.ndarray, seq_lens: np.ndarray, dtype: str) -> None:
    """Fill cache slots at positions >= seq_lens[b] with NaN, in place."""
    fill = BF16_NAN_BITS if dtype == "bf16" else np.float32(np.nan)
    for b, t in enumerate(seq_lens):
        cache[b, :, int(t):, :] = fill


def make_prefill(cfg: PrefillConfig) -> PrefillInputs:
    _, r_q, r_k, r_v = _streams(cfg.seed)
    B, Hq, Hkv, N, d = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.seq_len, cfg.head_dim
    q = _normals(r_q, (B, Hq, N, d), cfg.dtype)
    k = _normals(r_k, (B, Hkv, N, d), cfg.dtype)
    v = _normals(r_v, (B, Hkv, N, d), cfg.dtype)
    return PrefillInputs(cfg, q, k, v)


def small_decode(dtype: str, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 seq_lens, max_seq_len: int, seed: int) -> DecodeInputs:
    """Decode inputs of an arbitrary small shape (edge cases, ragged tails)."""
    lens = np.asarray(seq_lens, dtype=np.int32)
    cfg = DecodeConfig(f"small-{seed}", dtype, batch, num_q_heads, num_kv_heads, head_dim,
                       max_seq_len, int(lens.min()) if lens.size else 0,
                       int(lens.max()) if lens.size else 0, seed)
    _, r_q, r_k, r_v = _streams(seed)
    q = _normals(r_q, (batch, num_q_heads, head_dim), dtype)
    k = _normals(r_k, (batch, num_kv_heads, max_seq_len, head_dim), dtype)
    v = _normals(r_v, (batch, num_kv_heads, max_seq_len, head_dim), dtype)
    poison_past_lengths(k, lens, dtype)
    poison_past_lengths(v, lens, dtype)
    return DecodeInputs(cfg, q, k, v, lens)


def small_prefill(batch: int, num_q_heads: int, num_kv_heads: int, seq_len: int,
                  head_dim: int, seed: int) -> PrefillInputs:
    cfg = PrefillConfig(f"small-{seed}", "bf16", batch, num_q_heads, num_kv_heads,
                        head_dim, seq_len, seed)
    return make_prefill(cfg)


def make_dout(cfg: PrefillConfig) -> np.ndarray:
    """Upstream gradient of the prefill output, [B, Hq, N, d], for the
    backward pass: i.i.d. standard normal from the fifth child stream of the
    workload's seed (the first four, and hence q/k/v, are unchanged), stored
    like q (bf16 bits for bf16 workloads)."""
    r_do = np.random.Generator(np.random.PCG64(np.random.SeedSequence(cfg.seed).spawn(5)[4]))
    return _normals(r_do, (cfg.batch, cfg.num_q_heads, cfg.seq_len, cfg.head_dim), cfg.dtype)


# ---------------------------------------------------------------------------
# Paged KV cache (storage layout only; no attention arithmetic)
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class PagedInputs:
    """Decode inputs whose K/V live in a shared pool of fixed-size pages.

    k_pages, v_pages: [num_pages, Hkv, page_size, d]; block_table[b, i] is the
    pool index of the page holding tokens i*page_size .. (i+1)*page_size - 1 of
    sequence b, or -1 where the sequence has no such page.  Pool order is a
    seeded random permutation; pages no sequence uses are filled with NaN."""
    cfg: DecodeConfig
    q: np.ndarray
    k_pages: np.ndarray
    v_pages: np.ndarray
    block_table: np.ndarray   # [B, max_pages] int32
    seq_lens: np.ndarray      # [B] int32
    page_size: int


def make_paged(inp: DecodeInputs, page_size: int, spare_pages: int = 7, seed: int = 7) -> PagedInputs:
    """Scatter a contiguous decode cache into a permuted page pool."""
    cfg = inp.cfg
    B, Hkv, T, d = inp.k_cache.shape
    max_pages = -(-T // page_size)
    used = [-(-int(t) // page_size) for t in inp.seq_lens]
    n_pool = sum(used) + spare_pages
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    perm = rng.permutation(n_pool).astype(np.int32)
    fill = BF16_NAN_BITS if cfg.dtype == "bf16" else np.float32(np.nan)
    k_pages = np.full((n_pool, Hkv, page_size, d), fill, dtype=inp.k_cache.dtype)
    v_pages = np.full((n_pool, Hkv, page_size, d), fill, dtype=inp.v_cache.dtype)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    nxt = 0
    for b in range(B):
        for i in range(used[b]):
            pid = int(perm[nxt])
            nxt += 1
            table[b, i] = pid
            lo, hi = i * page_size, min((i + 1) * page_size, T)
            k_pages[pid, :, :hi - lo] = inp.k_cache[b, :, lo:hi]
            v_pages[pid, :, :hi - lo] = inp.v_cache[b, :, lo:hi]
    return PagedInputs(cfg, inp.q, k_pages, v_pages, table, inp.seq_lens, page_size)


# ---------------------------------------------------------------------------
# FP8 (OCP E4M3) KV cache (storage format only; no attention arithmetic)
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def _e4m3_positive_grid() -> np.ndarray:
    """Values of the 127 non-negative finite E4M3 codes 0x00..0x7E, indexed by
    code: exponent field e (bias 7), mantissa m (3 bits); e = 0 is subnormal."""
    codes = np.arange(0x7F)
    e, m = codes >> 3, codes & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (e - 7.0))


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round finite values to OCP E4M3 (nearest, ties to even mantissa),
    saturating at +-448; returns uint8 codes.  Never produces NaN."""
    x = np.asarray(x, dtype=np.float64)
    grid = _e4m3_positive_grid()
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(grid, a, side="left"), 0, len(grid) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - grid[lo], grid[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x) & (code != 0), code | 0x80, code).astype(np.uint8)


@dataclasses.dataclass
class Fp8Inputs:
    """Decode inputs with an E4M3 cache and one float32 scale per KV head for
    K and for V: stored value * scale[kv head] is the cache value."""
    cfg: DecodeConfig
    q: np.ndarray          # [B, Hq, d] bf16 bits
    k_cache: np.ndarray    # [B, Hkv, T_cap, d] uint8 E4M3 codes
    v_cache: np.ndarray
    k_scale: np.ndarray    # [Hkv] float32
    v_scale: np.ndarray
    seq_lens: np.ndarray


def make_fp8(inp: DecodeInputs) -> Fp8Inputs:
    """Quantise a bf16 decode cache per KV head: scale = max |x| / 448 over the
    head's live tokens (amax scaling), codes = E4M3(x / scale).  Slots past a
    sequence's length hold the NaN code 0x7F."""
    assert inp.cfg.dtype == "bf16"
    B, Hkv, T, d = inp.k_cache.shape
    out = []
    for cache in (inp.k_cache, inp.v_cache):
        scales = np.empty(Hkv, dtype=np.float32)
        codes = np.empty((B, Hkv, T, d), dtype=np.uint8)
        for kv in range(Hkv):
            amax = 0.0
            for b in range(B):
                t = int(inp.seq_lens[b])
                if t:
                    amax = max(amax, float(np.max(np.abs(bf16_bits_to_f32(cache[b, kv, :t])))))
            scales[kv] = np.float32(amax / E4M3_MAX if amax > 0 else 1.0)
            for b in range(B):
                codes[b, kv] = f32_to_e4m3_bits(bf16_bits_to_f32(cache[b, kv]).astype(np.float64)
                                                / np.float64(scales[kv]))
                codes[b, kv, int(inp.seq_lens[b]):] = 0x7F
        out += [codes, scales]
    return Fp8Inputs(inp.cfg, inp.q, out[0], out[2], out[1], out[3], inp.seq_lens)


# ---------------------------------------------------------------------------
# Wide shared rows (absorbed-MLA decode)
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class WideInputs:
    cfg: WideConfig
    q: np.ndarray          # [B, Hq, d_k]          bf16 bits
    kv_cache: np.ndarray   # [B, Hkv, T_cap, d_k]  bf16 bits; value = first d_v columns
    seq_lens: np.ndarray   # [B] int32


def make_wide(cfg: WideConfig) -> WideInputs:
    """Streams (lengths, q, cache) of SeedSequence(seed).spawn(4); N(0,1)
    values rounded to bf16; cache rows past each length are NaN."""
    r_len, r_q, r_kv, _ = _streams(cfg.seed)
    if cfg.ragged:
        lens = r_len.integers(cfg.min_len, cfg.max_len, endpoint=True, size=cfg.batch).astype(np.int32)
    else:
        lens = np.full(cfg.batch, cfg.max_len, dtype=np.int32)
    q = _normals(r_q, (cfg.batch, cfg.num_q_heads, cfg.d_k), "bf16")
    kv = np.empty((cfg.batch, cfg.num_kv_heads, cfg.max_seq_len, cfg.d_k), dtype=np.uint16)
    for b in range(cfg.batch):
        kv[b] = _normals(r_kv, (cfg.num_kv_heads, cfg.max_seq_len, cfg.d_k), "bf16")
    poison_past_lengths(kv, lens, "bf16")
    return WideInputs(cfg, q, kv, lens)


def small_wide(batch: int, num_q_heads: int, num_kv_heads: int, d_k: int, d_v: int, seq_lens,
               max_seq_len: int, seed: int, scale_dim: int = 192) -> WideInputs:
    """Wide-row decode inputs of an arbitrary small shape (given lengths)."""
    lens = np.asarray(seq_lens, dtype=np.int32)
    cfg = WideConfig(f"small-wide-{seed}", batch, num_q_heads, num_kv_heads, d_k, d_v, max_seq_len,
                     int(lens.min()), int(lens.max()), seed, scale_dim)
    _, r_q, r_kv, _ = _streams(seed)
    q = _normals(r_q, (batch, num_q_heads, d_k), "bf16")
    kv = _normals(r_kv, (batch, num_kv_heads, max_seq_len, d_k), "bf16")
    poison_past_lengths(kv, lens, "bf16")
    return WideInputs(cfg, q, kv, lens)
