"""Pins of the FP8 (E4M3) cache oracle (oracle/fp8.py), written as functions of
the module so test_oracle_fp8.py can run them against broken copies too."""
import json
import os

import numpy as np

import gqa_inputs as gi
import oracle
from brute import brute_decode, e4m3_scalar

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "e4m3_codes.json")


def pin_e4m3_spec_values(f):
    """Code values and NaN codes of the OCP E4M3 definition."""
    g = json.load(open(GOLDEN))
    for code, val in g["codes"].items():
        assert f.e4m3_value(int(code, 16)) == val, code
    for code in g["nan_codes"]:
        assert np.isnan(f.e4m3_value(int(code, 16))), code


def pin_e4m3_all_codes_scalar(f):
    """Every one of the 256 codes against the scalar ldexp decoder."""
    got = f.e4m3_value(np.arange(256))
    for c in range(256):
        ref = e4m3_scalar(c)
        assert (np.isnan(ref) and np.isnan(got[c])) or got[c] == ref, hex(c)


def pin_e4m3_grid_structure(f):
    """Positive finite codes increase strictly, negative codes mirror them,
    and the generator's independent encoder inverts the decoder."""
    pos = f.e4m3_value(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0) and pos[-1] == 448.0
    assert np.array_equal(f.e4m3_value(np.arange(0x80, 0xFF)), -pos)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0x80, 0xFF)])
    assert np.array_equal(gi.f32_to_e4m3_bits(f.e4m3_value(codes)), codes)


def _tiny():
    inp = gi.small_decode("bf16", 2, 4, 2, 6, [5, 3], 6, seed=307)
    return gi.make_fp8(inp)


def pin_fp8_brute(f):
    """Tiny decode against the brute force on scalar-decoded, scaled values."""
    fp = _tiny()
    B, Hkv, T, d = fp.k_cache.shape
    kv = lambda codes, sc: [[[[e4m3_scalar(int(codes[b, h, t, i])) * float(sc[h]) for i in range(d)]
                              for t in range(T)] for h in range(Hkv)] for b in range(B)]
    q = gi.to_f64(fp.q, "bf16")
    ref = np.asarray(brute_decode(q.tolist(), kv(fp.k_cache, fp.k_scale), kv(fp.v_cache, fp.v_scale),
                                  fp.seq_lens.tolist(), 0.4))
    got = f.decode_fp8(q, fp.k_cache, fp.v_cache, fp.k_scale, fp.v_scale, fp.seq_lens, 0.4)
    assert np.max(np.abs(got - ref)) <= 1e-12


def pin_scale_homogeneity(f):
    """Doubling the V scales doubles the output exactly; scaling the K scales
    by c equals scaling the softmax scale by c."""
    fp = _tiny()
    q = gi.to_f64(fp.q, "bf16")
    a = f.decode_fp8(q, fp.k_cache, fp.v_cache, fp.k_scale, fp.v_scale, fp.seq_lens, 0.4)
    b = f.decode_fp8(q, fp.k_cache, fp.v_cache, fp.k_scale, fp.v_scale * 2, fp.seq_lens, 0.4)
    assert np.array_equal(b, 2 * a)
    c = f.decode_fp8(q, fp.k_cache, fp.v_cache, fp.k_scale.astype(np.float64) * 3, fp.v_scale, fp.seq_lens, 0.4)
    d = f.decode_fp8(q, fp.k_cache, fp.v_cache, fp.k_scale, fp.v_scale, fp.seq_lens, 1.2)
    assert np.allclose(c, d, rtol=0, atol=1e-12)


def pin_per_head_scales(f):
    """A scale belongs to one KV head: changing head 1's V scale leaves the
    query heads of KV head 0 unchanged and moves those of head 1."""
    fp = _tiny()
    q = gi.to_f64(fp.q, "bf16")
    a = f.decode_fp8(q, fp.k_cache, fp.v_cache, fp.k_scale, fp.v_scale, fp.seq_lens, 0.4)
    vs = fp.v_scale.copy()
    vs[1] *= 5
    b = f.decode_fp8(q, fp.k_cache, fp.v_cache, fp.k_scale, vs, fp.seq_lens, 0.4)
    assert np.array_equal(a[:, :2], b[:, :2]) and not np.allclose(a[:, 2:], b[:, 2:])


def pin_quantisation_error_bound(f):
    """Dequantised cache values lie within half a unit in the last place of
    the originals (2^-4 relative for normals, 2^-10 * scale absolute for
    subnormals)."""
    inp = gi.small_decode("bf16", 2, 4, 2, 16, [40, 17], 40, seed=311)
    fp = gi.make_fp8(inp)
    for b, t in enumerate(inp.seq_lens):
        x = gi.to_f64(inp.k_cache[b, :, :t], "bf16")
        y = f.dequantize(fp.k_cache[b:b + 1, :, :t], fp.k_scale)[0]
        sc = fp.k_scale.astype(np.float64)[:, None, None]
        assert np.all(np.abs(y - x) <= np.maximum(np.abs(x) * 2.0 ** -4, sc * 2.0 ** -10) * (1 + 1e-12))


FP8_PINS = [pin_e4m3_spec_values, pin_e4m3_all_codes_scalar, pin_e4m3_grid_structure, pin_fp8_brute,
            pin_scale_homogeneity, pin_per_head_scales, pin_quantisation_error_bound]
