"""The C ABI without a GPU: the library loads, exports every declared entry
point, and rejects bad arguments with status codes before any HIP call."""
import ctypes
import os
import re

import pytest

import grouped_query_attention_gqa_amd as gqa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa.h")

OK, NULL, SHAPE, UNSUP, WS, HIP, ALIGN = 0, 1, 2, 3, 4, 5, 6
F32, BF16 = 0, 1
FAKE = ctypes.c_void_p(0x100000)        # aligned, never dereferenced: every call below fails validation
MISALIGNED = ctypes.c_void_p(0x100008)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return gqa.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"gqa_decode", "gqa_prefill_causal", "gqa_decode_plan", "gqa_decode_split",
            "gqa_decode_merge"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


# Every entry point of include/gqa.h.  The first group are the calls of the
# boundary as first specified (decode with a caller-sized workspace, causal
# prefill, the version and the status text); every other export is listed with
# the reason it exists, so a new export has to be added here knowingly.
BOUNDARY_CALLS = {"gqa_decode", "gqa_decode_workspace_bytes", "gqa_prefill_causal", "gqa_abi_version",
                  "gqa_status_str"}
EXTRA_CALLS = {
    "gqa_status_string": "status text taking the int32 the calls return (gqa_status_str takes the enum)",
    "gqa_last_hip_error": "text of the HIP error behind GQA_ERR_HIP",
    "gqa_device_info": "compute units and clock of the device, to derive the roofline peaks of the board measured",
    "gqa_decode_plan": "exact workspace for one (Hkv, dtype, range size), the grid and the range size",
    "gqa_decode_noalloc": "gqa_decode for callers that cannot allocate (library-owned per-GPU scratch)",
    "gqa_decode_split": "first decode stage alone (partials), the cut a sequence-parallel decode merges across",
    "gqa_decode_merge": "second decode stage alone (log-sum-exp merge of the partials)",
    "gqa_decode_paged": "decode over a paged cache (block table)",
    "gqa_decode_paged_split": "first stage of the paged decode",
    "gqa_decode_fp8": "decode over an E4M3 cache with per-KV-head scales",
    "gqa_decode_fp8_split": "first stage of the E4M3 decode",
    "gqa_decode_wide_plan": "workspace and ranges of the wide-row decode",
    "gqa_decode_wide": "decode over 576-column rows that are key and value (absorbed-MLA shape)",
    "gqa_prefill_backward_workspace": "workspace of the prefill backward",
    "gqa_prefill_causal_backward": "gradients of causal prefill",
}


def test_exports_match_the_boundary_table(lib):
    names = set(declared_functions())
    assert BOUNDARY_CALLS <= names
    assert names == BOUNDARY_CALLS | set(EXTRA_CALLS), sorted(names ^ (BOUNDARY_CALLS | set(EXTRA_CALLS)))


def test_status_str_matches_status_string(lib):
    for code in range(-1, 9):
        assert lib.gqa_status_str(code) == lib.gqa_status_string(code)


def test_workspace_bytes_cover_every_grouping():
    for (B, hq, d, tcap) in [(32, 32, 128, 8192), (64, 32, 128, 32768), (4, 16, 128, 131072),
                             (1, 8, 64, 256), (3, 71, 128, 320), (2, 12, 64, 1), (1, 128, 128, 65536),
                             (2, 96, 64, 4096)]:
        bound = gqa.gqa_decode_workspace_bytes(B, hq, d, tcap)
        assert bound > 0
        for hkv in [h for h in range(1, hq + 1) if hq % h == 0]:
            for dt in (F32, BF16, 2):
                assert gqa.gqa_decode_plan(B, hq, hkv, d, tcap, dt).workspace_bytes <= bound, (B, hq, hkv, d)
        assert max(gqa.gqa_decode_plan(B, hq, hkv, d, tcap, BF16).workspace_bytes
                   for hkv in range(1, hq + 1) if hq % hkv == 0) == bound


@pytest.mark.parametrize("args", [(0, 8, 64, 256), (1, 0, 64, 256), (1, 8, 96, 256), (1, 8, 64, 0)])
def test_workspace_bytes_zero_for_bad_arguments(args):
    assert gqa.gqa_decode_workspace_bytes(*args) == 0


def test_version_and_status_strings(lib):
    assert lib.gqa_abi_version() == 1
    for code, name in [(OK, b"GQA_OK"), (NULL, b"GQA_ERR_NULL"), (SHAPE, b"GQA_ERR_SHAPE"),
                       (UNSUP, b"GQA_ERR_UNSUPPORTED"), (WS, b"GQA_ERR_WORKSPACE"),
                       (HIP, b"GQA_ERR_HIP"), (ALIGN, b"GQA_ERR_ALIGN")]:
        assert lib.gqa_status_string(code) == name
    assert lib.gqa_status_string(99) == b"GQA_ERR_UNKNOWN"
    assert lib.gqa_last_hip_error() == b""


def test_device_info_rejects_null_outputs(lib):
    x = ctypes.c_int32(7)
    assert lib.gqa_device_info(0, None, ctypes.byref(x)) == NULL
    assert lib.gqa_device_info(0, ctypes.byref(x), None) == NULL
    assert x.value == 7   # checked before any HIP call; nothing written


def test_plan_auto_and_explicit():
    p = gqa.gqa_decode_plan(32, 32, 8, 128, 8192, BF16)
    assert p.range_tokens == 0 and p.workgroups == 512      # persistent grid, range size on device
    units = 32 * 8
    slots = p.workgroups + units                            # ranges + one extra piece per unit
    assert p.workspace_bytes >= units * 8 + slots * 16 * (128 + 1) * 4
    one = gqa.gqa_decode_plan(1, 8, 2, 64, 256, F32)
    assert one.workgroups == 2                              # 2 units x 256 tokens, 256-token minimum
    e = gqa.gqa_decode_plan(2, 4, 1, 64, 1000, BF16, split_tokens=128)
    assert e.range_tokens == 128 and e.workgroups == 16     # ceil(2 * 1000 / 128)
    # 71 query heads on one KV head: 5 blocks of 16 heads; a bf16 unit holds two
    # blocks (32 heads read one pass of K/V), so 3 units; fp32 keeps one block per unit
    big = gqa.gqa_decode_plan(1, 71, 1, 128, 4096, BF16, split_tokens=4096)
    assert big.workgroups == 3
    assert gqa.gqa_decode_plan(1, 71, 1, 128, 4096, F32, split_tokens=4096).workgroups == 5
    assert gqa.gqa_decode_plan(1, 32, 1, 128, 4096, BF16, split_tokens=4096).workgroups == 1
    assert gqa.gqa_decode_plan(1, 16, 1, 128, 4096, BF16, split_tokens=4096).workgroups == 1


@pytest.mark.parametrize("args,status", [
    ((1, 8, 3, 64, 256, BF16, 0), SHAPE),      # Hkv does not divide Hq
    ((1, 8, 0, 64, 256, BF16, 0), SHAPE),
    ((0, 8, 2, 64, 256, BF16, 0), SHAPE),
    ((1, 8, 2, 64, 0, BF16, 0), SHAPE),
    ((1, 8, 2, 96, 256, BF16, 0), UNSUP),      # head_dim
    ((1, 8, 2, 64, 256, 7, 0), UNSUP),         # dtype
    ((1, 8, 2, 64, 256, BF16, 100), UNSUP),    # range not a multiple of 32
    ((1, 8, 2, 64, 256, BF16, -64), UNSUP),
])
def test_plan_rejects(lib, args, status):
    assert lib.gqa_decode_plan(*args, None, None, None) == status


def _decode(lib, q=FAKE, k=FAKE, v=FAKE, lens=FAKE, out=FAKE, B=1, hq=8, hkv=2, d=64, tcap=256,
            dtype=BF16, split=0, ws=FAKE, ws_bytes=1 << 30):
    return lib.gqa_decode(q, k, v, lens, out, B, hq, hkv, d, tcap, 0.125, dtype, split, ws, ws_bytes, None)


def test_decode_validation(lib):
    assert _decode(lib, q=None) == NULL
    assert _decode(lib, lens=None) == NULL
    assert _decode(lib, out=None) == NULL
    assert _decode(lib, ws=None) == NULL
    assert _decode(lib, hkv=3) == SHAPE
    assert _decode(lib, B=0) == SHAPE
    assert _decode(lib, d=32) == UNSUP
    assert _decode(lib, dtype=5) == UNSUP
    assert _decode(lib, q=MISALIGNED) == ALIGN
    assert _decode(lib, out=MISALIGNED) == ALIGN
    assert _decode(lib, ws_bytes=16) == WS
    need = gqa.gqa_decode_plan(1, 8, 2, 64, 256, BF16).workspace_bytes
    assert _decode(lib, ws_bytes=need - 1) == WS


def _noalloc(lib, q=FAKE, k=FAKE, v=FAKE, lens=FAKE, out=FAKE, B=1, hq=8, hkv=2, d=64, tcap=256, dtype=BF16,
             split=0):
    return lib.gqa_decode_noalloc(q, k, v, lens, out, B, hq, hkv, d, tcap, 0.125, dtype, split, None)


def test_noalloc_validation(lib):
    """Argument errors of the allocation-free decode, all before any HIP call."""
    assert _noalloc(lib, q=None) == NULL
    assert _noalloc(lib, out=None) == NULL
    assert _noalloc(lib, hkv=3) == SHAPE
    assert _noalloc(lib, d=96) == UNSUP
    assert _noalloc(lib, dtype=2) == UNSUP             # E4M3 needs the scales of gqa_decode_fp8
    assert _noalloc(lib, k=MISALIGNED) == ALIGN
    # a shape whose workspace exceeds the library's 16 MiB scratch
    big = gqa.gqa_decode_plan(4096, 64, 64, 128, 65536, BF16).workspace_bytes
    assert big > 16 << 20
    assert _noalloc(lib, B=4096, hq=64, hkv=64, d=128, tcap=65536) == WS


def test_split_and_merge_validation(lib):
    assert lib.gqa_decode_split(FAKE, FAKE, None, FAKE, FAKE, 1, 8, 2, 64, 256, 0.1, BF16, 0, FAKE, 1 << 30, None) == NULL
    assert lib.gqa_decode_split(FAKE, FAKE, FAKE, FAKE, None, 1, 8, 2, 64, 256, 0.1, BF16, 0, FAKE, 1 << 30, None) == NULL
    assert lib.gqa_decode_split(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 64, 256, 0.1, BF16, 0, FAKE, 8, None) == WS
    assert lib.gqa_decode_merge(FAKE, None, 1, 8, 2, 64, 256, BF16, 0, FAKE, 1 << 30, None) == NULL
    assert lib.gqa_decode_merge(FAKE, FAKE, 1, 9, 2, 64, 256, BF16, 0, FAKE, 1 << 30, None) == SHAPE
    assert lib.gqa_decode_merge(FAKE, FAKE, 1, 8, 2, 64, 256, BF16, 0, FAKE, 8, None) == WS


def test_prefill_validation(lib):
    def call(q=FAKE, out=FAKE, lse=None, B=1, hq=8, hkv=2, n=128, d=128, dtype=BF16):
        return lib.gqa_prefill_causal(q, FAKE, FAKE, out, lse, B, hq, hkv, n, d, 0.1, dtype, None)
    assert call(q=None) == NULL
    assert call(out=None) == NULL
    assert call(hkv=3) == SHAPE
    assert call(n=0) == SHAPE
    assert call(d=80) == UNSUP
    assert call(dtype=F32) == UNSUP
    assert call(q=MISALIGNED) == ALIGN
    assert call(lse=ctypes.c_void_p(0x100002)) == ALIGN


def test_prefill_backward_validation(lib):
    ws_need = ctypes.c_int64()
    assert lib.gqa_prefill_backward_workspace(2, 8, 2, 100, 128, ctypes.byref(ws_need)) == OK
    assert ws_need.value == (2 * 8 * 100 * 8 + 255) // 256 * 256
    assert lib.gqa_prefill_backward_workspace(2, 8, 3, 100, 128, ctypes.byref(ws_need)) == SHAPE
    assert lib.gqa_prefill_backward_workspace(2, 8, 2, 100, 128, None) == NULL

    def call(q=FAKE, lse=FAKE, dout=FAKE, dk=FAKE, ws=FAKE, ws_bytes=1 << 20, B=1, hq=8, hkv=2, n=128,
             d=128, dtype=BF16):
        return lib.gqa_prefill_causal_backward(q, FAKE, FAKE, FAKE, lse, dout, FAKE, dk, FAKE, B, hq, hkv,
                                               n, d, 0.1, dtype, ws, ws_bytes, None)
    assert call(q=None) == NULL
    assert call(lse=None) == NULL
    assert call(dout=None) == NULL
    assert call(dk=None) == NULL
    assert call(ws=None) == NULL
    assert call(hkv=3) == SHAPE
    assert call(n=0) == SHAPE
    assert call(n=1 << 23) == SHAPE      # one head's rows would pass 2 GiB of buffer offsets
    assert call(d=96) == UNSUP
    assert call(dtype=F32) == UNSUP
    assert call(ws_bytes=8 * 128 * 8 - 1) == WS
    assert call(dout=MISALIGNED) == ALIGN
    assert call(ws=MISALIGNED) == ALIGN
    assert call(lse=ctypes.c_void_p(0x100002)) == ALIGN


def test_python_binding_raises_without_gpu_work():
    import torch
    q = torch.zeros(1, 8, 64)
    with pytest.raises(ValueError):
        gqa.gqa_decode(q, torch.zeros(1, 3, 16, 64), torch.zeros(1, 3, 16, 64),
                       torch.zeros(1, dtype=torch.int32))


def test_decode_wide_validation(lib):
    rng, nb = ctypes.c_int32(), ctypes.c_int64()
    assert lib.gqa_decode_wide_plan(64, 128, 1, 576, 512, 4096, 0, ctypes.byref(rng), ctypes.byref(nb)) == OK
    assert rng.value >= 2 and nb.value > 0
    assert lib.gqa_decode_wide_plan(512, 128, 1, 576, 512, 4096, 0, ctypes.byref(rng), ctypes.byref(nb)) == OK
    assert rng.value == 1 and nb.value == 0                       # enough units: one range, no merge
    assert lib.gqa_decode_wide_plan(2, 128, 1, 576, 512, 4096, 1024, ctypes.byref(rng), ctypes.byref(nb)) == OK
    assert rng.value == 4
    assert lib.gqa_decode_wide_plan(2, 128, 3, 576, 512, 64, 0, None, None) == SHAPE
    # 32-bit buffer offsets: rows up to max_seq_len + 64 (tiles loaded ahead) must stay below 2^31 bytes
    t_max = (2 ** 31 - 1) // 1152 - 64
    assert lib.gqa_decode_wide_plan(2, 128, 1, 576, 512, t_max, 0, None, None) == OK
    assert lib.gqa_decode_wide_plan(2, 128, 1, 576, 512, t_max + 1, 0, None, None) == SHAPE

    def call(q=FAKE, kv=FAKE, lens=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 30, B=2, hq=128, hkv=1, dk=576,
             dv=512, T=4096, split=0):
        return lib.gqa_decode_wide(q, kv, lens, out, B, hq, hkv, dk, dv, T, 0.07, split, ws, ws_bytes, None)
    assert call(q=None) == NULL
    assert call(lens=None) == NULL
    assert call(ws=None) == NULL              # this shape needs partials
    assert call(hkv=3) == SHAPE
    assert call(T=0) == SHAPE
    assert call(T=1 << 21) == SHAPE           # cache rows past 2 GiB of buffer offsets
    assert call(dk=512) == UNSUP
    assert call(dv=256) == UNSUP
    assert call(split=48) == UNSUP
    assert call(ws_bytes=1024) == WS
    assert call(out=MISALIGNED) == ALIGN
    assert call(lens=ctypes.c_void_p(0x100002)) == ALIGN
