"""Python binding of libgqa.so: grouped-query attention over a KV cache on
AMD Instinct MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/gqa.h.  PyTorch supplies device
memory and the current stream; nothing here computes attention, and there is
no fallback: if the library is missing, loading it raises.

Functions mirror the C entry points:

    gqa_decode(q, k_cache, v_cache, seq_lens, scale=None, ...)       -> out
    gqa_decode_split(...) / gqa_decode_merge(...)                    (two stages)
    gqa_decode_plan(batch, Hq, Hkv, d, max_seq_len, dtype, split)    -> Plan
    gqa_prefill_causal(q, k, v, scale=None, return_lse=False)        -> out[, lse]
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import NamedTuple, Optional

import torch

__all__ = [
    "GqaError", "Plan", "load_library", "library_path", "gqa_abi_version", "gqa_device_info",
    "gqa_decode_plan", "gqa_decode_workspace_bytes", "decode_workspace", "gqa_decode", "gqa_decode_noalloc", "gqa_decode_split",
    "gqa_decode_merge",
    "gqa_prefill_causal", "gqa_prefill_backward_workspace", "gqa_prefill_causal_backward",
    "gqa_decode_wide_plan", "gqa_decode_wide",
    "GQA_F32", "GQA_BF16",
]

HERE = os.path.dirname(os.path.abspath(__file__))
GQA_F32, GQA_BF16 = 0, 1
GQA_FP8_E4M3 = 2   # bf16 q with an E4M3-coded cache and per-KV-head scales
_STATUS = {0: "GQA_OK", 1: "GQA_ERR_NULL", 2: "GQA_ERR_SHAPE", 3: "GQA_ERR_UNSUPPORTED",
           4: "GQA_ERR_WORKSPACE", 5: "GQA_ERR_HIP", 6: "GQA_ERR_ALIGN"}

_lib = None


class GqaError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str = ""):
        self.status = status
        msg = f"{fn} failed with {_STATUS.get(status, status)}"
        super().__init__(msg + (f": {detail}" if detail else ""))


class Plan(NamedTuple):
    range_tokens: int      # fixed range size, 0 = chosen on the device
    workgroups: int        # workgroups the split kernel launches
    workspace_bytes: int


def library_path() -> str:
    return os.environ.get("GQA_LIBRARY", os.path.join(HERE, "libgqa.so"))


def load_library():
    """Load libgqa.so (built by grouped_query_attention_gqa_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m grouped_query_attention_gqa_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.gqa_abi_version.restype = I32
    lib.gqa_status_string.restype = ctypes.c_char_p
    lib.gqa_status_string.argtypes = [I32]
    lib.gqa_status_str.restype = ctypes.c_char_p
    lib.gqa_status_str.argtypes = [ctypes.c_int]
    lib.gqa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.gqa_decode_workspace_bytes.argtypes = [I32] * 4
    lib.gqa_last_hip_error.restype = ctypes.c_char_p
    lib.gqa_device_info.restype = I32
    lib.gqa_device_info.argtypes = [I32, ctypes.POINTER(I32), ctypes.POINTER(I32)]
    lib.gqa_decode_plan.restype = I32
    lib.gqa_decode_plan.argtypes = [I32] * 7 + [ctypes.POINTER(I32), ctypes.POINTER(I32),
                                                ctypes.POINTER(I64)]
    lib.gqa_decode.restype = I32
    lib.gqa_decode.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32, F32, I32, I32, P, I64, P]
    lib.gqa_decode_noalloc.restype = I32
    lib.gqa_decode_noalloc.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32, F32, I32, I32, P]
    lib.gqa_decode_split.restype = I32
    lib.gqa_decode_split.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32, F32, I32, I32, P, I64, P]
    lib.gqa_decode_merge.restype = I32
    lib.gqa_decode_merge.argtypes = [P, P, I32, I32, I32, I32, I32, I32, I32, P, I64, P]
    lib.gqa_decode_paged.restype = I32
    lib.gqa_decode_paged.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, F32, I32, I32,
                                     P, I64, P]
    lib.gqa_decode_paged_split.restype = I32
    lib.gqa_decode_paged_split.argtypes = lib.gqa_decode_paged.argtypes
    lib.gqa_decode_fp8.restype = I32
    lib.gqa_decode_fp8.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, F32, I32, P, I64, P]
    lib.gqa_decode_fp8_split.restype = I32
    lib.gqa_decode_fp8_split.argtypes = lib.gqa_decode_fp8.argtypes
    lib.gqa_prefill_causal.restype = I32
    lib.gqa_prefill_causal.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32, F32, I32, P]
    lib.gqa_decode_wide_plan.restype = I32
    lib.gqa_decode_wide_plan.argtypes = [I32] * 7 + [ctypes.POINTER(I32), ctypes.POINTER(I64)]
    lib.gqa_decode_wide.restype = I32
    lib.gqa_decode_wide.argtypes = [P, P, P, P] + [I32] * 6 + [F32, I32, P, I64, P]
    lib.gqa_prefill_backward_workspace.restype = I32
    lib.gqa_prefill_backward_workspace.argtypes = [I32] * 5 + [ctypes.POINTER(I64)]
    lib.gqa_prefill_causal_backward.restype = I32
    lib.gqa_prefill_causal_backward.argtypes = [P] * 9 + [I32] * 5 + [F32, I32, P, I64, P]
    _lib = lib
    return lib


def gqa_abi_version() -> int:
    return load_library().gqa_abi_version()


def gqa_device_info(device: int = 0):
    """(compute units, peak shader clock in kHz) of a HIP device."""
    cus, khz = ctypes.c_int32(0), ctypes.c_int32(0)
    _check("gqa_device_info", load_library().gqa_device_info(device, ctypes.byref(cus), ctypes.byref(khz)))
    return cus.value, khz.value


def _check(fn: str, status: int):
    if status != 0:
        lib = load_library()
        detail = lib.gqa_last_hip_error().decode() if status == 5 else ""
        if status in (1, 2, 3, 4, 6):
            raise ValueError(str(GqaError(fn, status, detail)))
        raise GqaError(fn, status, detail)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GQA_BF16
    if t.dtype == torch.float32:
        return GQA_F32
    raise ValueError(f"unsupported dtype {t.dtype}: expected torch.bfloat16 or torch.float32")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _on_gpu(*tensors: torch.Tensor):
    dev = tensors[0].device
    for t in tensors:
        _require(t.is_cuda and t.device == dev, "all tensors must be on the same GPU device")
        _require(t.is_contiguous(), "all tensors must be contiguous")
    return dev


def gqa_decode_plan(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                    max_seq_len: int, dtype: int, split_tokens: int = 0) -> Plan:
    lib = load_library()
    c, n, w = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    _check("gqa_decode_plan", lib.gqa_decode_plan(batch, num_q_heads, num_kv_heads, head_dim,
                                                  max_seq_len, dtype, split_tokens,
                                                  ctypes.byref(c), ctypes.byref(n), ctypes.byref(w)))
    return Plan(c.value, n.value, w.value)


def gqa_decode_workspace_bytes(batch: int, num_q_heads: int, head_dim: int, max_seq_len: int) -> int:
    """Decode workspace bytes that serve every KV-head count dividing
    ``num_q_heads`` with automatic ranges (0 for invalid arguments)."""
    return int(load_library().gqa_decode_workspace_bytes(batch, num_q_heads, head_dim, max_seq_len))


def _decode_args(q, k_cache, v_cache, seq_lens):
    _require(q.dim() == 3 and k_cache.dim() == 4 and v_cache.dim() == 4,
             "expected q [B,Hq,d] and k_cache/v_cache [B,Hkv,T_cap,d]")
    _require(k_cache.shape == v_cache.shape, "k_cache and v_cache shapes differ")
    B, Hq, d = q.shape
    B2, Hkv, tcap, d2 = k_cache.shape
    _require(B == B2 and d == d2, "q and cache disagree on batch or head_dim")
    _require(q.dtype == k_cache.dtype == v_cache.dtype, "q, k_cache, v_cache must share a dtype")
    _require(seq_lens.dtype == torch.int32 and seq_lens.shape == (B,), "seq_lens must be int32 [B]")
    dev = _on_gpu(q, k_cache, v_cache, seq_lens)
    return dev, B, Hq, Hkv, tcap, d, _dtype_code(q)


def decode_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A device workspace of ``nbytes`` for the decode entry points (its
    contents on entry do not matter)."""
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def _workspace(workspace, plan: Plan, dev):
    if workspace is None:
        return decode_workspace(plan.workspace_bytes, dev)
    _require(workspace.is_cuda and workspace.device == dev and workspace.is_contiguous(),
             "workspace must be a contiguous tensor on the same device")
    return workspace


def gqa_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
               seq_lens: torch.Tensor, scale: Optional[float] = None,
               out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
               split_tokens: int = 0) -> torch.Tensor:
    """One GQA decode step; returns out [B, Hq, d] float32 (see gqa.h)."""
    dev, B, Hq, Hkv, tcap, d, dt = _decode_args(q, k_cache, v_cache, seq_lens)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    plan = gqa_decode_plan(B, Hq, Hkv, d, tcap, dt, split_tokens)
    ws = _workspace(workspace, plan, dev)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    _require(out.dtype == torch.float32 and out.shape == (B, Hq, d), "out must be float32 [B,Hq,d]")
    _on_gpu(q, out)
    lib = load_library()
    _check("gqa_decode", lib.gqa_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                                        _ptr(out), B, Hq, Hkv, d, tcap, scale, dt, split_tokens,
                                        _ptr(ws), ws.numel(), _stream(dev)))
    return out


def gqa_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                       seq_lens: torch.Tensor, out: torch.Tensor, scale: Optional[float] = None,
                       split_tokens: int = 0) -> torch.Tensor:
    """gqa_decode with the library's own per-GPU scratch instead of a
    workspace: the C call allocates nothing (``out`` is the caller's)."""
    dev, B, Hq, Hkv, tcap, d, dt = _decode_args(q, k_cache, v_cache, seq_lens)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _require(out.dtype == torch.float32 and out.shape == (B, Hq, d), "out must be float32 [B,Hq,d]")
    _on_gpu(q, out)
    lib = load_library()
    _check("gqa_decode_noalloc", lib.gqa_decode_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(out), B, Hq, Hkv, d, tcap, scale, dt,
        split_tokens, _stream(dev)))
    return out


def _paged_args(q, k_pages, v_pages, block_table, seq_lens):
    _require(q.dim() == 3 and k_pages.dim() == 4 and k_pages.shape == v_pages.shape,
             "expected q [B,Hq,d] and k/v pages [num_pages,Hkv,page_size,d]")
    _require(block_table.dim() == 2 and block_table.dtype == torch.int32,
             "block_table must be int32 [B, max_pages]")
    _require(seq_lens.dtype == torch.int32 and seq_lens.dim() == 1, "seq_lens must be int32 [B]")
    B, Hq, d = q.shape
    num_pages, Hkv, page_size, d2 = k_pages.shape
    _require(d == d2 and block_table.shape[0] == B and seq_lens.shape[0] == B, "shape mismatch")
    _require(q.dtype == k_pages.dtype == v_pages.dtype, "q and the pages must share a dtype")
    dev = _on_gpu(q, k_pages, v_pages, block_table, seq_lens)
    return dev, B, Hq, Hkv, d, num_pages, page_size, block_table.shape[1], _dtype_code(q)


def gqa_decode_paged(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                     block_table: torch.Tensor, seq_lens: torch.Tensor, scale: Optional[float] = None,
                     out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     split_tokens: int = 0, stage: str = "both") -> torch.Tensor:
    """One GQA decode step over a paged cache; returns out [B, Hq, d] float32.

    k_pages, v_pages: [num_pages, Hkv, page_size, d] bf16; block_table:
    [B, max_pages] int32 (see gqa.h).  stage="split" runs only the first
    stage (gqa_decode_paged_split); gqa_decode_merge with max_seq_len =
    max_pages * page_size completes it."""
    dev, B, Hq, Hkv, d, num_pages, page_size, max_pages, dt = _paged_args(q, k_pages, v_pages, block_table,
                                                                         seq_lens)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    plan = gqa_decode_plan(B, Hq, Hkv, d, max_pages * page_size, dt, split_tokens)
    ws = _workspace(workspace, plan, dev)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    _require(out.dtype == torch.float32 and out.shape == (B, Hq, d), "out must be float32 [B,Hq,d]")
    _on_gpu(q, out)
    _require(stage in ("both", "split"), "stage must be 'both' or 'split'")
    lib = load_library()
    fn = lib.gqa_decode_paged if stage == "both" else lib.gqa_decode_paged_split
    _check("gqa_decode_paged" if stage == "both" else "gqa_decode_paged_split", fn(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seq_lens), _ptr(out), B, Hq, Hkv, d,
        page_size, num_pages, max_pages, scale, dt, split_tokens, _ptr(ws), ws.numel(), _stream(dev)))
    return out


def gqa_decode_fp8(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: torch.Tensor,
                   v_scale: torch.Tensor, seq_lens: torch.Tensor, scale: Optional[float] = None,
                   out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                   split_tokens: int = 0, stage: str = "both") -> torch.Tensor:
    """One GQA decode step over an E4M3 cache; returns out [B, Hq, d] float32.

    q [B, Hq, d] bf16; k_cache, v_cache [B, Hkv, T_cap, d] uint8 codes;
    k_scale, v_scale [Hkv] float32 (see gqa.h).  stage="split" runs only
    gqa_decode_fp8_split (complete it with gqa_decode_merge, dtype
    GQA_FP8_E4M3)."""
    _require(q.dim() == 3 and q.dtype == torch.bfloat16, "q must be bf16 [B,Hq,d]")
    _require(k_cache.dim() == 4 and k_cache.shape == v_cache.shape and k_cache.dtype == torch.uint8
             and v_cache.dtype == torch.uint8, "k_cache/v_cache must be uint8 [B,Hkv,T_cap,d] codes")
    B, Hq, d = q.shape
    B2, Hkv, tcap, d2 = k_cache.shape
    _require(B == B2 and d == d2, "q and cache disagree on batch or head_dim")
    _require(k_scale.dtype == torch.float32 and v_scale.dtype == torch.float32 and k_scale.shape == (Hkv,)
             and v_scale.shape == (Hkv,), "k_scale/v_scale must be float32 [Hkv]")
    _require(seq_lens.dtype == torch.int32 and seq_lens.shape == (B,), "seq_lens must be int32 [B]")
    dev = _on_gpu(q, k_cache, v_cache, k_scale, v_scale, seq_lens)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    plan = gqa_decode_plan(B, Hq, Hkv, d, tcap, GQA_FP8_E4M3, split_tokens)
    ws = _workspace(workspace, plan, dev)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    _require(out.dtype == torch.float32 and out.shape == (B, Hq, d), "out must be float32 [B,Hq,d]")
    _on_gpu(q, out)
    _require(stage in ("both", "split"), "stage must be 'both' or 'split'")
    lib = load_library()
    fn, name = (lib.gqa_decode_fp8, "gqa_decode_fp8") if stage == "both" else \
        (lib.gqa_decode_fp8_split, "gqa_decode_fp8_split")
    _check(name, fn(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(seq_lens),
                    _ptr(out), B, Hq, Hkv, d, tcap, scale, split_tokens, _ptr(ws), ws.numel(), _stream(dev)))
    return out


def gqa_decode_split(q, k_cache, v_cache, seq_lens, out, workspace, scale=None, split_tokens=0):
    """Stage 1 of decode: final rows of single-range sequences into ``out``,
    partials of the others into ``workspace`` (uint8 tensor)."""
    dev, B, Hq, Hkv, tcap, d, dt = _decode_args(q, k_cache, v_cache, seq_lens)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _workspace(workspace, Plan(0, 0, 0), dev)
    _require(out.dtype == torch.float32 and out.shape == (B, Hq, d), "out must be float32 [B,Hq,d]")
    _on_gpu(q, out)
    lib = load_library()
    _check("gqa_decode_split", lib.gqa_decode_split(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(out), B, Hq, Hkv, d, tcap,
        scale, dt, split_tokens, _ptr(workspace), workspace.numel(), _stream(dev)))
    return out


def gqa_decode_merge(seq_lens, out, workspace, num_kv_heads, max_seq_len, dtype, split_tokens=0):
    """Stage 2 of decode: merge the partials in ``workspace`` into ``out``."""
    dev = _on_gpu(seq_lens, out, workspace)
    B, Hq, d = out.shape
    _require(out.dtype == torch.float32, "out must be float32")
    lib = load_library()
    _check("gqa_decode_merge", lib.gqa_decode_merge(
        _ptr(seq_lens), _ptr(out), B, Hq, num_kv_heads, d, max_seq_len, dtype, split_tokens,
        _ptr(workspace), workspace.numel(), _stream(dev)))
    return out


def gqa_prefill_causal(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                       scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                       return_lse: bool = False, lse: Optional[torch.Tensor] = None):
    """Causal GQA prefill; returns out [B, Hq, N, d] float32 (and lse)."""
    _require(q.dim() == 4 and k.dim() == 4 and v.dim() == 4, "expected 4-d q, k, v")
    _require(k.shape == v.shape, "k and v shapes differ")
    B, Hq, N, d = q.shape
    B2, Hkv, N2, d2 = k.shape
    _require(B == B2 and N == N2 and d == d2, "q and k/v disagree on batch, length or head_dim")
    _require(q.dtype == k.dtype == v.dtype, "q, k, v must share a dtype")
    dev = _on_gpu(q, k, v)
    dt = _dtype_code(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    if lse is not None:
        _require(lse.dtype == torch.float32 and lse.shape == (B, Hq, N), "lse must be float32 [B,Hq,N]")
        _on_gpu(q, lse)
    _require(out.dtype == torch.float32 and out.shape == (B, Hq, N, d), "out must be float32 [B,Hq,N,d]")
    _on_gpu(q, out)
    lib = load_library()
    _check("gqa_prefill_causal", lib.gqa_prefill_causal(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, N, d, scale, dt, _stream(dev)))
    return (out, lse) if (return_lse or lse is not None) else out


def gqa_prefill_backward_workspace(batch: int, num_q_heads: int, num_kv_heads: int, seq_len: int,
                                   head_dim: int) -> int:
    """Workspace bytes of ``gqa_prefill_causal_backward`` for this shape."""
    lib = load_library()
    nbytes = ctypes.c_int64()
    _check("gqa_prefill_backward_workspace", lib.gqa_prefill_backward_workspace(
        batch, num_q_heads, num_kv_heads, seq_len, head_dim, ctypes.byref(nbytes)))
    return nbytes.value


def gqa_prefill_causal_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                                lse: torch.Tensor, dout: torch.Tensor, scale: Optional[float] = None,
                                workspace: Optional[torch.Tensor] = None, grads=None):
    """Gradients (dq, dk, dv) of causal GQA prefill, all float32 (see gqa.h).

    ``out`` and ``lse`` are what ``gqa_prefill_causal`` returned for these
    q, k, v and scale; ``dout`` [B, Hq, N, d] bf16 is the gradient of the
    loss with respect to ``out``.  ``grads`` may supply the three output
    tensors."""
    _require(q.dim() == 4 and k.dim() == 4 and v.dim() == 4, "expected 4-d q, k, v")
    _require(k.shape == v.shape, "k and v shapes differ")
    B, Hq, N, d = q.shape
    B2, Hkv, N2, d2 = k.shape
    _require(B == B2 and N == N2 and d == d2, "q and k/v disagree on batch, length or head_dim")
    _require(q.dtype == k.dtype == v.dtype == dout.dtype, "q, k, v, dout must share a dtype")
    _require(dout.shape == q.shape, "dout must have q's shape")
    _require(out.dtype == torch.float32 and out.shape == q.shape, "out must be float32 [B,Hq,N,d]")
    _require(lse.dtype == torch.float32 and lse.shape == (B, Hq, N), "lse must be float32 [B,Hq,N]")
    dev = _on_gpu(q, k, v, out, lse, dout)
    dt = _dtype_code(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if grads is None:
        grads = (torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev),
                 torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev),
                 torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev))
    dq, dk, dv = grads
    _require(dq.dtype == torch.float32 and dq.shape == q.shape, "dq must be float32 [B,Hq,N,d]")
    _require(dk.dtype == torch.float32 and dk.shape == k.shape, "dk must be float32 [B,Hkv,N,d]")
    _require(dv.dtype == torch.float32 and dv.shape == k.shape, "dv must be float32 [B,Hkv,N,d]")
    _on_gpu(q, dq, dk, dv)
    if workspace is None:
        nbytes = gqa_prefill_backward_workspace(B, Hq, Hkv, N, d) if dt == GQA_BF16 else 256
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _on_gpu(q, workspace)
    lib = load_library()
    _check("gqa_prefill_causal_backward", lib.gqa_prefill_causal_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        B, Hq, Hkv, N, d, scale, dt, _ptr(workspace), workspace.numel(), _stream(dev)))
    return dq, dk, dv


def gqa_decode_wide_plan(batch: int, num_q_heads: int, num_kv_heads: int, max_seq_len: int,
                         head_dim_qk: int = 576, head_dim_v: int = 512, split_tokens: int = 0):
    """(token ranges per sequence, workspace bytes) of ``gqa_decode_wide``."""
    lib = load_library()
    rng, nbytes = ctypes.c_int32(), ctypes.c_int64()
    _check("gqa_decode_wide_plan", lib.gqa_decode_wide_plan(
        batch, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, max_seq_len, split_tokens,
        ctypes.byref(rng), ctypes.byref(nbytes)))
    return rng.value, nbytes.value


def gqa_decode_wide(q: torch.Tensor, kv_cache: torch.Tensor, seq_lens: torch.Tensor, head_dim_v: int = 512,
                    scale: Optional[float] = None, split_tokens: int = 0,
                    out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Decode over cached rows that are key and (leading head_dim_v columns)
    value, the absorbed-MLA shape; returns out [B, Hq, head_dim_v] float32.
    ``scale`` defaults to 1/sqrt(192), the per-head query/key width of the
    MLA layer before absorption (128 + 64)."""
    _require(q.dim() == 3 and kv_cache.dim() == 4, "expected q [B,Hq,dk] and kv_cache [B,Hkv,T,dk]")
    B, Hq, dk = q.shape
    B2, Hkv, T, dk2 = kv_cache.shape
    _require(B == B2 and dk == dk2, "q and kv_cache disagree on batch or head_dim_qk")
    _require(q.dtype == kv_cache.dtype == torch.bfloat16, "q and kv_cache must be bfloat16")
    _require(seq_lens.dtype == torch.int32 and seq_lens.shape == (B,), "seq_lens must be int32 [B]")
    dev = _on_gpu(q, kv_cache, seq_lens)
    scale = 1.0 / math.sqrt(192.0) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, Hq, head_dim_v), dtype=torch.float32, device=dev)
    _require(out.dtype == torch.float32 and out.shape == (B, Hq, head_dim_v), "out must be float32 [B,Hq,dv]")
    _on_gpu(q, out)
    if workspace is None:
        _, nbytes = gqa_decode_wide_plan(B, Hq, Hkv, T, dk, head_dim_v, split_tokens)
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    _on_gpu(q, workspace)
    lib = load_library()
    _check("gqa_decode_wide", lib.gqa_decode_wide(
        _ptr(q), _ptr(kv_cache), _ptr(seq_lens), _ptr(out), B, Hq, Hkv, dk, head_dim_v, T, scale,
        split_tokens, _ptr(workspace), workspace.numel(), _stream(dev)))
    return out
