"""paged_kv_split_attn_amd: paged-KV split-KV decode attention for MI355X (gfx950).

Thin ctypes binding over libpkv.so, whose C ABI is declared in include/pkv.h.
Each function here has the name of the C entry point it calls and only
marshals arguments: torch tensors supply device pointers, torch's current
stream supplies the hipStream_t.  Every step of the computation runs in the
library's HIP kernels; there is no Python or CPU fallback.  If the library is
missing or fails to load, the calls raise.

torch is imported before the library is loaded so that libpkv binds to the
HIP runtime torch already holds (both carry the soname libamdhip64.so.7).
"""

from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass
from typing import Optional

import torch

__all__ = [
    "PkvError",
    "Desc",
    "Pool",
    "library_path",
    "load_library",
    "declared_functions",
    "pkv_status_str",
    "pkv_version",
    "pkv_workspace_bytes",
    "pkv_build_metadata",
    "pkv_append_kv",
    "pkv_append_kv_ragged",
    "pkv_decode",
    "pkv_decode_append",
    "pkv_decode_plan",
    "pkv_decode_masked",
    "pkv_decode_tokens",
    "pkv_prefill",
    "pkv_decode_scratch",
    "pkv_debug_validate",
    "pkv_debug_read_ceiling",
    "WAVES_PER_GROUP",
    "SCRATCH_BYTES",
    "PKV_OK",
    "PKV_ERR_INVALID_ARG",
    "PKV_ERR_UNSUPPORTED",
    "PKV_ERR_WORKSPACE_TOO_SMALL",
    "PKV_ERR_CAPACITY",
    "PKV_ERR_LAUNCH",
    "PKV_ERR_DEVICE_DATA",
    "PKV_ERR_SCRATCH_TOO_SMALL",
]

PKV_OK = 0
PKV_ERR_INVALID_ARG = 1
PKV_ERR_UNSUPPORTED = 2
PKV_ERR_WORKSPACE_TOO_SMALL = 3
PKV_ERR_CAPACITY = 4
PKV_ERR_LAUNCH = 5
PKV_ERR_DEVICE_DATA = 6
PKV_ERR_SCRATCH_TOO_SMALL = 7
_PKG = os.path.dirname(os.path.abspath(__file__))
_HEADER = os.path.join(os.path.dirname(_PKG), "include", "pkv.h")


def _header_define(name: str) -> int:
    """Integer value of a #define in pkv.h (the header is the single source)."""
    with open(_HEADER) as f:
        m = re.search(rf"^#define\s+{name}\s+(\d+)", f.read(), re.M)
    if m is None:
        raise RuntimeError(f"{name} not defined in {_HEADER}")
    return int(m.group(1))


WAVES_PER_GROUP = _header_define("PKV_WAVES_PER_WORKGROUP")  # waves per decode workgroup


def library_path() -> str:
    return os.environ.get("PKV_LIBRARY", os.path.join(_PKG, "lib", "libpkv.so"))


class PkvError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


class _CPool(ctypes.Structure):
    _fields_ = [("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p)]


class _CDesc(ctypes.Structure):
    _fields_ = [("max_batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_workgroups", ctypes.c_int32),
                ("min_tiles_per_group", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_i32p = ctypes.POINTER(ctypes.c_int32)
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_SIGNATURES = {
    "pkv_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "pkv_version": (_i32, []),
    "pkv_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(_CDesc)]),
    "pkv_build_metadata": (ctypes.c_int, [ctypes.POINTER(_CDesc), _vp, _i32, _i32, _vp, _vp,
                                          ctypes.c_size_t, _vp]),
    "pkv_append_kv": (ctypes.c_int, [ctypes.POINTER(_CPool), _vp, _vp, _vp, _vp, _i32, _vp, _i32,
                                     _vp]),
    "pkv_append_kv_ragged": (ctypes.c_int, [ctypes.POINTER(_CPool), _vp, _vp, _vp, _vp, _vp, _i32,
                                            _vp, _i32, _i32, _vp]),
    "pkv_decode": (ctypes.c_int, [ctypes.POINTER(_CPool), ctypes.POINTER(_CDesc), _vp, _vp, _vp,
                                  _i32, _vp, _i32, ctypes.c_float, _vp, ctypes.c_size_t, _vp,
                                  _vp]),
    "pkv_decode_append": (ctypes.c_int, [ctypes.POINTER(_CPool), ctypes.POINTER(_CDesc), _vp, _vp,
                                         _vp, _vp, _vp, _i32, _vp, _i32, ctypes.c_float, _vp,
                                         ctypes.c_size_t, _vp, _vp]),
    "pkv_decode_plan": (ctypes.c_int, [ctypes.POINTER(_CPool), ctypes.POINTER(_CDesc), _vp, _vp,
                                       _vp, _vp, _i32, _i32, _vp, _vp, _i32, ctypes.c_float, _vp,
                                       ctypes.c_size_t, _vp, _vp]),
    "pkv_decode_masked": (ctypes.c_int, [ctypes.POINTER(_CPool), ctypes.POINTER(_CDesc), _vp, _vp,
                                         _i32, _vp, _vp, _i32, _vp, _i32, ctypes.c_float, _vp,
                                         ctypes.c_size_t, _vp, _vp]),
    "pkv_decode_tokens": (ctypes.c_int, [ctypes.POINTER(_CDesc), _vp, _vp, _i32, _vp, _i32, _vp,
                                         _vp, _vp, _i32, ctypes.c_float, _vp, ctypes.c_size_t,
                                         _vp, _vp]),
    "pkv_prefill": (ctypes.c_int, [ctypes.POINTER(_CPool), ctypes.POINTER(_CDesc), _vp, _vp, _vp,
                                   _vp, _i32, _vp, _i32, _i32, _i32, ctypes.c_float, _vp, _vp]),
    "pkv_decode_scratch": (ctypes.c_int, [ctypes.POINTER(_CPool), ctypes.POINTER(_CDesc), _vp, _vp,
                                          _vp, _i32, _i32, ctypes.c_float, _vp, _vp, _vp]),
    "pkv_debug_read_ceiling": (ctypes.c_int, [_vp, ctypes.c_size_t, _vp, ctypes.c_size_t, _vp]),
    "pkv_debug_validate": (ctypes.c_int, [ctypes.POINTER(_CDesc), _vp, _vp, _vp, _i32, _i32, _i32,
                                          _vp, ctypes.c_size_t, _i32p, _i32p, _vp]),
}

_lib: Optional[ctypes.CDLL] = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libpkv.so once and declare its signatures.  Raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or library_path()
    if not os.path.exists(p):
        raise RuntimeError(
            f"libpkv.so not found at {p}; build it with `python -m paged_kv_split_attn_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def declared_functions(header: str = _HEADER):
    """Names of the functions include/pkv.h declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_]+)\s*\(", text)))


def _check(fn: str, status: int) -> None:
    if status != PKV_OK:
        raise PkvError(fn, status, pkv_status_str(status))


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: torch.Tensor, name: str, dtypes=None, numel: Optional[int] = None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    return t.data_ptr()


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_I32 = (torch.int32,)


@dataclass
class Desc:
    """Fixed capacities and shapes (mirror of pkv_desc)."""

    max_batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_workgroups: int = 0
    min_tiles_per_group: int = 0

    def c(self) -> _CDesc:
        return _CDesc(self.max_batch, self.num_q_heads, self.num_kv_heads, self.head_dim,
                      self.page_size, self.num_workgroups, self.min_tiles_per_group, 0)

    def groups(self) -> int:
        """Decode grid size: num_workgroups, or the current device's compute units."""
        if self.num_workgroups > 0:
            return self.num_workgroups
        return torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count


@dataclass
class Pool:
    """One layer's pool: bf16 device tensors k [num_pages, Hkv, P/16, head_dim/8, 16, 8]
    and v [num_pages, Hkv, P/16, head_dim, 16] (the library's tile layouts: each
    16-token step of a page stored K in 8-channel blocks, V channel-major)."""

    k: torch.Tensor
    v: torch.Tensor

    def c(self) -> _CPool:
        if self.k.dim() != 6 or self.v.dim() != 5 or self.k.shape[4:] != (16, 8) or \
                self.v.shape[4] != 16:
            raise ValueError("k must be [num_pages, Hkv, P/16, head_dim/8, 16, 8] and v "
                             "[num_pages, Hkv, P/16, head_dim, 16]")
        n, h, s, d8 = self.k.shape[:4]
        if tuple(self.v.shape) != (n, h, s, d8 * 8, 16):
            raise ValueError("v must be [num_pages, Hkv, P/16, head_dim, 16] matching k")
        return _CPool(n, s * 16, h, d8 * 8, _ptr(self.k, "pool.k", _BF16),
                      _ptr(self.v, "pool.v", _BF16))


def pkv_status_str(status: int) -> str:
    return load_library().pkv_status_str(int(status)).decode()


def pkv_version() -> int:
    return int(load_library().pkv_version())


def pkv_workspace_bytes(desc: Desc) -> int:
    n = load_library().pkv_workspace_bytes(ctypes.byref(desc.c()))
    if n == 0:
        raise PkvError("pkv_workspace_bytes", PKV_ERR_INVALID_ARG, "invalid descriptor")
    return int(n)


def pkv_build_metadata(desc: Desc, seq_lens: torch.Tensor, forced_groups: int,
                       kv_indptr: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    B = seq_lens.numel()
    st = load_library().pkv_build_metadata(
        ctypes.byref(desc.c()), _ptr(seq_lens, "seq_lens", _I32), B, int(forced_groups),
        _ptr(kv_indptr, "kv_indptr", _I32, B + 1), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check("pkv_build_metadata", st)


def pkv_append_kv(pool: Pool, k_new: torch.Tensor, v_new: torch.Tensor, kv_indptr: torch.Tensor,
                  kv_indices: torch.Tensor, seq_lens: torch.Tensor, stream=None) -> None:
    B = seq_lens.numel()
    cp = pool.c()
    per = cp.num_kv_heads * cp.head_dim
    st = load_library().pkv_append_kv(
        ctypes.byref(cp), _ptr(k_new, "k_new", _BF16, B * per), _ptr(v_new, "v_new", _BF16, B * per),
        _ptr(kv_indptr, "kv_indptr", _I32, B + 1), _ptr(kv_indices, "kv_indices", _I32),
        kv_indices.numel(), _ptr(seq_lens, "seq_lens", _I32), B, _stream(stream))
    _check("pkv_append_kv", st)


def pkv_append_kv_ragged(pool: Pool, k_new: torch.Tensor, v_new: torch.Tensor,
                         qo_indptr: torch.Tensor, kv_indptr: torch.Tensor,
                         kv_indices: torch.Tensor, seq_lens: torch.Tensor, max_new_rows: int,
                         stream=None) -> None:
    """Append each request's new tokens (rows qo_indptr[b] .. qo_indptr[b+1] of
    k_new / v_new, [rows, Hkv, D]) at positions seq_len - n_b .. seq_len - 1."""
    B = seq_lens.numel()
    cp = pool.c()
    per = cp.num_kv_heads * cp.head_dim
    if k_new.numel() % per or v_new.numel() != k_new.numel():
        raise ValueError("k_new and v_new must be [rows, num_kv_heads, head_dim]")
    st = load_library().pkv_append_kv_ragged(
        ctypes.byref(cp), _ptr(k_new, "k_new", _BF16), _ptr(v_new, "v_new", _BF16),
        _ptr(qo_indptr, "qo_indptr", _I32, B + 1), _ptr(kv_indptr, "kv_indptr", _I32, B + 1),
        _ptr(kv_indices, "kv_indices", _I32), kv_indices.numel(),
        _ptr(seq_lens, "seq_lens", _I32), B, int(max_new_rows), _stream(stream))
    _check("pkv_append_kv_ragged", st)


def pkv_decode(pool: Pool, desc: Desc, q: torch.Tensor, kv_indptr: torch.Tensor,
               kv_indices: torch.Tensor, seq_lens: torch.Tensor, sm_scale: float,
               workspace: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    B = seq_lens.numel()
    n = B * desc.num_q_heads * desc.head_dim
    st = load_library().pkv_decode(
        ctypes.byref(pool.c()), ctypes.byref(desc.c()), _ptr(q, "q", _BF16, n),
        _ptr(kv_indptr, "kv_indptr", _I32, B + 1), _ptr(kv_indices, "kv_indices", _I32),
        kv_indices.numel(), _ptr(seq_lens, "seq_lens", _I32), B, float(sm_scale),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(out, "out", _BF16, n), _stream(stream))
    _check("pkv_decode", st)


def pkv_decode_append(pool: Pool, desc: Desc, q: torch.Tensor, k_new: torch.Tensor,
                      v_new: torch.Tensor, kv_indptr: torch.Tensor, kv_indices: torch.Tensor,
                      seq_lens: torch.Tensor, sm_scale: float, workspace: torch.Tensor,
                      out: torch.Tensor, stream=None) -> None:
    """pkv_append_kv followed by pkv_decode, in one launch."""
    B = seq_lens.numel()
    n = B * desc.num_q_heads * desc.head_dim
    nkv = B * desc.num_kv_heads * desc.head_dim
    st = load_library().pkv_decode_append(
        ctypes.byref(pool.c()), ctypes.byref(desc.c()), _ptr(q, "q", _BF16, n),
        _ptr(k_new, "k_new", _BF16, nkv), _ptr(v_new, "v_new", _BF16, nkv),
        _ptr(kv_indptr, "kv_indptr", _I32, B + 1), _ptr(kv_indices, "kv_indices", _I32),
        kv_indices.numel(), _ptr(seq_lens, "seq_lens", _I32), B, float(sm_scale),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(out, "out", _BF16, n), _stream(stream))
    _check("pkv_decode_append", st)


def pkv_decode_plan(pool: Pool, desc: Desc, q: torch.Tensor, k_new: Optional[torch.Tensor],
                    v_new: Optional[torch.Tensor], seq_lens: torch.Tensor, forced_groups: int,
                    kv_indptr: torch.Tensor, kv_indices: torch.Tensor, sm_scale: float,
                    workspace: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """pkv_build_metadata followed by pkv_decode_append (or pkv_decode when
    k_new and v_new are None), in one launch."""
    B = seq_lens.numel()
    n = B * desc.num_q_heads * desc.head_dim
    nkv = B * desc.num_kv_heads * desc.head_dim
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    kp = None if k_new is None else _ptr(k_new, "k_new", _BF16, nkv)
    vp = None if v_new is None else _ptr(v_new, "v_new", _BF16, nkv)
    st = load_library().pkv_decode_plan(
        ctypes.byref(pool.c()), ctypes.byref(desc.c()), _ptr(q, "q", _BF16, n), kp, vp,
        _ptr(seq_lens, "seq_lens", _I32), B, int(forced_groups),
        _ptr(kv_indptr, "kv_indptr", _I32, B + 1), _ptr(kv_indices, "kv_indices", _I32),
        kv_indices.numel(), float(sm_scale), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _ptr(out, "out", _BF16, n), _stream(stream))
    _check("pkv_decode_plan", st)


def pkv_decode_masked(pool: Pool, desc: Desc, q: torch.Tensor, mask: torch.Tensor,
                      kv_indptr: torch.Tensor, kv_indices: torch.Tensor, seq_lens: torch.Tensor,
                      sm_scale: float, workspace: torch.Tensor, out: torch.Tensor,
                      stream=None) -> None:
    """Decode with a keep mask: bool or uint8 [batch, S], S a multiple of 4."""
    B = seq_lens.numel()
    n = B * desc.num_q_heads * desc.head_dim
    if mask.dim() != 2 or mask.shape[0] != B:
        raise ValueError(f"mask must be [batch, S], got {tuple(mask.shape)}")
    st = load_library().pkv_decode_masked(
        ctypes.byref(pool.c()), ctypes.byref(desc.c()), _ptr(q, "q", _BF16, n),
        _ptr(mask, "mask", (torch.bool, torch.uint8)), int(mask.shape[1]),
        _ptr(kv_indptr, "kv_indptr", _I32, B + 1), _ptr(kv_indices, "kv_indices", _I32),
        kv_indices.numel(), _ptr(seq_lens, "seq_lens", _I32), B, float(sm_scale),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(out, "out", _BF16, n), _stream(stream))
    _check("pkv_decode_masked", st)


def pkv_decode_tokens(desc: Desc, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      slot_table: Optional[torch.Tensor], table_stride: int, q: torch.Tensor,
                      kv_indptr: torch.Tensor, seq_lens: torch.Tensor, sm_scale: float,
                      workspace: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """Decode over token-major K/V [num_slots, Hkv, D]: through slot_table
    [batch, table_stride] (int32), or contiguous (slot b * table_stride + t)
    when slot_table is None.  desc.page_size must be 16."""
    B = seq_lens.numel()
    n = B * desc.num_q_heads * desc.head_dim
    row = desc.num_kv_heads * desc.head_dim
    if k_cache.numel() % row or v_cache.numel() != k_cache.numel():
        raise ValueError("k_cache and v_cache must be [num_slots, num_kv_heads, head_dim]")
    table = 0
    if slot_table is not None:
        table = _ptr(slot_table, "slot_table", _I32, B * int(table_stride))
    st = load_library().pkv_decode_tokens(
        ctypes.byref(desc.c()), _ptr(k_cache, "k_cache", _BF16), _ptr(v_cache, "v_cache", _BF16),
        k_cache.numel() // row, table or None, int(table_stride), _ptr(q, "q", _BF16, n),
        _ptr(kv_indptr, "kv_indptr", _I32, B + 1), _ptr(seq_lens, "seq_lens", _I32), B,
        float(sm_scale), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _ptr(out, "out", _BF16, n), _stream(stream))
    _check("pkv_decode_tokens", st)


def pkv_prefill(pool: Pool, desc: Desc, q: torch.Tensor, qo_indptr: torch.Tensor,
                kv_indptr: torch.Tensor, kv_indices: torch.Tensor, seq_lens: torch.Tensor,
                max_q_len: int, causal: bool, sm_scale: float, out: torch.Tensor,
                stream=None) -> None:
    """Paged prefill / extend: q and out are [total_q, Hq, D]."""
    B = seq_lens.numel()
    n = q.numel()
    st = load_library().pkv_prefill(
        ctypes.byref(pool.c()), ctypes.byref(desc.c()), _ptr(q, "q", _BF16),
        _ptr(qo_indptr, "qo_indptr", _I32, B + 1), _ptr(kv_indptr, "kv_indptr", _I32, B + 1),
        _ptr(kv_indices, "kv_indices", _I32), kv_indices.numel(),
        _ptr(seq_lens, "seq_lens", _I32), B, int(max_q_len), int(bool(causal)), float(sm_scale),
        _ptr(out, "out", _BF16, n), _stream(stream))
    _check("pkv_prefill", st)


def pkv_decode_scratch(pool: Pool, desc: Desc, q: torch.Tensor, seq_lens: torch.Tensor,
                       kv_indices: torch.Tensor, sm_scale: float, kv_indptr: torch.Tensor,
                       out: torch.Tensor, stream=None) -> None:
    """pkv_build_metadata + pkv_decode with the library's static scratch as the
    workspace (no workspace argument, nothing allocated); writes kv_indptr."""
    B = seq_lens.numel()
    n = B * desc.num_q_heads * desc.head_dim
    st = load_library().pkv_decode_scratch(
        ctypes.byref(pool.c()), ctypes.byref(desc.c()), _ptr(q, "q", _BF16, n),
        _ptr(seq_lens, "seq_lens", _I32), _ptr(kv_indices, "kv_indices", _I32),
        kv_indices.numel(), B, float(sm_scale), _ptr(kv_indptr, "kv_indptr", _I32, B + 1),
        _ptr(out, "out", _BF16, n), _stream(stream))
    _check("pkv_decode_scratch", st)


def pkv_debug_validate(desc: Desc, seq_lens: torch.Tensor, kv_indptr: torch.Tensor,
                       kv_indices: torch.Tensor, num_pages: int, workspace: torch.Tensor,
                       stream=None) -> dict:
    """Synchronising check of device metadata; returns the status and the plan.

    ``waves`` lists {request, head group, first page, tiles} for every wave of
    the decode grid, ``groups`` the workgroups the plan uses.
    """
    B = seq_lens.numel()
    nw = desc.groups() * WAVES_PER_GROUP
    waves = (ctypes.c_int32 * (4 * nw))()
    groups = ctypes.c_int32(0)
    st = load_library().pkv_debug_validate(
        ctypes.byref(desc.c()), _ptr(seq_lens, "seq_lens", _I32),
        _ptr(kv_indptr, "kv_indptr", _I32, B + 1), _ptr(kv_indices, "kv_indices", _I32),
        kv_indices.numel(), int(num_pages), B, _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), ctypes.byref(groups), waves,
        _stream(stream))
    if st not in (PKV_OK, PKV_ERR_DEVICE_DATA):
        _check("pkv_debug_validate", st)
    w = [tuple(waves[4 * i: 4 * i + 4]) for i in range(nw)]
    return {"status": st, "groups": groups.value, "waves": w}


READ_CEILING_GROUPS = _header_define("PKV_READ_CEILING_GROUPS")
SCRATCH_BYTES = _header_define("PKV_SCRATCH_BYTES")  # static scratch of pkv_decode_scratch


def pkv_debug_read_ceiling(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """One read-only launch over src (a diagnostic of the achievable read rate);
    sink is uint32/int32 with at least READ_CEILING_GROUPS * 64 * WAVES_PER_GROUP
    elements."""
    nbytes = src.numel() * src.element_size()
    st = load_library().pkv_debug_read_ceiling(
        _ptr(src, "src"), nbytes, _ptr(sink, "sink", (torch.int32, torch.uint32)), sink.numel(),
        _stream(stream))
    _check("pkv_debug_read_ceiling", st)
