"""Python binding of libhta (include/hta.h): argument marshalling only.

Every function here has the name of the C entry point it calls. Tensors are
torch tensors already on the GPU; the binding checks dtype, shape, device
and contiguity, passes ``data_ptr()`` values and the stream handle, and
turns a negative return code into :class:`HtaError`. All the arithmetic runs
in the HIP kernels of ``libhta.so``; if that library is missing the import
of any entry point fails loudly (build it with ``__graft_entry__.build()``).
"""

from __future__ import annotations

import ctypes
import math
import os
import re
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhta.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "hta.h")

HTA_OK = 0
HTA_ERR_INVALID_ARG = -1
HTA_ERR_UNSUPPORTED = -2
HTA_ERR_NO_MEMORY = -3
HTA_ERR_HIP = -4
HTA_ERR_BAD_TREE = -5
HTA_ERR_BAD_PREFIX = -6
HTA_ERR_NO_DEVICE = -7
HTA_ERR_TOO_LARGE = -8
HTA_NOALLOC_SCRATCH_BYTES = 32 << 20

HTA_F32 = 0
HTA_BF16 = 1

HTA_STATUS_BAD_TREE = 1
HTA_STATUS_BAD_PREFIX = 2
HTA_STATUS_COMMIT_OVERFLOW = 4
HTA_STATUS_BAD_PATH = 8
HTA_STATUS_MERGE_TIMEOUT = 16

HTA_PATH_AUTO = 0
HTA_PATH_MFMA = 1
HTA_PATH_VALU = 2
HTA_PATH_DOT = 3


class HtaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {hta_status_string(code)} ({code})")


class HtaConfig(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("tree_nodes", ctypes.c_int32),
        ("kv_capacity", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("num_workgroups", ctypes.c_int32),
        ("force_path", ctypes.c_int32),
        ("qblocks_per_wave", ctypes.c_int32),
        ("fuse_merge", ctypes.c_int32),
    ]


HTA_MAX_TREE_GUESSES = 31
HTA_MAX_NGRAM = 8


class HtaTreeParams(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_int32),
        ("m", ctypes.c_int32),
        ("keep_first", ctypes.c_int32),
        ("keep", ctypes.c_int32 * HTA_MAX_TREE_GUESSES),
    ]


def make_tree_params(k: int, m: int, keep_first: int, keep) -> HtaTreeParams:
    p = HtaTreeParams(k=k, m=m, keep_first=keep_first)
    for r, v in enumerate(keep):
        p.keep[r] = int(v)
    return p


class HtaPlan(ctypes.Structure):
    _fields_ = [
        ("path", ctypes.c_int32),
        ("num_workgroups", ctypes.c_int32),
        ("row_groups", ctypes.c_int32),
        ("rows_per_group", ctypes.c_int32),
        ("waves_per_workgroup", ctypes.c_int32),
        ("qblocks_per_wave", ctypes.c_int32),
        ("tile_tokens", ctypes.c_int32),
        ("max_slots", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_int64),
        ("device", ctypes.c_int32),
        ("compute_units", ctypes.c_int32),
    ]


_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_SIGNATURES = {
    "hta_validate_config": (ctypes.c_int, [ctypes.POINTER(HtaConfig)]),
    "hta_create": (ctypes.c_int, [ctypes.POINTER(_vp), ctypes.POINTER(HtaConfig)]),
    "hta_destroy": (ctypes.c_int, [_vp]),
    "hta_get_plan": (ctypes.c_int, [_vp, ctypes.POINTER(HtaPlan)]),
    "hta_verify_attn": (ctypes.c_int, [_vp] + [_vp] * 9 + [_vp]),
    "hta_tree_mask": (ctypes.c_int, [_vp, _vp, _vp, _vp]),
    "hta_tree_attn": (ctypes.c_int, [_vp] * 7 + [_vp]),
    "hta_prefix_attn": (ctypes.c_int, [_vp] * 7 + [_vp]),
    "hta_cross_attn": (ctypes.c_int, [_vp] * 7 + [_vp]),
    "hta_window_attn": (ctypes.c_int, [_vp] * 9 + [_vp]),
    "hta_build_tree": (ctypes.c_int, [_vp, _vp, _i32, _i32, _vp, _i32, _vp, ctypes.POINTER(HtaTreeParams)]
                       + [_vp] * 3 + [_vp]),
    "hta_window_append": (ctypes.c_int, [_vp] * 6 + [_vp]),
    "hta_ngram_index_create": (ctypes.c_int, [ctypes.POINTER(_vp), _i32, _i32, _i32]),
    "hta_ngram_index_destroy": (ctypes.c_int, [_vp]),
    "hta_ngram_index_reset": (ctypes.c_int, [_vp, _i32, _vp]),
    "hta_build_tree_indexed": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _vp, _vp, ctypes.POINTER(HtaTreeParams)]
                               + [_vp] * 3 + [_vp]),
    "hta_prefix_partials": (ctypes.c_int, [_vp] * 5 + [_vp]),
    "hta_merge_prefix": (ctypes.c_int, [_vp] * 4 + [_vp]),
    "hta_lse_merge": (ctypes.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _vp]),
    "hta_accept": (ctypes.c_int, [_vp, _vp, _i32, _i32] + [_vp] * 6 + [_vp]),
    "hta_commit": (ctypes.c_int, [_vp] * 8 + [_vp]),
    "hta_get_status": (ctypes.c_int, [_vp, _vp, ctypes.POINTER(_i32)]),
    "hta_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "hta_verify_attn_noalloc": (ctypes.c_int, [ctypes.POINTER(HtaConfig)] + [_vp] * 10 + [_vp]),
}

_lib: Optional[ctypes.CDLL] = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libhta.so (once) and declare its signatures. Raises if it is not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def header_functions(header: str = HEADER_PATH) -> list:
    """Names of the functions include/hta.h declares."""
    txt = open(header).read()
    return sorted(set(re.findall(r"HTA_API\s+(?:const\s+)?\w+\**\s+\**(hta_\w+)\s*\(", txt)))


def _check(code: int, where: str) -> None:
    if code != HTA_OK:
        raise HtaError(code, where)


def hta_status_string(code: int) -> str:
    try:
        return load_library().hta_status_string(code).decode()
    except RuntimeError:
        return f"status {code}"


def make_config(*, batch, n_q_heads, n_kv_heads, head_dim, tree_nodes, kv_capacity, dtype="bf16",
                softmax_scale=0.0, num_workgroups=0, force_path=HTA_PATH_AUTO,
                qblocks_per_wave=0, fuse_merge=0) -> HtaConfig:
    dt = {"bf16": HTA_BF16, "f32": HTA_F32, HTA_BF16: HTA_BF16, HTA_F32: HTA_F32}[dtype]
    return HtaConfig(batch, n_q_heads, n_kv_heads, head_dim, tree_nodes, kv_capacity, dt,
                     float(softmax_scale), num_workgroups, force_path, qblocks_per_wave, fuse_merge)


def hta_validate_config(cfg: HtaConfig) -> int:
    return load_library().hta_validate_config(ctypes.byref(cfg))


class Handle:
    """An hta_handle_t plus the config it was created with (for argument checks)."""

    def __init__(self, ptr: int, cfg: HtaConfig):
        self.ptr = ptr
        self.cfg = cfg

    @property
    def dims(self):
        c = self.cfg
        return c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim, c.tree_nodes, c.kv_capacity

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        hta_destroy(self)


def hta_create(cfg: HtaConfig) -> Handle:
    out = _vp()
    _check(load_library().hta_create(ctypes.byref(out), ctypes.byref(cfg)), "hta_create")
    return Handle(out.value, cfg)


def hta_destroy(h: Handle) -> None:
    if h.ptr:
        code = load_library().hta_destroy(_vp(h.ptr))
        h.ptr = None
        _check(code, "hta_destroy")


def hta_get_plan(h: Handle) -> dict:
    p = HtaPlan()
    _check(load_library().hta_get_plan(_vp(h.ptr), ctypes.byref(p)), "hta_get_plan")
    return {name: getattr(p, name) for name, _ in HtaPlan._fields_}


# ----------------------------------------------------------------------------
# tensor marshalling
# ----------------------------------------------------------------------------

def _stream_ptr(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _tensor(t, name, dtype, shape):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _io_dtype(h: Handle):
    import torch
    return torch.bfloat16 if h.cfg.dtype == HTA_BF16 else torch.float32


def hta_verify_attn(h: Handle, q, k_cache, v_cache, k_tree, v_tree, parent, prefix_len, out, lse,
                    stream=None) -> None:
    import torch
    B, Hq, Hkv, D, T, Lcap = h.dims
    dt = _io_dtype(h)
    args = [
        _tensor(q, "q", dt, (B, Hq, T, D)),
        _tensor(k_cache, "k_cache", dt, (B, Hkv, Lcap, D)),
        _tensor(v_cache, "v_cache", dt, (B, Hkv, Lcap, D)),
        _tensor(k_tree, "k_tree", dt, (B, Hkv, T, D)),
        _tensor(v_tree, "v_tree", dt, (B, Hkv, T, D)),
        _tensor(parent, "parent", torch.int32, (B, T)),
        _tensor(prefix_len, "prefix_len", torch.int32, (B,)),
        _tensor(out, "out", dt, (B, Hq, T, D)),
        _tensor(lse, "lse", torch.float32, (B, Hq, T)),
    ]
    _check(load_library().hta_verify_attn(_vp(h.ptr), *[_vp(a) for a in args], _vp(_stream_ptr(stream))),
           "hta_verify_attn")


def hta_verify_attn_noalloc(cfg: HtaConfig, q, k_cache, v_cache, k_tree, v_tree, parent, prefix_len, out, lse,
                            status, stream=None) -> None:
    """hta_verify_attn without a handle or any allocation; status: int32 [1] on the device."""
    import torch
    B, Hq, Hkv, D, T, Lcap = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.tree_nodes, cfg.kv_capacity
    dt = torch.bfloat16 if cfg.dtype == HTA_BF16 else torch.float32
    args = [
        _tensor(q, "q", dt, (B, Hq, T, D)),
        _tensor(k_cache, "k_cache", dt, (B, Hkv, Lcap, D)),
        _tensor(v_cache, "v_cache", dt, (B, Hkv, Lcap, D)),
        _tensor(k_tree, "k_tree", dt, (B, Hkv, T, D)),
        _tensor(v_tree, "v_tree", dt, (B, Hkv, T, D)),
        _tensor(parent, "parent", torch.int32, (B, T)),
        _tensor(prefix_len, "prefix_len", torch.int32, (B,)),
        _tensor(out, "out", dt, (B, Hq, T, D)),
        _tensor(lse, "lse", torch.float32, (B, Hq, T)),
        _tensor(status, "status", torch.int32, (1,)),
    ]
    _check(load_library().hta_verify_attn_noalloc(ctypes.byref(cfg), *[_vp(a) for a in args],
                                                  _vp(_stream_ptr(stream))), "hta_verify_attn_noalloc")


def hta_tree_mask(h: Handle, parent, mask_out, stream=None) -> None:
    import torch
    B, _, _, _, T, _ = h.dims
    p = _tensor(parent, "parent", torch.int32, (B, T))
    m = _tensor(mask_out, "mask_out", torch.int64, (B, T))
    _check(load_library().hta_tree_mask(_vp(h.ptr), _vp(p), _vp(m), _vp(_stream_ptr(stream))),
           "hta_tree_mask")


def hta_tree_attn(h: Handle, q, k_tree, v_tree, parent, o_tree, lse_tree, stream=None) -> None:
    import torch
    B, Hq, Hkv, D, T, _ = h.dims
    dt = _io_dtype(h)
    args = [
        _tensor(q, "q", dt, (B, Hq, T, D)),
        _tensor(k_tree, "k_tree", dt, (B, Hkv, T, D)),
        _tensor(v_tree, "v_tree", dt, (B, Hkv, T, D)),
        _tensor(parent, "parent", torch.int32, (B, T)),
        _tensor(o_tree, "o_tree", torch.float32, (B, Hq, T, D)),
        _tensor(lse_tree, "lse_tree", torch.float32, (B, Hq, T)),
    ]
    _check(load_library().hta_tree_attn(_vp(h.ptr), *[_vp(a) for a in args], _vp(_stream_ptr(stream))),
           "hta_tree_attn")


def hta_cross_attn(h: Handle, q, k_cache, v_cache, prefix_len, out, lse, stream=None) -> None:
    """The drafter's cross-attention over the target's cache; out in the handle's dtype."""
    import torch
    B, Hq, Hkv, D, T, Lcap = h.dims
    dt = _io_dtype(h)
    args = [
        _tensor(q, "q", dt, (B, Hq, T, D)),
        _tensor(k_cache, "k_cache", dt, (B, Hkv, Lcap, D)),
        _tensor(v_cache, "v_cache", dt, (B, Hkv, Lcap, D)),
        _tensor(prefix_len, "prefix_len", torch.int32, (B,)),
        _tensor(out, "out", dt, (B, Hq, T, D)),
        _tensor(lse, "lse", torch.float32, (B, Hq, T)),
    ]
    _check(load_library().hta_cross_attn(_vp(h.ptr), *[_vp(a) for a in args], _vp(_stream_ptr(stream))),
           "hta_cross_attn")


def hta_build_tree(h: Handle, logits, history, history_len, params: HtaTreeParams, tree_tokens, parent, n_nodes,
                   stream=None) -> None:
    """logits [B, V] float32 or bfloat16 (last position); history [B, cap] int32; see include/hta.h."""
    import torch
    B, _, _, _, T, _ = h.dims
    if not isinstance(logits, torch.Tensor) or logits.dim() != 2:
        raise ValueError("logits must be a [B, V] tensor")
    if logits.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"logits has dtype {logits.dtype}, expected float32 or bfloat16")
    V = int(logits.shape[1])
    cap = int(history.shape[1]) if isinstance(history, torch.Tensor) and history.dim() == 2 else -1
    ldt = HTA_BF16 if logits.dtype == torch.bfloat16 else HTA_F32
    lp = _tensor(logits, "logits", logits.dtype, (B, V))
    hp = _tensor(history, "history", torch.int32, (B, cap))
    args = [
        _tensor(history_len, "history_len", torch.int32, (B,)),
    ]
    outs = [
        _tensor(tree_tokens, "tree_tokens", torch.int32, (B, T)),
        _tensor(parent, "parent", torch.int32, (B, T)),
        _tensor(n_nodes, "n_nodes", torch.int32, (B,)),
    ]
    _check(load_library().hta_build_tree(_vp(h.ptr), _vp(lp), V, ldt, _vp(hp), cap, _vp(args[0]),
                                         ctypes.byref(params), *[_vp(a) for a in outs], _vp(_stream_ptr(stream))),
           "hta_build_tree")


class NgramIndex:
    """An hta_ngram_index_t plus the sizes it was created with (for argument checks)."""

    def __init__(self, ptr: int, batch: int, history_cap: int, m: int):
        self.ptr = ptr
        self.batch, self.history_cap, self.m = batch, history_cap, m

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        hta_ngram_index_destroy(self)


def hta_ngram_index_create(batch: int, history_cap: int, m: int) -> NgramIndex:
    out = _vp()
    _check(load_library().hta_ngram_index_create(ctypes.byref(out), batch, history_cap, m), "hta_ngram_index_create")
    return NgramIndex(out.value, batch, history_cap, m)


def hta_ngram_index_destroy(idx: NgramIndex) -> None:
    if idx.ptr:
        code = load_library().hta_ngram_index_destroy(_vp(idx.ptr))
        idx.ptr = None
        _check(code, "hta_ngram_index_destroy")


def hta_ngram_index_reset(idx: NgramIndex, seq: int = -1, stream=None) -> None:
    """Empties sequence seq of the index (-1: every sequence), on the stream."""
    _check(load_library().hta_ngram_index_reset(_vp(idx.ptr), int(seq), _vp(_stream_ptr(stream))),
           "hta_ngram_index_reset")


def hta_build_tree_indexed(h: Handle, idx: NgramIndex, logits, history, history_len, params: HtaTreeParams,
                           tree_tokens, parent, n_nodes, stream=None) -> None:
    """hta_build_tree with the retrieval through idx; history [B, idx.history_cap] int32."""
    import torch
    B, _, _, _, T, _ = h.dims
    if not isinstance(logits, torch.Tensor) or logits.dim() != 2:
        raise ValueError("logits must be a [B, V] tensor")
    if logits.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"logits has dtype {logits.dtype}, expected float32 or bfloat16")
    V = int(logits.shape[1])
    ldt = HTA_BF16 if logits.dtype == torch.bfloat16 else HTA_F32
    lp = _tensor(logits, "logits", logits.dtype, (B, V))
    hp = _tensor(history, "history", torch.int32, (idx.batch, idx.history_cap))
    lenp = _tensor(history_len, "history_len", torch.int32, (B,))
    outs = [
        _tensor(tree_tokens, "tree_tokens", torch.int32, (B, T)),
        _tensor(parent, "parent", torch.int32, (B, T)),
        _tensor(n_nodes, "n_nodes", torch.int32, (B,)),
    ]
    _check(load_library().hta_build_tree_indexed(_vp(h.ptr), _vp(idx.ptr), _vp(lp), V, ldt, _vp(hp), _vp(lenp),
                                                 ctypes.byref(params), *[_vp(a) for a in outs],
                                                 _vp(_stream_ptr(stream))),
           "hta_build_tree_indexed")


def hta_window_attn(h: Handle, q, k_ring, v_ring, k_new, v_new, pos, out, lse, stream=None) -> None:
    """Sliding-window self-attention of the drafter: ring of W = kv_capacity slots, Tn = tree_nodes new tokens."""
    import torch
    B, Hq, Hkv, D, T, W = h.dims
    dt = _io_dtype(h)
    args = [
        _tensor(q, "q", dt, (B, Hq, T, D)),
        _tensor(k_ring, "k_ring", dt, (B, Hkv, W, D)),
        _tensor(v_ring, "v_ring", dt, (B, Hkv, W, D)),
        _tensor(k_new, "k_new", dt, (B, Hkv, T, D)),
        _tensor(v_new, "v_new", dt, (B, Hkv, T, D)),
        _tensor(pos, "pos", torch.int32, (B,)),
        _tensor(out, "out", dt, (B, Hq, T, D)),
        _tensor(lse, "lse", torch.float32, (B, Hq, T)),
    ]
    _check(load_library().hta_window_attn(_vp(h.ptr), *[_vp(a) for a in args], _vp(_stream_ptr(stream))),
           "hta_window_attn")


def hta_window_append(h: Handle, k_new, v_new, k_ring, v_ring, pos, stream=None) -> None:
    import torch
    B, Hq, Hkv, D, T, W = h.dims
    dt = _io_dtype(h)
    args = [
        _tensor(k_new, "k_new", dt, (B, Hkv, T, D)),
        _tensor(v_new, "v_new", dt, (B, Hkv, T, D)),
        _tensor(k_ring, "k_ring", dt, (B, Hkv, W, D)),
        _tensor(v_ring, "v_ring", dt, (B, Hkv, W, D)),
        _tensor(pos, "pos", torch.int32, (B,)),
    ]
    _check(load_library().hta_window_append(_vp(h.ptr), *[_vp(a) for a in args], _vp(_stream_ptr(stream))),
           "hta_window_append")


def hta_prefix_attn(h: Handle, q, k_cache, v_cache, prefix_len, o_prefix, lse_prefix, stream=None) -> None:
    import torch
    B, Hq, Hkv, D, T, Lcap = h.dims
    dt = _io_dtype(h)
    args = [
        _tensor(q, "q", dt, (B, Hq, T, D)),
        _tensor(k_cache, "k_cache", dt, (B, Hkv, Lcap, D)),
        _tensor(v_cache, "v_cache", dt, (B, Hkv, Lcap, D)),
        _tensor(prefix_len, "prefix_len", torch.int32, (B,)),
        _tensor(o_prefix, "o_prefix", torch.float32, (B, Hq, T, D)),
        _tensor(lse_prefix, "lse_prefix", torch.float32, (B, Hq, T)),
    ]
    _check(load_library().hta_prefix_attn(_vp(h.ptr), *[_vp(a) for a in args], _vp(_stream_ptr(stream))),
           "hta_prefix_attn")


def hta_prefix_partials(h: Handle, q, k_cache, v_cache, prefix_len, stream=None) -> None:
    import torch
    B, Hq, Hkv, D, T, Lcap = h.dims
    dt = _io_dtype(h)
    args = [
        _tensor(q, "q", dt, (B, Hq, T, D)),
        _tensor(k_cache, "k_cache", dt, (B, Hkv, Lcap, D)),
        _tensor(v_cache, "v_cache", dt, (B, Hkv, Lcap, D)),
        _tensor(prefix_len, "prefix_len", torch.int32, (B,)),
    ]
    _check(load_library().hta_prefix_partials(_vp(h.ptr), *[_vp(a) for a in args],
                                              _vp(_stream_ptr(stream))), "hta_prefix_partials")


def hta_merge_prefix(h: Handle, prefix_len, o_prefix, lse_prefix, stream=None) -> None:
    import torch
    B, Hq, _, D, T, _ = h.dims
    args = [
        _tensor(prefix_len, "prefix_len", torch.int32, (B,)),
        _tensor(o_prefix, "o_prefix", torch.float32, (B, Hq, T, D)),
        _tensor(lse_prefix, "lse_prefix", torch.float32, (B, Hq, T)),
    ]
    _check(load_library().hta_merge_prefix(_vp(h.ptr), *[_vp(a) for a in args], _vp(_stream_ptr(stream))),
           "hta_merge_prefix")


def hta_lse_merge(h: Handle, o_parts, lse_parts, out, lse, stream=None) -> None:
    import torch
    B, Hq, _, D, T, _ = h.dims
    n = int(o_parts.shape[0]) if o_parts.dim() > 0 else 0
    args = [
        _tensor(o_parts, "o_parts", torch.float32, (n, B, Hq, T, D)),
        _tensor(lse_parts, "lse_parts", torch.float32, (n, B, Hq, T)),
        _tensor(out, "out", torch.float32, (B, Hq, T, D)),
        _tensor(lse, "lse", torch.float32, (B, Hq, T)),
    ]
    _check(load_library().hta_lse_merge(_vp(h.ptr), n, *[_vp(a) for a in args], _vp(_stream_ptr(stream))),
           "hta_lse_merge")


def hta_accept(h: Handle, logits, parent, tree_tokens, target_tokens, accept_len, accept_path, bonus_token,
               stream=None) -> None:
    """logits [B, T, V] float32 or bfloat16; the int32 tensors as in include/hta.h."""
    import torch
    B, _, _, _, T, _ = h.dims
    if not isinstance(logits, torch.Tensor) or logits.dim() != 3:
        raise ValueError("logits must be a [B, T, V] tensor")
    if logits.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"logits has dtype {logits.dtype}, expected float32 or bfloat16")
    V = int(logits.shape[2])
    ldt = HTA_BF16 if logits.dtype == torch.bfloat16 else HTA_F32
    args = [
        _tensor(parent, "parent", torch.int32, (B, T)),
        _tensor(tree_tokens, "tree_tokens", torch.int32, (B, T)),
        _tensor(target_tokens, "target_tokens", torch.int32, (B, T)),
        _tensor(accept_len, "accept_len", torch.int32, (B,)),
        _tensor(accept_path, "accept_path", torch.int32, (B, T)),
        _tensor(bonus_token, "bonus_token", torch.int32, (B,)),
    ]
    lp = _tensor(logits, "logits", logits.dtype, (B, T, V))
    _check(load_library().hta_accept(_vp(h.ptr), _vp(lp), V, ldt, *[_vp(a) for a in args],
                                     _vp(_stream_ptr(stream))), "hta_accept")


def hta_commit(h: Handle, k_tree, v_tree, accept_len, accept_path, k_cache, v_cache, prefix_len,
               stream=None) -> None:
    import torch
    B, _, Hkv, D, T, Lcap = h.dims
    dt = _io_dtype(h)
    args = [
        _tensor(k_tree, "k_tree", dt, (B, Hkv, T, D)),
        _tensor(v_tree, "v_tree", dt, (B, Hkv, T, D)),
        _tensor(accept_len, "accept_len", torch.int32, (B,)),
        _tensor(accept_path, "accept_path", torch.int32, (B, T)),
        _tensor(k_cache, "k_cache", dt, (B, Hkv, Lcap, D)),
        _tensor(v_cache, "v_cache", dt, (B, Hkv, Lcap, D)),
        _tensor(prefix_len, "prefix_len", torch.int32, (B,)),
    ]
    _check(load_library().hta_commit(_vp(h.ptr), *[_vp(a) for a in args], _vp(_stream_ptr(stream))),
           "hta_commit")


def hta_get_status(h: Handle, stream=None) -> int:
    v = _i32(0)
    _check(load_library().hta_get_status(_vp(h.ptr), _vp(_stream_ptr(stream)), ctypes.byref(v)),
           "hta_get_status")
    return int(v.value)


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
