"""ragattn: ragged, batched, masked GQA attention for MI355X (gfx950).

Thin Python binding over the C ABI of ``libragattn.so`` (declared in
``include/ragattn.h``). These functions only marshal arguments: they check
tensor dtypes/devices, read sizes from tensor shapes, allocate ``out``/``lse``
when the caller does not pass them, and call the C entry point of the same
name on the current HIP stream. Every step of the attention runs in the HIP
kernels; there is no fallback path. If the library has not been built (see
``attention_ragged_gqa_amd.build``) the first call raises.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

__all__ = [
    "RagAttnError",
    "library",
    "lib_path",
    "EXPORTED_SYMBOLS",
    "ra_tree_attn",
    "ra_paged_attn",
    "ra_ragged_prefill",
    "ra_paged_attn_split",
    "ra_paged_attn_split_workspace",
    "ra_paged_attn_split_noalloc",
    "ra_merge_states",
    "ra_mla_paged_prefill",
    "ra_paged_kv_append",
    "ra_set_workgroup_waves",
    "ra_attn_workgroup_waves",
    "ra_last_error",
]

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libragattn.so"

EXPORTED_SYMBOLS = ("ra_tree_attn", "ra_paged_attn", "ra_ragged_prefill", "ra_paged_attn_split",
                    "ra_paged_attn_split_workspace", "ra_paged_attn_split_noalloc",
                    "ra_merge_states", "ra_mla_paged_prefill", "ra_paged_kv_append",
                    "ra_set_workgroup_waves", "ra_attn_workgroup_waves", "ra_last_error")

RA_OK, RA_EINVAL, RA_EUNSUPPORTED, RA_EHIP = 0, -1, -2, -3
RA_F16, RA_BF16 = 0, 1
_STATUS = {RA_EINVAL: "RA_EINVAL", RA_EUNSUPPORTED: "RA_EUNSUPPORTED", RA_EHIP: "RA_EHIP"}
_DTYPES = {torch.float16: RA_F16, torch.bfloat16: RA_BF16}


class RagAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (_STATUS.get(status, str(status)), message))
        self.status = status


_lib = None


def lib_path() -> str:
    return os.environ.get("RAGATTN_LIB", os.path.join(_PKG_DIR, LIB_NAME))


def library() -> ctypes.CDLL:
    """Load libragattn.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(
            "%s not found: build it with `python -m attention_ragged_gqa_amd.build`" % path)
    lib = ctypes.CDLL(path)
    i32, f32, vp = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
    lib.ra_tree_attn.restype = i32
    lib.ra_tree_attn.argtypes = [vp] * 10 + [i32] * 8 + [i32, f32, f32, f32, vp]
    lib.ra_paged_attn.restype = i32
    lib.ra_paged_attn.argtypes = ([vp] * 6 + [i32] + [vp] * 4 + [i32] + [vp] * 2 + [i32] * 9
                                  + [i32, i32, f32, f32, f32, vp])
    lib.ra_ragged_prefill.restype = i32
    lib.ra_ragged_prefill.argtypes = [vp] * 6 + [i32, i32, vp, vp] + [i32] * 7 + [f32, vp]
    lib.ra_paged_attn_split.restype = i32
    lib.ra_paged_attn_split.argtypes = ([vp] * 6 + [i32] + [vp] * 4 + [i32] + [vp] * 2 + [i32] * 9
                                        + [i32, i32, f32, f32, f32, i32, vp, ctypes.c_size_t, vp])
    lib.ra_paged_attn_split_noalloc.restype = i32
    lib.ra_paged_attn_split_noalloc.argtypes = ([vp] * 6 + [i32] + [vp] * 4 + [i32] + [vp] * 2
                                                + [i32] * 9 + [i32, i32, f32, f32, f32, i32, vp])
    lib.ra_paged_attn_split_workspace.restype = ctypes.c_size_t
    lib.ra_paged_attn_split_workspace.argtypes = [i32] * 4
    lib.ra_merge_states.restype = i32
    lib.ra_merge_states.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp]
    lib.ra_mla_paged_prefill.restype = i32
    lib.ra_mla_paged_prefill.argtypes = [vp] * 6 + [i32, vp, vp] + [i32] * 8 + [i32, f32, vp]
    lib.ra_paged_kv_append.restype = i32
    lib.ra_paged_kv_append.argtypes = [vp] * 8 + [i32] * 7 + [i32, f32, f32, vp]
    lib.ra_set_workgroup_waves.restype = i32
    lib.ra_set_workgroup_waves.argtypes = [i32]
    lib.ra_attn_workgroup_waves.restype = i32
    lib.ra_attn_workgroup_waves.argtypes = [i32] * 4
    lib.ra_last_error.restype = ctypes.c_char_p
    lib.ra_last_error.argtypes = []
    _lib = lib
    return lib


def ra_last_error() -> str:
    return library().ra_last_error().decode()


def ra_set_workgroup_waves(waves: int) -> None:
    """Fix the attention kernels' workgroup shape for later launches in this
    process: 4 or 8 waves (128 or 256 packed query rows per work item), or 0
    to let each launch choose (the default). A tuning override; results are
    the same either way."""
    st = library().ra_set_workgroup_waves(int(waves))
    if st != RA_OK:
        raise RagAttnError(st, ra_last_error())


def ra_attn_workgroup_waves(total_q: int, h_q: int, h_kv: int, num_kv_splits: int = 1) -> int:
    """Waves per workgroup (4 or 8) an attention launch of these sizes uses
    (0 for sizes the entry points reject)."""
    return int(library().ra_attn_workgroup_waves(int(total_q), int(h_q), int(h_kv), int(num_kv_splits)))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_dev(name: str, t: Optional[torch.Tensor], dtype=None, device=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor (got %s)" % (name, t.device))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))


def _stream(device, stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _raise(status: int):
    if status != RA_OK:
        raise RagAttnError(status, ra_last_error())


def _out_lse(q, out, lse):
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
    _check_dev("out", out, q.dtype, q.device)
    _check_dev("lse", lse, torch.float32, q.device)
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != tuple(q.shape[:2]):
        raise ValueError("out must be shaped like q and lse like q[:, :, 0]")
    return out, lse


def _need(cond: bool, msg: str, *args):
    if not cond:
        raise ValueError(msg % args if args else msg)


def _numel_is(name: str, t, n: int):
    if t is not None:
        _need(t.numel() == n, "%s must hold %d entries (got %d)", name, n, t.numel())


def _check_qkv(q, k, v):
    """q [total_q, h_q, d]; k and v [total_kv, h_kv, d] of one shape, h_kv
    dividing h_q."""
    _need(q.dim() == 3, "q must be [total_q, h_q, head_dim] (got %d dims)", q.dim())
    _need(k.dim() == 3 and tuple(k.shape) == tuple(v.shape),
          "k and v must both be [total_kv, h_kv, head_dim] (got %s and %s)",
          tuple(k.shape), tuple(v.shape))
    _need(k.shape[2] == q.shape[2], "k/v head_dim %d != q head_dim %d", k.shape[2], q.shape[2])
    _need(k.shape[1] > 0 and q.shape[1] % k.shape[1] == 0,
          "h_q (%d) must be a multiple of h_kv (%d)", q.shape[1], k.shape[1])


def _check_indptr(name: str, t, batch: int):
    _need(t is not None and t.dim() == 1 and t.numel() == batch + 1,
          "%s must be a [batch + 1] array (batch %d)", name, batch)


def _check_paged_shapes(q, q_indptr, pages, page_indptr, length_info, sliding_window,
                        k_rope_pos_offset, q_rope_position, tree_order_indptr, tree_order):
    _need(q.dim() == 3, "q must be [total_q, h_q, head_dim] (got %d dims)", q.dim())
    _need(q_indptr is not None and q_indptr.dim() == 1 and q_indptr.numel() >= 1,
          "q_indptr must be a [batch + 1] array")
    batch = q_indptr.numel() - 1
    _need(pages.dim() == 5 and pages.shape[1] == 2,
          "pages must be [num_pages, 2, h_kv, page_size, head_dim] (got %s)", tuple(pages.shape))
    _need(pages.shape[4] == q.shape[2], "pages head_dim %d != q head_dim %d", pages.shape[4], q.shape[2])
    _need(pages.shape[2] > 0 and q.shape[1] % pages.shape[2] == 0,
          "h_q (%d) must be a multiple of h_kv (%d)", q.shape[1], pages.shape[2])
    _check_indptr("page_indptr", page_indptr, batch)
    _need(length_info is not None, "length_info is required")
    if sliding_window:
        _need(tuple(length_info.shape) == (3, batch),
              "length_info must be [3, batch] with a sliding window (got %s)", tuple(length_info.shape))
    else:
        _need(length_info.numel() == batch, "length_info must hold batch (%d) entries", batch)
    _numel_is("k_rope_pos_offset", k_rope_pos_offset, batch)
    _numel_is("q_rope_position", q_rope_position, q.shape[0])
    if tree_order is not None or tree_order_indptr is not None:
        _need(tree_order_indptr is not None, "tree_order given without tree_order_indptr")
        _check_indptr("tree_order_indptr", tree_order_indptr, batch)
        _need(tree_order is not None and tree_order.dim() == 2 and tree_order.shape[1] == 2,
              "tree_order must be [n, 2]")
    return batch


def ra_tree_attn(q, q_indptr, k, v, kv_indptr, q_rope_position, mn_indptr, tree_mask,
                 out=None, lse=None, rotary_mode: int = 0, rope_scale: float = 1.0,
                 rope_theta: float = 1e4, sm_scale: Optional[float] = None, stream=None):
    """Batched tree attention over contiguous KV (C: ra_tree_attn).

    q [total_q, h_q, d], k/v [total_kv, h_kv, d] (fp16/bf16); q_indptr,
    kv_indptr, mn_indptr [b+1], q_rope_position [total_q] (or None when
    rotary_mode == 0), tree_mask [n, 2] int32. Returns (out, lse)."""
    # shapes first: a mismatch must never reach the kernels
    _check_qkv(q, k, v)
    _need(q_indptr is not None and q_indptr.dim() == 1 and q_indptr.numel() >= 1,
          "q_indptr must be a [batch + 1] array")
    batch = q_indptr.numel() - 1
    _check_indptr("kv_indptr", kv_indptr, batch)
    _check_indptr("mn_indptr", mn_indptr, batch)
    _need(tree_mask is not None and tree_mask.dim() == 2 and tree_mask.shape[1] == 2,
          "tree_mask must be [n, 2]")
    if rotary_mode == 1:
        _need(q_rope_position is not None, "rotary_mode 1 needs q_rope_position")
    _numel_is("q_rope_position", q_rope_position, q.shape[0])
    dev = q.device
    i32 = torch.int32
    _check_dev("q", q, None, dev)
    if q.dtype not in _DTYPES:
        raise TypeError("q must be fp16 or bf16")
    for name, t in (("k", k), ("v", v)):
        _check_dev(name, t, q.dtype, dev)
    for name, t in (("q_indptr", q_indptr), ("kv_indptr", kv_indptr), ("mn_indptr", mn_indptr),
                    ("q_rope_position", q_rope_position), ("tree_mask", tree_mask)):
        _check_dev(name, t, i32, dev)
    out, lse = _out_lse(q, out, lse)
    total_q, h_q, d = q.shape
    total_kv, h_kv = k.shape[0], k.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    st = library().ra_tree_attn(
        _ptr(q), _ptr(q_indptr), _ptr(k), _ptr(v), _ptr(kv_indptr), _ptr(q_rope_position),
        _ptr(mn_indptr), _ptr(tree_mask), _ptr(out), _ptr(lse),
        q_indptr.numel() - 1, total_q, total_kv, tree_mask.shape[0], h_q, h_kv, d,
        _DTYPES[q.dtype], rotary_mode, rope_scale, rope_theta, sm_scale, _stream(dev, stream))
    _raise(st)
    return out, lse


def ra_paged_attn(q, q_indptr, pages, page_indptr, page_values, length_info,
                  sliding_window: int = 0, k_rope_pos_offset=None, q_rope_position=None,
                  tree_order_indptr=None, tree_order=None, causal: int = 1, out=None, lse=None,
                  rotary_mode: int = 0, rope_scale: float = 1.0, rope_theta: float = 1e4,
                  sm_scale: Optional[float] = None, stream=None):
    """Ragged prefill / tree attention over a paged KV cache (C: ra_paged_attn).

    pages [num_pages, 2, h_kv, 16, d]; length_info [b] or [3, b] int32.
    Returns (out, lse)."""
    _check_paged_shapes(q, q_indptr, pages, page_indptr, length_info, sliding_window,
                        k_rope_pos_offset, q_rope_position, tree_order_indptr, tree_order)
    if rotary_mode == 1:
        _need(q_rope_position is not None, "rotary_mode 1 needs q_rope_position")
    dev = q.device
    i32 = torch.int32
    _check_dev("q", q, None, dev)
    if q.dtype not in _DTYPES:
        raise TypeError("q must be fp16 or bf16")
    _check_dev("pages", pages, q.dtype, dev)
    for name, t in (("q_indptr", q_indptr), ("page_indptr", page_indptr),
                    ("page_values", page_values), ("length_info", length_info),
                    ("k_rope_pos_offset", k_rope_pos_offset), ("q_rope_position", q_rope_position),
                    ("tree_order_indptr", tree_order_indptr), ("tree_order", tree_order)):
        _check_dev(name, t, i32, dev)
    if pages.dim() != 5 or pages.shape[1] != 2:
        raise ValueError("pages must be [num_pages, 2, h_kv, page_size, d]")
    out, lse = _out_lse(q, out, lse)
    total_q, h_q, d = q.shape
    num_pages, _, h_kv, page_size, dp = pages.shape
    if dp != d:
        raise ValueError("pages head_dim %d != q head_dim %d" % (dp, d))
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    tree_size = 0 if tree_order is None else tree_order.shape[0]
    st = library().ra_paged_attn(
        _ptr(q), _ptr(q_indptr), _ptr(pages), _ptr(page_indptr), _ptr(page_values),
        _ptr(length_info), int(sliding_window), _ptr(k_rope_pos_offset), _ptr(q_rope_position),
        _ptr(tree_order_indptr), _ptr(tree_order), int(causal), _ptr(out), _ptr(lse),
        q_indptr.numel() - 1, total_q, num_pages, page_values.numel(), tree_size, page_size,
        h_q, h_kv, d, _DTYPES[q.dtype], rotary_mode, rope_scale, rope_theta, sm_scale,
        _stream(dev, stream))
    _raise(st)
    return out, lse


def ra_ragged_prefill(q, q_indptr, k, v, kv_indptr, valid_len=None, pad_mode: int = 0,
                      causal: int = 1, out=None, lse=None, sm_scale: Optional[float] = None,
                      stream=None):
    """Ragged prefill over contiguous K/V with optional padded-batch masks
    (C: ra_ragged_prefill). q [total_q, h_q, d], k/v [total_kv, h_kv, d];
    pad_mode 0 plain (causal or not), 1 right padding (non-causal),
    2 left padding (causal) with valid_len [b]. Returns (out, lse)."""
    _check_qkv(q, k, v)
    _need(q_indptr is not None and q_indptr.dim() == 1 and q_indptr.numel() >= 1,
          "q_indptr must be a [batch + 1] array")
    batch = q_indptr.numel() - 1
    _check_indptr("kv_indptr", kv_indptr, batch)
    if pad_mode != 0:
        _need(valid_len is not None, "pad_mode %d needs valid_len", pad_mode)
    _numel_is("valid_len", valid_len, batch)
    dev = q.device
    i32 = torch.int32
    _check_dev("q", q, None, dev)
    if q.dtype not in _DTYPES:
        raise TypeError("q must be fp16 or bf16")
    for name, t in (("k", k), ("v", v)):
        _check_dev(name, t, q.dtype, dev)
    for name, t in (("q_indptr", q_indptr), ("kv_indptr", kv_indptr), ("valid_len", valid_len)):
        _check_dev(name, t, i32, dev)
    out, lse = _out_lse(q, out, lse)
    total_q, h_q, d = q.shape
    total_kv, h_kv = k.shape[0], k.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    st = library().ra_ragged_prefill(
        _ptr(q), _ptr(q_indptr), _ptr(k), _ptr(v), _ptr(kv_indptr), _ptr(valid_len), int(pad_mode),
        int(causal), _ptr(out), _ptr(lse), q_indptr.numel() - 1, total_q, total_kv, h_q, h_kv, d,
        _DTYPES[q.dtype], sm_scale, _stream(dev, stream))
    _raise(st)
    return out, lse


def ra_paged_attn_split_workspace(total_q: int, h_q: int, head_dim: int, num_kv_splits: int) -> int:
    """Workspace bytes ra_paged_attn_split needs (C: ra_paged_attn_split_workspace)."""
    return int(library().ra_paged_attn_split_workspace(total_q, h_q, head_dim, num_kv_splits))


def ra_paged_attn_split(q, q_indptr, pages, page_indptr, page_values, length_info,
                        sliding_window: int = 0, k_rope_pos_offset=None, q_rope_position=None,
                        tree_order_indptr=None, tree_order=None, causal: int = 1, out=None,
                        lse=None, rotary_mode: int = 0, rope_scale: float = 1.0,
                        rope_theta: float = 1e4, sm_scale: Optional[float] = None,
                        num_kv_splits: int = 0, workspace=None, stream=None):
    """Split-KV paged attention (C: ra_paged_attn_split). Arguments as
    ra_paged_attn, plus num_kv_splits (0: the library chooses) and an optional
    uint8 device workspace; when it is None one is allocated here for the
    largest split count (64). Returns (out, lse)."""
    _check_paged_shapes(q, q_indptr, pages, page_indptr, length_info, sliding_window,
                        k_rope_pos_offset, q_rope_position, tree_order_indptr, tree_order)
    if rotary_mode == 1:
        _need(q_rope_position is not None, "rotary_mode 1 needs q_rope_position")
    dev = q.device
    i32 = torch.int32
    _check_dev("q", q, None, dev)
    if q.dtype not in _DTYPES:
        raise TypeError("q must be fp16 or bf16")
    _check_dev("pages", pages, q.dtype, dev)
    for name, t in (("q_indptr", q_indptr), ("page_indptr", page_indptr),
                    ("page_values", page_values), ("length_info", length_info),
                    ("k_rope_pos_offset", k_rope_pos_offset), ("q_rope_position", q_rope_position),
                    ("tree_order_indptr", tree_order_indptr), ("tree_order", tree_order)):
        _check_dev(name, t, i32, dev)
    if pages.dim() != 5 or pages.shape[1] != 2:
        raise ValueError("pages must be [num_pages, 2, h_kv, page_size, d]")
    out, lse = _out_lse(q, out, lse)
    total_q, h_q, d = q.shape
    num_pages, _, h_kv, page_size, dp = pages.shape
    if dp != d:
        raise ValueError("pages head_dim %d != q head_dim %d" % (dp, d))
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if workspace is None:
        n = ra_paged_attn_split_workspace(total_q, h_q, d, num_kv_splits if num_kv_splits > 0 else 64)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    _check_dev("workspace", workspace, None, dev)
    tree_size = 0 if tree_order is None else tree_order.shape[0]
    st = library().ra_paged_attn_split(
        _ptr(q), _ptr(q_indptr), _ptr(pages), _ptr(page_indptr), _ptr(page_values),
        _ptr(length_info), int(sliding_window), _ptr(k_rope_pos_offset), _ptr(q_rope_position),
        _ptr(tree_order_indptr), _ptr(tree_order), int(causal), _ptr(out), _ptr(lse),
        q_indptr.numel() - 1, total_q, num_pages, page_values.numel(), tree_size, page_size,
        h_q, h_kv, d, _DTYPES[q.dtype], rotary_mode, rope_scale, rope_theta, sm_scale,
        int(num_kv_splits), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(dev, stream))
    _raise(st)
    return out, lse


NOALLOC_SCRATCH_BYTES = 32 << 20   # the library's per-GPU partial-state array


def ra_paged_attn_split_noalloc(q, q_indptr, pages, page_indptr, page_values, length_info,
                                sliding_window: int = 0, k_rope_pos_offset=None,
                                q_rope_position=None, tree_order_indptr=None, tree_order=None,
                                causal: int = 1, out=None, lse=None, rotary_mode: int = 0,
                                rope_scale: float = 1.0, rope_theta: float = 1e4,
                                sm_scale: Optional[float] = None, num_kv_splits: int = 0,
                                stream=None):
    """Split-KV paged attention whose partial states live in the library's
    own per-GPU scratch array (C: ra_paged_attn_split_noalloc): the C call
    allocates nothing. out and lse must be passed in for a call that
    allocates nothing here either. Calls overlapping on one GPU race.
    Returns (out, lse)."""
    _check_paged_shapes(q, q_indptr, pages, page_indptr, length_info, sliding_window,
                        k_rope_pos_offset, q_rope_position, tree_order_indptr, tree_order)
    if rotary_mode == 1:
        _need(q_rope_position is not None, "rotary_mode 1 needs q_rope_position")
    dev = q.device
    i32 = torch.int32
    _check_dev("q", q, None, dev)
    if q.dtype not in _DTYPES:
        raise TypeError("q must be fp16 or bf16")
    _check_dev("pages", pages, q.dtype, dev)
    for name, t in (("q_indptr", q_indptr), ("page_indptr", page_indptr),
                    ("page_values", page_values), ("length_info", length_info),
                    ("k_rope_pos_offset", k_rope_pos_offset), ("q_rope_position", q_rope_position),
                    ("tree_order_indptr", tree_order_indptr), ("tree_order", tree_order)):
        _check_dev(name, t, i32, dev)
    out, lse = _out_lse(q, out, lse)
    total_q, h_q, d = q.shape
    num_pages, _, h_kv, page_size, _ = pages.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    tree_size = 0 if tree_order is None else tree_order.shape[0]
    st = library().ra_paged_attn_split_noalloc(
        _ptr(q), _ptr(q_indptr), _ptr(pages), _ptr(page_indptr), _ptr(page_values),
        _ptr(length_info), int(sliding_window), _ptr(k_rope_pos_offset), _ptr(q_rope_position),
        _ptr(tree_order_indptr), _ptr(tree_order), int(causal), _ptr(out), _ptr(lse),
        q_indptr.numel() - 1, total_q, num_pages, page_values.numel(), tree_size, page_size,
        h_q, h_kv, d, _DTYPES[q.dtype], rotary_mode, rope_scale, rope_theta, sm_scale,
        int(num_kv_splits), _stream(dev, stream))
    _raise(st)
    return out, lse


def ra_merge_states(part_out, part_lse, out, lse, stream=None):
    """Merge split-KV partial states (C: ra_merge_states).

    part_out [S, rows, d] fp32, part_lse [S, rows] fp32 (base-2 lse);
    out [rows, d] (or [tokens, heads, d]) fp16/bf16, lse [rows] fp32."""
    dev = part_out.device
    _check_dev("part_out", part_out, torch.float32, dev)
    _check_dev("part_lse", part_lse, torch.float32, dev)
    if out.dtype not in _DTYPES:
        raise TypeError("out must be fp16 or bf16")
    _check_dev("out", out, None, dev)
    _check_dev("lse", lse, torch.float32, dev)
    S, rows, d = part_out.shape
    if tuple(part_lse.shape) != (S, rows) or out.numel() != rows * d or lse.numel() != rows:
        raise ValueError("shapes: part_out [S, rows, d], part_lse [S, rows], out rows*d, lse rows")
    st = library().ra_merge_states(_ptr(part_out), _ptr(part_lse), S, rows, d, _DTYPES[out.dtype],
                                   _ptr(out), _ptr(lse), _stream(dev, stream))
    _raise(st)
    return out, lse


def ra_mla_paged_prefill(q, q_indptr, pages, page_indptr, page_values, last_page_len,
                         causal: int = 1, d_latent: int = 512, out=None, lse=None,
                         sm_scale: Optional[float] = None, stream=None):
    """Multi-head latent attention over a paged latent cache
    (C: ra_mla_paged_prefill). q [total_q, h_q, d_qk]; pages
    [num_pages, 16, d_qk], one latent row per cached token shared by every
    head (K = all d_qk values, V = the first d_latent); last_page_len [b].
    Returns (out [total_q, h_q, d_latent], lse [total_q, h_q])."""
    _need(q.dim() == 3, "q must be [total_q, h_q, d_qk] (got %d dims)", q.dim())
    _need(q_indptr is not None and q_indptr.dim() == 1 and q_indptr.numel() >= 1,
          "q_indptr must be a [batch + 1] array")
    batch = q_indptr.numel() - 1
    _need(pages.dim() == 3 and pages.shape[2] == q.shape[2],
          "pages must be [num_pages, page_size, d_qk] with q's d_qk (got %s)", tuple(pages.shape))
    _need(0 < d_latent <= q.shape[2], "d_latent must be in (0, d_qk]")
    _check_indptr("page_indptr", page_indptr, batch)
    _numel_is("last_page_len", last_page_len, batch)
    _need(last_page_len is not None, "last_page_len is required")
    dev = q.device
    i32 = torch.int32
    _check_dev("q", q, None, dev)
    if q.dtype not in _DTYPES:
        raise TypeError("q must be fp16 or bf16")
    _check_dev("pages", pages, q.dtype, dev)
    for name, t in (("q_indptr", q_indptr), ("page_indptr", page_indptr),
                    ("page_values", page_values), ("last_page_len", last_page_len)):
        _check_dev(name, t, i32, dev)
    total_q, h_q, d_qk = q.shape
    if out is None:
        out = torch.empty(total_q, h_q, d_latent, dtype=q.dtype, device=dev)
    if lse is None:
        lse = torch.empty(total_q, h_q, dtype=torch.float32, device=dev)
    _check_dev("out", out, q.dtype, dev)
    _check_dev("lse", lse, torch.float32, dev)
    _need(tuple(out.shape) == (total_q, h_q, d_latent) and tuple(lse.shape) == (total_q, h_q),
          "out must be [total_q, h_q, d_latent] and lse [total_q, h_q]")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d_qk)
    num_pages, page_size, _ = pages.shape
    st = library().ra_mla_paged_prefill(
        _ptr(q), _ptr(q_indptr), _ptr(pages), _ptr(page_indptr), _ptr(page_values),
        _ptr(last_page_len), int(causal), _ptr(out), _ptr(lse), batch, total_q, num_pages,
        page_values.numel(), page_size, h_q, d_qk, d_latent, _DTYPES[q.dtype], sm_scale,
        _stream(dev, stream))
    _raise(st)
    return out, lse


def ra_paged_kv_append(k, v, append_indptr, append_start, rope_position, page_indptr,
                       page_values, pages, rope_scale: float = 1.0, rope_theta: float = 1e4,
                       stream=None):
    """Write tokens k/v [n, h_kv, d] into ``pages`` in place, rotating K at
    rope_position when it is given (C: ra_paged_kv_append)."""
    _need(pages.dim() == 5 and pages.shape[1] == 2,
          "pages must be [num_pages, 2, h_kv, page_size, head_dim] (got %s)", tuple(pages.shape))
    _need(k.dim() == 3 and tuple(k.shape) == tuple(v.shape)
          and tuple(k.shape[1:]) == (pages.shape[2], pages.shape[4]),
          "k and v must both be [n_tokens, h_kv, head_dim] = [n, %d, %d] (got %s and %s)",
          pages.shape[2], pages.shape[4], tuple(k.shape), tuple(v.shape))
    _need(append_indptr is not None and append_indptr.dim() == 1 and append_indptr.numel() >= 1,
          "append_indptr must be a [batch + 1] array")
    batch = append_indptr.numel() - 1
    _numel_is("append_start", append_start, batch)
    _check_indptr("page_indptr", page_indptr, batch)
    _numel_is("rope_position", rope_position, k.shape[0])
    dev = pages.device
    i32 = torch.int32
    _check_dev("pages", pages, None, dev)
    if pages.dtype not in _DTYPES:
        raise TypeError("pages must be fp16 or bf16")
    for name, t in (("k", k), ("v", v)):
        _check_dev(name, t, pages.dtype, dev)
    for name, t in (("append_indptr", append_indptr), ("append_start", append_start),
                    ("rope_position", rope_position), ("page_indptr", page_indptr),
                    ("page_values", page_values)):
        _check_dev(name, t, i32, dev)
    num_pages, _, h_kv, page_size, d = pages.shape
    st = library().ra_paged_kv_append(
        _ptr(k), _ptr(v), _ptr(append_indptr), _ptr(append_start), _ptr(rope_position),
        _ptr(page_indptr), _ptr(page_values), _ptr(pages), append_indptr.numel() - 1,
        k.shape[0], num_pages, page_values.numel(), page_size, h_kv, d, _DTYPES[pages.dtype],
        rope_scale, rope_theta, _stream(dev, stream))
    _raise(st)
    return pages
