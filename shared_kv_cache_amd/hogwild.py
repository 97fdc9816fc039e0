"""Thin ctypes binding of the Hogwild! decode library (``include/hogwild.h``).

Functions carry the C names and only marshal arguments: every step of the path
runs in the library's host code and gfx950 kernels. ``HogwildCache`` is a small
convenience owner that allocates the pools and the workspace as torch device
tensors (PyTorch supplies device memory and streams, nothing else).

There is no fallback: if ``_lib/libhogwild.so`` is missing, importing this
module's functions raises ``ImportError`` telling how to build it. The environment
variable ``HOGWILD_LIBRARY`` names another build of the same library to load instead
(for instance the sanitizer build of ``build.py --asan-host``).
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_double, c_float, c_int, c_int32, c_int64, c_size_t, c_uint32, c_void_p
from typing import Optional, Sequence

LIB_PATH = os.environ.get("HOGWILD_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "_lib", "libhogwild.so")

HW_OK, HW_ERR_INVALID_ARG, HW_ERR_OUT_OF_PAGES, HW_ERR_STALE_VIEW, HW_ERR_WORKSPACE, HW_ERR_HIP = range(6)
HW_BF16, HW_F32 = 0, 1
STATUS_NAMES = {0: "HW_OK", 1: "HW_ERR_INVALID_ARG", 2: "HW_ERR_OUT_OF_PAGES",
                3: "HW_ERR_STALE_VIEW", 4: "HW_ERR_WORKSPACE", 5: "HW_ERR_HIP"}

# every symbol the headers declare
EXPORTS = ["hw_create", "hw_destroy", "hw_last_error", "hw_workspace_bytes", "hw_set_workspace",
           "hw_append_kv", "hw_set_views", "hw_concurrent_decode", "hw_concurrent_decode_tokens",
           "hw_concurrent_decode_noalloc", "hw_reset_block", "hw_plan_steps", "hw_append_step", "hw_decode_step",
           "hw_plan_end",
           "hw_set_split", "hw_block_info", "hw_free_pages", "hw_debug_reserve",
           "hw_debug_resolve", "hw_debug_kernel_events", "hw_debug_kernel_elapsed",
           "hw_debug_stream_read", "hw_debug_partition"]


class HwConfig(ctypes.Structure):
    _fields_ = [
        ("n_layers", c_int32), ("n_q_heads", c_int32), ("n_kv_heads", c_int32),
        ("head_dim", c_int32), ("page_size", c_int32), ("n_pages", c_int32),
        ("max_blocks", c_int32), ("max_workers", c_int32), ("max_position", c_int32),
        ("max_splits", c_int32), ("max_query_tokens", c_int32), ("kv_dtype", c_int),
        ("page_seed", c_uint32),
        ("rope_theta", c_double), ("softmax_scale", c_float),
        ("k_pool", c_void_p), ("v_pool", c_void_p),
    ]


class HwError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


_LIB = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m shared_kv_cache_amd.build` "
                          "(there is no fallback path)")
    # PyTorch ships its own HIP runtime under the same soname. Importing it first makes the
    # library bind to that copy; loaded the other way round, the process would hold two HIP
    # runtimes, and the second to initialise finds no device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P32, P64 = POINTER(c_int32), POINTER(c_int64)
    sig = {
        "hw_create": (c_int, [POINTER(HwConfig), POINTER(c_void_p)]),
        "hw_destroy": (c_int, [c_void_p]),
        "hw_last_error": (ctypes.c_char_p, [c_void_p]),
        "hw_workspace_bytes": (c_size_t, [c_void_p]),
        "hw_set_workspace": (c_int, [c_void_p, c_void_p, c_size_t]),
        "hw_append_kv": (c_int, [c_void_p, c_int32, c_int32, P32, P32, c_void_p, c_void_p, c_void_p]),
        "hw_set_views": (c_int, [c_void_p, c_int32, P32, P32, P64, P64]),
        "hw_concurrent_decode": (c_int, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
        "hw_concurrent_decode_tokens": (c_int, [c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                                                c_void_p, c_void_p]),
        "hw_concurrent_decode_noalloc": (c_int, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                                 c_void_p]),
        "hw_reset_block": (c_int, [c_void_p, c_int32]),
        "hw_plan_steps": (c_int, [c_void_p, c_int32, c_int32, P32, P32, c_void_p]),
        "hw_append_step": (c_int, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p]),
        "hw_decode_step": (c_int, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_void_p]),
        "hw_plan_end": (c_int, [c_void_p, c_void_p]),
        "hw_set_split": (c_int, [c_void_p, c_int32]),
        "hw_block_info": (c_int, [c_void_p, c_int32, c_int32, P32, P32, c_int32, P32]),
        "hw_free_pages": (c_int, [c_void_p, P32]),
        "hw_debug_reserve": (c_int, [c_void_p, c_int32, c_int32, P32, P32, P32, c_int32, P32]),
        "hw_debug_resolve": (c_int, [c_void_p, c_int32, P32, P32, c_int32, P32, P32, c_int32, P32, P32]),
        "hw_debug_kernel_events": (c_int, [c_void_p, c_int32]),
        "hw_debug_kernel_elapsed": (c_int, [c_void_p, POINTER(c_float), c_int32, P32]),
        "hw_debug_stream_read": (c_int, [c_void_p, c_size_t, c_void_p, c_int32, c_void_p,
                                         POINTER(c_float)]),
        "hw_debug_partition": (c_int, [POINTER(ctypes.c_uint8), c_int32, c_int32, ctypes.c_double,
                                       P32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def _i32(values) -> ctypes.Array:
    values = [int(x) for x in values]
    return (c_int32 * max(1, len(values)))(*values)


def _i64(values) -> ctypes.Array:
    values = [int(x) for x in values]
    return (c_int64 * max(1, len(values)))(*values)


def _check(ctx, status: int):
    if status != HW_OK:
        raise HwError(status, hw_last_error(ctx))


# ---------------------------------------------------------------- C names

def hw_create(cfg: HwConfig) -> c_void_p:
    lib = load_library()
    ctx = c_void_p()
    st = lib.hw_create(ctypes.byref(cfg), ctypes.byref(ctx))
    if st != HW_OK:
        raise HwError(st, lib.hw_last_error(None).decode())
    return ctx


def hw_destroy(ctx) -> None:
    load_library().hw_destroy(ctx)


def hw_last_error(ctx) -> str:
    return load_library().hw_last_error(ctx).decode()


def hw_workspace_bytes(ctx) -> int:
    return int(load_library().hw_workspace_bytes(ctx))


def hw_set_workspace(ctx, dev_ptr: int, nbytes: int) -> None:
    _check(ctx, load_library().hw_set_workspace(ctx, c_void_p(dev_ptr), nbytes))


def hw_append_kv(ctx, layer: int, block_ids: Sequence[int], n_tokens: Sequence[int],
                 k_ptr: int, v_ptr: int, stream: int) -> None:
    _check(ctx, load_library().hw_append_kv(ctx, layer, len(block_ids), _i32(block_ids),
                                            _i32(n_tokens), c_void_p(k_ptr), c_void_p(v_ptr),
                                            c_void_p(stream)))


def hw_set_views(ctx, views: Sequence[Sequence[int]], offsets=None, q_pos=None) -> None:
    lens = [len(v) for v in views]
    flat = [b for v in views for b in v]
    offs = None if offsets is None else _i64([o for ov in offsets for o in ov])
    qp = None if q_pos is None else _i64(q_pos)
    _check(ctx, load_library().hw_set_views(ctx, len(views), _i32(lens), _i32(flat), offs, qp))


def hw_concurrent_decode(ctx, layer: int, q_ptr: int, out_ptr: int, lse_ptr: Optional[int],
                         stream: int) -> None:
    _check(ctx, load_library().hw_concurrent_decode(ctx, layer, c_void_p(q_ptr), c_void_p(out_ptr),
                                                    c_void_p(lse_ptr) if lse_ptr else None,
                                                    c_void_p(stream)))


def hw_concurrent_decode_tokens(ctx, layer: int, n_new: int, q_ptr: int, out_ptr: int,
                                lse_ptr: Optional[int], stream: int) -> None:
    _check(ctx, load_library().hw_concurrent_decode_tokens(
        ctx, layer, n_new, c_void_p(q_ptr), c_void_p(out_ptr),
        c_void_p(lse_ptr) if lse_ptr else None, c_void_p(stream)))


def hw_concurrent_decode_noalloc(ctx, layer: int, q_ptr: int, out_ptr: int,
                                 lse_ptr: Optional[int], stream: int) -> None:
    _check(ctx, load_library().hw_concurrent_decode_noalloc(
        ctx, layer, c_void_p(q_ptr), c_void_p(out_ptr), c_void_p(lse_ptr) if lse_ptr else None,
        c_void_p(stream)))


def hw_reset_block(ctx, block_id: int) -> None:
    _check(ctx, load_library().hw_reset_block(ctx, block_id))


def hw_plan_steps(ctx, n_steps: int, block_ids: Sequence[int], tokens_per_step: Sequence[int],
                  stream: int) -> None:
    _check(ctx, load_library().hw_plan_steps(ctx, n_steps, len(block_ids), _i32(block_ids),
                                             _i32(tokens_per_step), c_void_p(stream)))


def hw_append_step(ctx, layer: int, k_ptr: int, v_ptr: int, stream: int) -> None:
    _check(ctx, load_library().hw_append_step(ctx, layer, c_void_p(k_ptr), c_void_p(v_ptr),
                                              c_void_p(stream)))


def hw_decode_step(ctx, layer: int, k_ptr: int, v_ptr: int, q_ptr: int, out_ptr: int,
                   lse_ptr: Optional[int], stream: int) -> None:
    _check(ctx, load_library().hw_decode_step(ctx, layer, c_void_p(k_ptr), c_void_p(v_ptr),
                                              c_void_p(q_ptr), c_void_p(out_ptr),
                                              c_void_p(lse_ptr or 0), c_void_p(stream)))


def hw_plan_end(ctx, stream: int) -> None:
    _check(ctx, load_library().hw_plan_end(ctx, c_void_p(stream)))


def hw_set_split(ctx, n_splits: int) -> None:
    _check(ctx, load_library().hw_set_split(ctx, n_splits))


def hw_block_info(ctx, block_id: int, layer: int):
    lib = load_library()
    length, n = c_int32(), c_int32()
    _check(ctx, lib.hw_block_info(ctx, block_id, layer, ctypes.byref(length), None, 0, ctypes.byref(n)))
    pages = (c_int32 * max(1, n.value))()
    _check(ctx, lib.hw_block_info(ctx, block_id, layer, ctypes.byref(length), pages, n.value,
                                  ctypes.byref(n)))
    return length.value, list(pages[:n.value])


def hw_free_pages(ctx) -> int:
    n = c_int32()
    _check(ctx, load_library().hw_free_pages(ctx, ctypes.byref(n)))
    return n.value


def hw_debug_reserve(ctx, layer: int, block_ids, n_tokens, cap: int = 4096):
    runs = (c_int32 * (5 * cap))()
    n = c_int32()
    _check(ctx, load_library().hw_debug_reserve(ctx, layer, len(block_ids), _i32(block_ids),
                                                _i32(n_tokens), runs, cap, ctypes.byref(n)))
    return [tuple(runs[5 * i:5 * i + 5]) for i in range(n.value)]


def hw_debug_resolve(ctx, layer: int, n_workers: int, cap_segs: int = 4096,
                     cap_groups: int = 1 << 16):
    lib = load_library()
    n_seg, n_grp, n_split = c_int32(), c_int32(), c_int32()
    segs = (c_int32 * cap_segs)()
    # delta rows are n_workers wide; allocate for the largest plausible view set
    delta = (c_int32 * (cap_segs * 1024))()
    groups = (c_int32 * (4 * cap_groups))()
    _check(ctx, lib.hw_debug_resolve(ctx, layer, segs, delta, cap_segs, ctypes.byref(n_seg),
                                     groups, cap_groups, ctypes.byref(n_grp), ctypes.byref(n_split)))
    ns = n_seg.value
    return {"segs": list(segs[:ns]),
            "delta": [list(delta[s * n_workers:(s + 1) * n_workers]) for s in range(ns)],
            "n_segs": n_seg.value, "n_groups": n_grp.value, "n_splits": n_split.value,
            "groups": [tuple(groups[4 * i:4 * i + 4]) for i in range(n_grp.value)]}


def hw_debug_partition(block_first, n_splits: int, alpha: float):
    """Partition bounds (list of n_splits + 1 cuts) of a group list whose block starts are
    flagged in block_first (sequence of 0/1)."""
    lib = load_library()
    g = len(block_first)
    first = (ctypes.c_uint8 * max(1, g))(*[1 if x else 0 for x in block_first])
    out = (c_int32 * (n_splits + 1))()
    st = lib.hw_debug_partition(first if g else None, g, n_splits, ctypes.c_double(alpha), out)
    if st != HW_OK:
        raise HwError(st, lib.hw_last_error(None).decode())
    return list(out)


def hw_debug_kernel_events(ctx, capacity: int) -> None:
    _check(ctx, load_library().hw_debug_kernel_events(ctx, capacity))


def hw_debug_kernel_elapsed(ctx, cap: int = 1 << 16):
    dec = (c_float * cap)()
    n = c_int32()
    _check(ctx, load_library().hw_debug_kernel_elapsed(ctx, dec, cap, ctypes.byref(n)))
    return list(dec[:min(n.value, cap)])


def hw_debug_stream_read(src_ptr: int, nbytes: int, sink_ptr: int, n_blocks: int, stream,
                         timed: bool = False):
    """Enqueue the streaming-read probe; with timed, wait for it and return its duration in ms
    (from events recorded by its own dispatch)."""
    lib = load_library()
    ms = c_float()
    st = lib.hw_debug_stream_read(c_void_p(src_ptr), nbytes, c_void_p(sink_ptr), n_blocks,
                                  c_void_p(stream), ctypes.byref(ms) if timed else None)
    if st != HW_OK:
        raise HwError(st, lib.hw_last_error(None).decode())
    return ms.value if timed else None


# ---------------------------------------------------------------- owner

class HogwildCache:
    """Pools + workspace as torch device tensors, and a context over them."""

    def __init__(self, *, n_layers: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                 page_size: int, n_pages: int, max_blocks: int, max_workers: int,
                 max_position: int, kv_dtype: str = "bf16", page_seed: int = 0,
                 rope_theta: float = 1e4, softmax_scale: float = 0.0, max_splits: int = 0,
                 max_query_tokens: int = 0, device: str = "cuda"):
        import torch
        self.torch = torch
        load_library()
        self.kv_torch_dtype = {"bf16": torch.bfloat16, "f32": torch.float32}[kv_dtype]
        self.n_layers, self.n_q_heads, self.n_kv_heads = n_layers, n_q_heads, n_kv_heads
        self.head_dim, self.page_size, self.n_pages = head_dim, page_size, n_pages
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        elems = n_layers * n_pages * n_kv_heads * page_size * head_dim
        self.k_pool = torch.zeros(elems, dtype=self.kv_torch_dtype, device=self.device)
        self.v_pool = torch.zeros(elems, dtype=self.kv_torch_dtype, device=self.device)
        self.cfg = HwConfig(n_layers, n_q_heads, n_kv_heads, head_dim, page_size, n_pages,
                            max_blocks, max_workers, max_position, max_splits,
                            max_query_tokens, HW_BF16 if kv_dtype == "bf16" else HW_F32, page_seed,
                            rope_theta, softmax_scale, self.k_pool.data_ptr(),
                            self.v_pool.data_ptr())
        self.ctx = hw_create(self.cfg)
        nbytes = hw_workspace_bytes(self.ctx)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        hw_set_workspace(self.ctx, self.workspace.data_ptr(), nbytes)
        self.n_workers = 0

    def _stream(self) -> int:
        return self.torch.cuda.current_stream(self.device).cuda_stream

    def append(self, layer: int, block_ids: Sequence[int], n_tokens: Sequence[int], k, v) -> None:
        rows = int(sum(n_tokens))
        shape = (rows, self.n_kv_heads, self.head_dim)
        for t in (k, v):
            if t.dtype != self.kv_torch_dtype or tuple(t.shape) != shape or not t.is_contiguous() \
                    or t.device != self.device:
                raise HwError(HW_ERR_INVALID_ARG, f"k/v must be contiguous {self.kv_torch_dtype} "
                                                  f"{shape} on {self.device}")
        hw_append_kv(self.ctx, layer, block_ids, n_tokens, k.data_ptr(), v.data_ptr(), self._stream())

    def set_views(self, views, offsets=None, q_pos=None) -> None:
        hw_set_views(self.ctx, views, offsets, q_pos)
        self.n_workers = len(views)

    def _f32(self, name: str, t, shape) -> None:
        if t.dtype != self.torch.float32 or tuple(t.shape) != tuple(shape) or not t.is_contiguous() \
                or t.device != self.device:
            raise HwError(HW_ERR_INVALID_ARG, f"{name} must be contiguous float32 {tuple(shape)} "
                                              f"on {self.device}")

    def _io(self, q, out, lse, want_lse, shape):
        self._f32("q", q, shape)
        if out is None:
            out = self.torch.empty(shape, dtype=self.torch.float32, device=self.device)
        self._f32("out", out, shape)
        if lse is None and want_lse:
            lse = self.torch.empty(shape[:-1], dtype=self.torch.float32, device=self.device)
        if lse is not None:
            self._f32("lse", lse, shape[:-1])
        return out, lse

    def decode(self, layer: int, q, out=None, lse=None, want_lse: bool = True):
        """One query token per worker: q [n_workers, n_q_heads, head_dim] float32."""
        out, lse = self._io(q, out, lse, want_lse, (self.n_workers, self.n_q_heads, self.head_dim))
        hw_concurrent_decode(self.ctx, layer, q.data_ptr(), out.data_ptr(),
                             lse.data_ptr() if lse is not None else None, self._stream())
        return out, lse

    def decode_tokens(self, layer: int, q, out=None, lse=None, want_lse: bool = True):
        """n_new query tokens per worker, causal: q [n_workers, n_new, n_q_heads, head_dim]."""
        if q.dim() != 4:
            raise HwError(HW_ERR_INVALID_ARG, "q must be [n_workers, n_new, n_q_heads, head_dim]")
        n_new = int(q.shape[1])
        out, lse = self._io(q, out, lse, want_lse,
                            (self.n_workers, n_new, self.n_q_heads, self.head_dim))
        hw_concurrent_decode_tokens(self.ctx, layer, n_new, q.data_ptr(), out.data_ptr(),
                                    lse.data_ptr() if lse is not None else None, self._stream())
        return out, lse

    def plan_steps(self, n_steps: int, block_ids: Sequence[int], tokens_per_step: Sequence[int]) -> None:
        hw_plan_steps(self.ctx, n_steps, block_ids, tokens_per_step, self._stream())
        self.plan_rows = int(sum(tokens_per_step))

    def append_step(self, layer: int, k, v) -> None:
        """One planned step's tokens of one layer: k, v [rows, n_kv_heads, head_dim]."""
        self._kv_step(k, v)
        hw_append_step(self.ctx, layer, k.data_ptr(), v.data_ptr(), self._stream())

    def _kv_step(self, k, v) -> None:
        shape = (self.plan_rows, self.n_kv_heads, self.head_dim)
        for t in (k, v):
            if t.dtype != self.kv_torch_dtype or tuple(t.shape) != shape or not t.is_contiguous() \
                    or t.device != self.device:
                raise HwError(HW_ERR_INVALID_ARG, f"k/v must be contiguous {self.kv_torch_dtype} "
                                                  f"{shape} on {self.device}")

    def decode_step(self, layer: int, k, v, q, out=None, lse=None, want_lse: bool = True):
        """A planned step of one layer, append fused into the decode: k, v as append_step,
        q (and out, lse) as decode."""
        self._kv_step(k, v)
        out, lse = self._io(q, out, lse, want_lse, (self.n_workers, self.n_q_heads, self.head_dim))
        hw_decode_step(self.ctx, layer, k.data_ptr(), v.data_ptr(), q.data_ptr(), out.data_ptr(),
                       lse.data_ptr() if lse is not None else None, self._stream())
        return out, lse

    def plan_end(self) -> None:
        hw_plan_end(self.ctx, self._stream())

    def block_info(self, block: int, layer: int = 0):
        return hw_block_info(self.ctx, block, layer)

    def close(self) -> None:
        if getattr(self, "ctx", None) is not None:
            self.torch.cuda.synchronize(self.device)
            hw_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
