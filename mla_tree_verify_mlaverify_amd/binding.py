"""ctypes binding of libmlaverify.so (the C ABI in include/mlaverify.h).

Argument marshalling only: tensors are checked for dtype, shape, device and
layout, then their device pointers and the current HIP stream are passed to the
library.  Every step of the verify pass runs in the library's HIP kernels; there
is no fallback path.  torch provides device memory and streams.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# MLAVERIFY_LIBRARY may name another build of the same library (e.g. for A/B timing).
LIB_PATH = os.environ.get("MLAVERIFY_LIBRARY") or os.path.join(_PKG_DIR, "libmlaverify.so")

LATENT_DIM = 576
V_DIM = 512
MAX_TREE_NODES = 256

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_NO_MEMORY = -3
ERR_WORKSPACE = -4
ERR_HIP = -5

DEVERR_BAD_PARENT = 0x1
DEVERR_BAD_INDEX = 0x2
DEVERR_BAD_PREFIX = 0x4
DEVERR_RELOCATE_CONFLICT = 0x8
DEVERR_BAD_TREE_LEN = 0x10

FLAG_NO_FASTPATH = 0x1

# Every symbol include/mlaverify.h declares.
EXPORTED = (
    "mlaverify_validate_config",
    "mlaverify_workspace_bytes",
    "mlaverify_create",
    "mlaverify_run",
    "mlaverify_run_static",
    "mlaverify_run_ragged",
    "mlaverify_relocate",
    "mlaverify_accept",
    "mlaverify_tree_masks",
    "mlaverify_probe_gather",
    "mlaverify_read_plan",
    "mlaverify_read_device_errors",
    "mlaverify_profile_begin",
    "mlaverify_profile_end",
    "mlaverify_destroy",
    "mlaverify_status_string",
)


class MlaVerifyConfig(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("max_batch", ctypes.c_int32),
        ("max_tree_nodes", ctypes.c_int32),
        ("max_prefix_len", ctypes.c_int32),
        ("pool_slots", ctypes.c_int64),
        ("kv_row_stride", ctypes.c_int64),
        ("sm_scale", ctypes.c_float),
        ("split_tokens", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("page_size", ctypes.c_int32),
    ]


class MlaVerifyError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libmlaverify.so (built by mla_tree_verify_mlaverify_amd.build); raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with `python -m mla_tree_verify_mlaverify_amd.build` "
                          "(the HIP library is the only implementation)")
    lib = ctypes.CDLL(p)
    c_void_p, c_int32, c_size_t = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfg_p = ctypes.POINTER(MlaVerifyConfig)
    lib.mlaverify_validate_config.argtypes = [cfg_p]
    lib.mlaverify_validate_config.restype = ctypes.c_int
    lib.mlaverify_workspace_bytes.argtypes = [cfg_p]
    lib.mlaverify_workspace_bytes.restype = c_size_t
    lib.mlaverify_create.argtypes = [cfg_p, c_void_p, c_size_t, ctypes.POINTER(c_void_p)]
    lib.mlaverify_create.restype = ctypes.c_int
    lib.mlaverify_run.argtypes = [c_void_p, c_int32, c_int32] + [c_void_p] * 8
    lib.mlaverify_run.restype = ctypes.c_int
    lib.mlaverify_run_static.argtypes = [cfg_p, c_int32, c_int32] + [c_void_p] * 8
    lib.mlaverify_run_static.restype = ctypes.c_int
    lib.mlaverify_run_ragged.argtypes = [c_void_p, c_int32, c_int32] + [c_void_p] * 9
    lib.mlaverify_run_ragged.restype = ctypes.c_int
    lib.mlaverify_relocate.argtypes = [c_void_p, c_int32, c_int32] + [c_void_p] * 5
    lib.mlaverify_relocate.restype = ctypes.c_int
    lib.mlaverify_accept.argtypes = [c_void_p, c_int32, c_int32, c_int32] + [c_void_p] * 7
    lib.mlaverify_accept.restype = ctypes.c_int
    lib.mlaverify_tree_masks.argtypes = [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p]
    lib.mlaverify_tree_masks.restype = ctypes.c_int
    lib.mlaverify_probe_gather.argtypes = [c_void_p, ctypes.c_int64, ctypes.c_int64, c_void_p, c_int32, c_int32, c_int32,
                                           c_void_p, c_void_p]
    lib.mlaverify_probe_gather.restype = ctypes.c_int
    lib.mlaverify_read_plan.argtypes = [c_void_p, c_int32, c_void_p, ctypes.POINTER(c_int32), c_int32]
    lib.mlaverify_read_plan.restype = ctypes.c_int
    lib.mlaverify_read_device_errors.argtypes = [c_void_p, c_void_p, ctypes.POINTER(ctypes.c_uint32)]
    lib.mlaverify_read_device_errors.restype = ctypes.c_int
    lib.mlaverify_profile_begin.argtypes = [c_void_p, c_int32]
    lib.mlaverify_profile_begin.restype = ctypes.c_int
    lib.mlaverify_profile_end.argtypes = [c_void_p, ctypes.POINTER(ctypes.c_float), c_int32]
    lib.mlaverify_profile_end.restype = ctypes.c_int
    lib.mlaverify_destroy.argtypes = [c_void_p]
    lib.mlaverify_destroy.restype = ctypes.c_int
    lib.mlaverify_status_string.argtypes = [ctypes.c_int]
    lib.mlaverify_status_string.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load_library().mlaverify_status_string(status).decode()
    except ImportError:
        return "library not loaded"


def make_config(num_heads: int, max_batch: int, max_tree_nodes: int, max_prefix_len: int,
                pool_slots: int, kv_row_stride: int = LATENT_DIM, sm_scale: float = 1.0 / math.sqrt(192.0),
                split_tokens: int = 0, flags: int = 0, page_size: int = 0) -> MlaVerifyConfig:
    return MlaVerifyConfig(num_heads, max_batch, max_tree_nodes, max_prefix_len, pool_slots, kv_row_stride,
                           sm_scale, split_tokens, flags, page_size)


def validate_config(cfg: MlaVerifyConfig) -> int:
    return load_library().mlaverify_validate_config(ctypes.byref(cfg))


def workspace_bytes(cfg: MlaVerifyConfig) -> int:
    return load_library().mlaverify_workspace_bytes(ctypes.byref(cfg))


def _stream_handle(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(t: torch.Tensor, name: str, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class Verifier:
    """One library handle: DDTree tree-verify MLA attention on one GPU.

    The workspace is a torch allocation owned by this object (the library never
    allocates in run()), so run() can be captured into a HIP graph.
    """

    def __init__(self, num_heads: int, max_batch: int, max_tree_nodes: int, max_prefix_len: int,
                 pool_slots: int, kv_row_stride: int = LATENT_DIM, sm_scale: float = 1.0 / math.sqrt(192.0),
                 split_tokens: int = 0, flags: int = 0, page_size: int = 0, device=None):
        self.lib = load_library()
        self.cfg = make_config(num_heads, max_batch, max_tree_nodes, max_prefix_len, pool_slots, kv_row_stride,
                               sm_scale, split_tokens, flags, page_size)
        rc = self.lib.mlaverify_validate_config(ctypes.byref(self.cfg))
        if rc != OK:
            raise MlaVerifyError(rc, "invalid configuration")
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        nbytes = self.lib.mlaverify_workspace_bytes(ctypes.byref(self.cfg))
        with torch.cuda.device(self.device):
            self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            handle = ctypes.c_void_p()
            rc = self.lib.mlaverify_create(ctypes.byref(self.cfg), ctypes.c_void_p(self.workspace.data_ptr()),
                                           nbytes, ctypes.byref(handle))
        if rc != OK:
            raise MlaVerifyError(rc, "mlaverify_create")
        self.handle = handle
        self.num_heads = num_heads
        self.last_batch = None

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            try:
                self.lib.mlaverify_destroy(h)
            except Exception:  # interpreter shutdown
                pass
            self.handle = None

    def run(self, q, kv_pool, kv_indices, prefix_lens, tree_parent, out=None, lse=None, stream=None):
        """Verify attention for a batch; returns (out bf16 [B*T, H, 512], lse fp32 [B*T, H])."""
        b, t = tree_parent.shape if tree_parent.dim() == 2 else (None, None)
        if b is None:
            raise ValueError("tree_parent must be [batch, T]")
        h = self.num_heads
        dev = self.device
        _check(tree_parent, "tree_parent", torch.int32, (b, t), dev)
        _check(q, "q", torch.bfloat16, (b * t, h, LATENT_DIM), dev)
        _check(prefix_lens, "prefix_lens", torch.int32, (b,), dev)
        _check(kv_indices, "kv_indices", torch.int32, None, dev)
        if kv_indices.dim() != 1:
            raise ValueError("kv_indices must be 1-D")
        _check(kv_pool, "kv_pool", torch.bfloat16, (self.cfg.pool_slots, self.cfg.kv_row_stride), dev)
        if out is None:
            out = torch.empty((b * t, h, V_DIM), dtype=torch.bfloat16, device=dev)
        if lse is None:
            lse = torch.empty((b * t, h), dtype=torch.float32, device=dev)
        _check(out, "out", torch.bfloat16, (b * t, h, V_DIM), dev)
        _check(lse, "lse", torch.float32, (b * t, h), dev)
        with torch.cuda.device(dev):  # the library launches on its handle's device only
            rc = self.lib.mlaverify_run(self.handle, b, t, q.data_ptr(), kv_pool.data_ptr(), kv_indices.data_ptr(),
                                        prefix_lens.data_ptr(), tree_parent.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                        _stream_handle(stream))
        if rc != OK:
            raise MlaVerifyError(rc, "mlaverify_run")
        self.last_batch = b
        return out, lse

    def run_ragged(self, q, kv_pool, kv_indices, prefix_lens, tree_lens, tree_parent, max_tree_nodes: int,
                   out=None, lse=None, stream=None):
        """Verify attention for requests with trees of different sizes (mlaverify_run_ragged):
        tree_lens int32 [B] on the device, rows packed request after request; max_tree_nodes is
        the largest tree length of the call (a host int).  Returns (out [sum T_b, H, 512],
        lse [sum T_b, H]); the caller gives the row count through q's first dimension."""
        h = self.num_heads
        dev = self.device
        _check(tree_lens, "tree_lens", torch.int32, None, dev)
        if tree_lens.dim() != 1:
            raise ValueError("tree_lens must be 1-D")
        b = tree_lens.shape[0]
        if q.dim() != 3:
            raise ValueError("q must be [sum T_b, H, 576]")
        rows = q.shape[0]
        _check(q, "q", torch.bfloat16, (rows, h, LATENT_DIM), dev)
        _check(tree_parent, "tree_parent", torch.int32, (rows,), dev)
        _check(prefix_lens, "prefix_lens", torch.int32, (b,), dev)
        _check(kv_indices, "kv_indices", torch.int32, None, dev)
        if kv_indices.dim() != 1:
            raise ValueError("kv_indices must be 1-D")
        _check(kv_pool, "kv_pool", torch.bfloat16, (self.cfg.pool_slots, self.cfg.kv_row_stride), dev)
        if out is None:
            out = torch.empty((rows, h, V_DIM), dtype=torch.bfloat16, device=dev)
        if lse is None:
            lse = torch.empty((rows, h), dtype=torch.float32, device=dev)
        _check(out, "out", torch.bfloat16, (rows, h, V_DIM), dev)
        _check(lse, "lse", torch.float32, (rows, h), dev)
        with torch.cuda.device(dev):
            rc = self.lib.mlaverify_run_ragged(self.handle, b, max_tree_nodes, tree_lens.data_ptr(), q.data_ptr(),
                                               kv_pool.data_ptr(), kv_indices.data_ptr(), prefix_lens.data_ptr(),
                                               tree_parent.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                               _stream_handle(stream))
        if rc != OK:
            raise MlaVerifyError(rc, "mlaverify_run_ragged")
        self.last_batch = b
        return out, lse

    def relocate(self, kv_pool, kv_indices, prefix_lens, dst_start, tree_nodes: int, stream=None) -> None:
        """Tier-1 relocation of the batch's prefix rows into the runs starting at dst_start
        (in place on kv_pool and kv_indices; refusals show in read_device_errors)."""
        dev = self.device
        _check(prefix_lens, "prefix_lens", torch.int32, None, dev)
        if prefix_lens.dim() != 1:
            raise ValueError("prefix_lens must be 1-D")
        b = prefix_lens.shape[0]
        _check(dst_start, "dst_start", torch.int32, (b,), dev)
        _check(kv_indices, "kv_indices", torch.int32, None, dev)
        if kv_indices.dim() != 1:
            raise ValueError("kv_indices must be 1-D")
        _check(kv_pool, "kv_pool", torch.bfloat16, (self.cfg.pool_slots, self.cfg.kv_row_stride), dev)
        with torch.cuda.device(dev):  # the library launches on its handle's device only
            rc = self.lib.mlaverify_relocate(self.handle, b, tree_nodes, kv_pool.data_ptr(), kv_indices.data_ptr(),
                                             prefix_lens.data_ptr(), dst_start.data_ptr(), _stream_handle(stream))
        if rc != OK:
            raise MlaVerifyError(rc, "mlaverify_relocate")

    def accept(self, logits, draft_tokens, tree_parent, stream=None):
        """Greedy acceptance of a verified tree; returns (accept_len [B], accepted [B, T], bonus [B]).
        Invalid trees show in read_device_errors."""
        dev = self.device
        if tree_parent.dim() != 2:
            raise ValueError("tree_parent must be [batch, T]")
        b, t = tree_parent.shape
        _check(tree_parent, "tree_parent", torch.int32, (b, t), dev)
        _check(draft_tokens, "draft_tokens", torch.int32, (b, t), dev)
        if logits.dim() != 3 or logits.shape[0] != b or logits.shape[1] != t + 1:
            raise ValueError(f"logits must be [batch, T + 1, vocab] = [{b}, {t + 1}, V]")
        _check(logits, "logits", torch.float32, None, dev)
        accept_len = torch.empty(b, dtype=torch.int32, device=dev)
        accepted = torch.empty((b, t), dtype=torch.int32, device=dev)
        bonus = torch.empty(b, dtype=torch.int32, device=dev)
        with torch.cuda.device(dev):  # the library launches on its handle's device only
            rc = self.lib.mlaverify_accept(self.handle, b, t, logits.shape[2], logits.data_ptr(), draft_tokens.data_ptr(),
                                           tree_parent.data_ptr(), accept_len.data_ptr(), accepted.data_ptr(),
                                           bonus.data_ptr(), _stream_handle(stream))
        if rc != OK:
            raise MlaVerifyError(rc, "mlaverify_accept")
        return accept_len, accepted, bonus

    def read_plan(self, batch: int | None = None, stream=None) -> dict:
        """Work partition of the last run (synchronises the stream)."""
        batch = batch or self.last_batch
        cap = 6 + 5 * batch
        buf = (ctypes.c_int32 * cap)()
        n = self.lib.mlaverify_read_plan(self.handle, batch, _stream_handle(stream), buf, cap)
        if n < 0:
            raise MlaVerifyError(n, "mlaverify_read_plan")
        vals = list(buf)
        reqs = [dict(zip(("key_offset", "prefix_len", "first_unit", "units", "error_bits"), vals[6 + 5 * i:11 + 5 * i]))
                for i in range(batch)]
        return dict(split_len=vals[0], total_units=vals[1], n_mtiles=vals[2], fast_units=vals[3],
                    sclk_mhz=round(vals[4] / 1000.0, 1), rescales=vals[5], requests=reqs)

    def profile_begin(self, max_runs: int) -> None:
        """Record HIP events around the kernels of the next max_runs runs."""
        rc = self.lib.mlaverify_profile_begin(self.handle, max_runs)
        if rc != OK:
            raise MlaVerifyError(rc, "mlaverify_profile_begin")
        self._prof_cap = max_runs

    def profile_end(self):
        """Per recorded run: (partial_ms, merge_ms); synchronises."""
        cap = getattr(self, "_prof_cap", 0)
        buf = (ctypes.c_float * (2 * max(cap, 1)))()
        n = self.lib.mlaverify_profile_end(self.handle, buf, cap)
        if n < 0:
            raise MlaVerifyError(n, "mlaverify_profile_end")
        return [tuple(buf[2 * i:2 * i + 2]) for i in range(min(n, cap))]

    def read_device_errors(self, stream=None) -> int:
        """Sticky device-side data-error bits since the last call (synchronises the stream)."""
        flags = ctypes.c_uint32()
        rc = self.lib.mlaverify_read_device_errors(self.handle, _stream_handle(stream), ctypes.byref(flags))
        if rc != OK:
            raise MlaVerifyError(rc, "mlaverify_read_device_errors")
        return flags.value


def probe_gather(kv_pool, indices, lds_path: bool, grid: int, sink, pool_slots: int | None = None, stream=None) -> None:
    """One launch of the scattered-row read probe (mlaverify_probe_gather): reads kv_pool[indices]
    into registers (lds_path False) or into LDS (True); sink (uint32 [grid * 256]) keeps the loads live."""
    lib = load_library()
    dev = kv_pool.device
    _check(kv_pool, "kv_pool", torch.bfloat16, None, dev)
    _check(indices, "indices", torch.int32, None, dev)
    _check(sink, "sink", torch.int32, (grid * 256,), dev)
    slots, stride = kv_pool.shape
    with torch.cuda.device(dev):
        rc = lib.mlaverify_probe_gather(kv_pool.data_ptr(), stride, pool_slots or slots, indices.data_ptr(),
                                        indices.numel(), 1 if lds_path else 0, grid, sink.data_ptr(),
                                        _stream_handle(stream))
    if rc != OK:
        raise MlaVerifyError(rc, "mlaverify_probe_gather")


STATIC_SCRATCH_BYTES = 48 << 20


def run_static(cfg: MlaVerifyConfig, q, kv_pool, kv_indices, prefix_lens, tree_parent, out, lse, stream=None) -> None:
    """The verify pass over the library's static workspace (mlaverify_run_static): no handle,
    nothing allocated by the library or here; out and lse are written in place."""
    lib = load_library()
    if tree_parent.dim() != 2:
        raise ValueError("tree_parent must be [batch, T]")
    b, t = tree_parent.shape
    h = cfg.num_heads
    dev = q.device
    _check(tree_parent, "tree_parent", torch.int32, (b, t), dev)
    _check(q, "q", torch.bfloat16, (b * t, h, LATENT_DIM), dev)
    _check(prefix_lens, "prefix_lens", torch.int32, (b,), dev)
    _check(kv_indices, "kv_indices", torch.int32, None, dev)
    if kv_indices.dim() != 1:
        raise ValueError("kv_indices must be 1-D")
    _check(kv_pool, "kv_pool", torch.bfloat16, (cfg.pool_slots, cfg.kv_row_stride), dev)
    _check(out, "out", torch.bfloat16, (b * t, h, V_DIM), dev)
    _check(lse, "lse", torch.float32, (b * t, h), dev)
    with torch.cuda.device(dev):
        rc = lib.mlaverify_run_static(ctypes.byref(cfg), b, t, q.data_ptr(), kv_pool.data_ptr(), kv_indices.data_ptr(),
                                      prefix_lens.data_ptr(), tree_parent.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                      _stream_handle(stream))
    if rc != OK:
        raise MlaVerifyError(rc, "mlaverify_run_static")


def tree_masks(tree_parent: torch.Tensor, stream=None):
    """Ancestor-or-self bitmasks on the GPU: returns (masks int64 [B, T, ceil(T/64)] holding the uint64
    words, err int32 [B])."""
    lib = load_library()
    if tree_parent.dim() != 2:
        raise ValueError("tree_parent must be [batch, T]")
    b, t = tree_parent.shape
    _check(tree_parent, "tree_parent", torch.int32, (b, t))
    masks = torch.empty((b, t, (t + 63) // 64), dtype=torch.int64, device=tree_parent.device)
    err = torch.empty((b,), dtype=torch.int32, device=tree_parent.device)
    rc = lib.mlaverify_tree_masks(tree_parent.data_ptr(), b, t, masks.data_ptr(), err.data_ptr(),
                                  _stream_handle(stream))
    if rc != OK:
        raise MlaVerifyError(rc, "mlaverify_tree_masks")
    return masks, err
