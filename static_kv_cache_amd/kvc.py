"""Thin ctypes binding over libkvc.so (the C ABI declared in include/kvc.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of the library. torch is used for device memory (tensors are passed
by ``data_ptr()``) and for the current stream handle. The binding checks
tensor shapes, dtypes, devices and contiguity before any call so that a
kernel never sees a buffer smaller than its launch assumes.

If the library has not been built, every call raises ``RuntimeError``:
there is no fallback path.
"""

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvc.so")

KVC_OK, KVC_ERR_INVALID_ARG, KVC_ERR_CAPACITY, KVC_ERR_OOM = 0, 1, 2, 3
KVC_ERR_DEVICE, KVC_ERR_UNSUPPORTED, KVC_ERR_DEVICE_RANGE = 4, 5, 6
KVC_F32, KVC_BF16, KVC_I8 = 0, 1, 2
KVC_ATTN_GQA, KVC_ATTN_MLA = 0, 1

_DTYPES = {"f32": KVC_F32, "bf16": KVC_BF16, "i8": KVC_I8}


class Desc(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "attn", "dtype", "n_layers", "batch", "n_heads", "n_kv_heads", "head_dim",
        "max_context", "latent_dim", "rope_dim")]

    def __repr__(self):
        return "Desc(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class KvcError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib.kvc_strerror(status).decode() if _lib is not None else str(status)
        super().__init__(f"{where}: {msg} (status {status})")


_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_SIGS = {
    "kvc_bytes": [ctypes.POINTER(Desc), ctypes.POINTER(ctypes.c_uint64)],
    "kvc_alloc": [ctypes.POINTER(Desc), _p, ctypes.POINTER(_p)],
    "kvc_free": [_p],
    "kvc_layer_ptrs": [_p, _i32, ctypes.POINTER(_p), ctypes.POINTER(_p)],
    "kvc_layer_scales": [_p, _i32, ctypes.POINTER(_p), ctypes.POINTER(_p)],
    "kvc_logical_bytes": [_p, _p, ctypes.POINTER(ctypes.c_uint64)],
    "kvc_prefill_fill": [_p, _i32, _p, _p, _i32, _i32, _p],
    "kvc_append": [_p, _i32, _p, _p, _p, _i32, _p],
    "kvc_decode_attn": [_p, _i32, _p, _p, _p, _p, ctypes.c_float, _p],
    "kvc_decode_attn_noalloc": [ctypes.POINTER(Desc), _p, _p, _p, _p, _p, _p, ctypes.c_float, _p, _p],
    "kvc_mla_decode": [_p, _i32, _p, _p, _p, _p, _p, _p, _p, ctypes.c_float, _p],
    "kvc_append_decode_attn": [_p, _i32, _p, _p, _p, _p, _p, ctypes.c_float, _p],
    "kvc_prefill_attn": [_p, _i32, _p, _p, _p, _p, _i32, _i32, ctypes.c_float, _p],
    "kvc_bytes_paged": [ctypes.POINTER(Desc), _i32, _i32, ctypes.POINTER(ctypes.c_uint64)],
    "kvc_alloc_paged": [ctypes.POINTER(Desc), _i32, _i32, _p, ctypes.POINTER(_p)],
    "kvc_paged_append": [_p, _i32, _p, _p, _p, _p, _i32, _p],
    "kvc_paged_decode_attn": [_p, _i32, _p, _p, _p, _p, _p, ctypes.c_float, _p],
    "kvc_paged_append_decode_attn": [_p, _i32, _p, _p, _p, _p, _p, _p, ctypes.c_float, _p],
    "kvc_prefix_bytes": [_p, _p, ctypes.POINTER(ctypes.c_uint64)],
    "kvc_save_prefix": [_p, _p, _p, ctypes.c_uint64, _p],
    "kvc_load_prefix": [_p, _p, ctypes.c_uint64, _p, _p, _p],
    "kvc_set_workgroups": [_p, _i32],
    "kvc_get_workgroups": [_p, ctypes.POINTER(_i32), ctypes.POINTER(_i32)],
    "kvc_check": [_p, _p],
    "kvc_strerror": [ctypes.c_int],
}

_lib = None


def load(path=LIB_PATH):
    """Open libkvc.so and bind every entry point (raises if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
    # torch ships its own HIP runtime with the same soname; importing it first
    # makes libkvc.so bind to that one, so the process has a single runtime and
    # torch's streams and allocations are valid handles for the library.
    _torch()
    lib = ctypes.CDLL(path)
    lib.hipMemcpyAsync.argtypes = [_p, _p, ctypes.c_size_t, ctypes.c_int, _p]
    lib.hipMemcpyAsync.restype = ctypes.c_int
    for name, args in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "kvc_strerror" else ctypes.c_int
    _lib = lib
    return lib


def _call(name, *args):
    st = getattr(load(), name)(*args)
    if st != KVC_OK:
        raise KvcError(st, name)


def gqa_desc(n_layers, batch, n_heads, n_kv_heads, head_dim, max_context, dtype):
    return Desc(KVC_ATTN_GQA, _DTYPES[dtype], n_layers, batch, n_heads, n_kv_heads, head_dim,
                max_context, 0, 0)


def mla_desc(n_layers, batch, n_heads, max_context, latent_dim=512, rope_dim=64, head_dim=128,
             dtype="bf16"):
    return Desc(KVC_ATTN_MLA, _DTYPES[dtype], n_layers, batch, n_heads, 1, head_dim, max_context,
                latent_dim, rope_dim)


def cache_bytes(desc):
    out = ctypes.c_uint64(0)
    _call("kvc_bytes", ctypes.byref(desc), ctypes.byref(out))
    return out.value


def _torch():
    import torch
    return torch


def torch_dtype(dtype):
    """Storage element type of a cache dtype ("i8": the int8 codes)."""
    torch = _torch()
    return {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8}[dtype]


def io_dtype(dtype):
    """Type of the tensors handed to and from a cache of `dtype` (bf16 for an int8 cache)."""
    return "bf16" if dtype == "i8" else dtype


def to_device(a, device):
    """numpy (uint16 bf16 bits / float32 / int32) -> contiguous torch tensor on device."""
    torch = _torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    elif a.dtype in (np.float32, np.int32):
        t = torch.from_numpy(a)
    else:
        raise TypeError(f"unsupported array dtype {a.dtype}")
    return t.to(device)


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


class Cache:
    """One static cache (all layers) allocated once on the current device."""

    def __init__(self, desc, external=None):
        torch = _torch()
        self.desc = desc
        self.dtype = {KVC_F32: "f32", KVC_BF16: "bf16", KVC_I8: "i8"}[desc.dtype]
        self.io_dtype = io_dtype(self.dtype)
        self.device = torch.device("cuda", torch.cuda.current_device())
        self.nbytes = cache_bytes(desc)
        self._external = external
        ext = None
        if external is not None:
            if not (external.is_cuda and external.is_contiguous()
                    and external.numel() * external.element_size() >= self.nbytes):
                raise ValueError("external buffer must be a contiguous device tensor of >= kvc_bytes")
            ext = ctypes.c_void_p(external.data_ptr())
        h = ctypes.c_void_p()
        _call("kvc_alloc", ctypes.byref(desc), ext, ctypes.byref(h))
        self._h = h

    # -- shape helpers -------------------------------------------------------
    @property
    def is_mla(self):
        return self.desc.attn == KVC_ATTN_MLA

    @property
    def row_width(self):
        d = self.desc
        return d.latent_dim + d.rope_dim if self.is_mla else d.head_dim

    def _check(self, t, shape, dtype=None, name="tensor"):
        torch = _torch()
        want = torch_dtype(self.io_dtype) if dtype is None else dtype
        if t.device != self.device:
            raise ValueError(f"{name} must be on {self.device}, got {t.device}")
        if t.dtype != want:
            raise ValueError(f"{name} must be {want}, got {t.dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        if not t.is_contiguous() or t.data_ptr() % 16 != 0:
            raise ValueError(f"{name} must be contiguous and 16-byte aligned")
        return ctypes.c_void_p(t.data_ptr())

    def _idx(self, t, name):
        if t is None:
            return None
        return self._check(t, (self.desc.batch,), _torch().int32, name)

    @property
    def handle(self):
        if self._h is None:
            raise RuntimeError("cache already freed")
        return self._h

    # -- C ABI calls ---------------------------------------------------------
    def layer_ptrs(self, layer):
        k, v = ctypes.c_void_p(), ctypes.c_void_p()
        _call("kvc_layer_ptrs", self.handle, layer, ctypes.byref(k), ctypes.byref(v))
        return k.value, v.value

    def layer_tensors(self, layer):
        """Copies of one layer's region as torch tensors (K, V) or (rows, None)."""
        torch = _torch()
        d = self.desc
        k_ptr, v_ptr = self.layer_ptrs(layer)
        shape = (d.batch, d.max_context, self.row_width) if self.is_mla else \
            (d.batch, d.n_kv_heads, d.max_context, d.head_dim)
        n = int(np.prod(shape))
        out = []
        for ptr in (k_ptr, v_ptr):
            if ptr is None:
                out.append(None)
                continue
            t = torch.empty(shape, dtype=torch_dtype(self.dtype), device=self.device)
            _memcpy_d2d(t.data_ptr(), ptr, n * t.element_size(), self.device)
            out.append(t)
        return tuple(out)

    def layer_scales(self, layer):
        """Copies of one layer's row scales of an int8 cache: (K, V) float32 [B, H_kv, S]."""
        torch = _torch()
        d = self.desc
        k, v = ctypes.c_void_p(), ctypes.c_void_p()
        _call("kvc_layer_scales", self.handle, layer, ctypes.byref(k), ctypes.byref(v))
        out = []
        for ptr in (k.value, v.value):
            t = torch.empty((d.batch, d.n_kv_heads, d.max_context), dtype=torch.float32, device=self.device)
            _memcpy_d2d(t.data_ptr(), ptr, t.numel() * 4, self.device)
            out.append(t)
        return tuple(out)

    def logical_bytes(self, valid_lens):
        v = np.ascontiguousarray(valid_lens, dtype=np.int32)
        if v.shape != (self.desc.batch,):
            raise ValueError("valid_lens must have shape [B]")
        out = ctypes.c_uint64(0)
        _call("kvc_logical_bytes", self.handle, v.ctypes.data_as(ctypes.c_void_p), ctypes.byref(out))
        return out.value

    def prefill_fill(self, layer, k, v, start):
        d = self.desc
        if self.is_mla:
            t = k.shape[1]
            kp = self._check(k, (d.batch, t, self.row_width), name="rows")
            if v is not None:
                raise ValueError("latent cache takes no v")
            vp = None
        else:
            t = k.shape[2]
            shape = (d.batch, d.n_kv_heads, t, d.head_dim)
            kp, vp = self._check(k, shape, name="k"), self._check(v, shape, name="v")
        _call("kvc_prefill_fill", self.handle, layer, kp, vp, start, t, _stream(self.device))

    def append(self, layer, k_new, v_new, cache_index):
        d = self.desc
        if self.is_mla:
            t = k_new.shape[1]
            kp = self._check(k_new, (d.batch, t, self.row_width), name="rows_new")
            if v_new is not None:
                raise ValueError("latent cache takes no v_new")
            vp = None
        else:
            t = k_new.shape[2]
            shape = (d.batch, d.n_kv_heads, t, d.head_dim)
            kp, vp = self._check(k_new, shape, name="k_new"), self._check(v_new, shape, name="v_new")
        ci = self._idx(cache_index, "cache_index")
        _call("kvc_append", self.handle, layer, kp, vp, ci, t, _stream(self.device))

    def decode_attn(self, layer, q, out, valid_lens=None, cache_index=None, sm_scale=None):
        d = self.desc
        if self.is_mla:
            qp = self._check(q, (d.batch, d.n_heads, self.row_width), name="q")
            op = self._check(out, (d.batch, d.n_heads, d.latent_dim), name="out")
        else:
            qp = self._check(q, (d.batch, d.n_heads, d.head_dim), name="q")
            op = self._check(out, (d.batch, d.n_heads, d.head_dim), name="out")
        if sm_scale is None:
            raise ValueError("sm_scale is required")
        _call("kvc_decode_attn", self.handle, layer, qp, op, self._idx(valid_lens, "valid_lens"),
              self._idx(cache_index, "cache_index"), float(sm_scale), _stream(self.device))

    def append_decode_attn(self, layer, k_new, v_new, q, out, cache_index, sm_scale):
        """One launch: append the new row at cache_index, then attend rows
        [0, cache_index + 1) (kvc_append_decode_attn; GQA caches)."""
        d = self.desc
        shape = (d.batch, d.n_kv_heads, 1, d.head_dim)
        kp, vp = self._check(k_new, shape, name="k_new"), self._check(v_new, shape, name="v_new")
        qp = self._check(q, (d.batch, d.n_heads, d.head_dim), name="q")
        op = self._check(out, (d.batch, d.n_heads, d.head_dim), name="out")
        _call("kvc_append_decode_attn", self.handle, layer, kp, vp, qp, op, self._idx(cache_index, "cache_index"),
              float(sm_scale), _stream(self.device))

    def prefill_attn(self, layer, q, k, v, out, start, sm_scale):
        """Write the chunk's rows [start, start + t) and compute its causal attention
        (kvc_prefill_attn): q, out [B, H, t, D]; k, v [B, H_kv, t, D]."""
        d = self.desc
        t = q.shape[2]
        qp = self._check(q, (d.batch, d.n_heads, t, d.head_dim), name="q")
        op = self._check(out, (d.batch, d.n_heads, t, d.head_dim), name="out")
        shape = (d.batch, d.n_kv_heads, t, d.head_dim)
        kp, vp = self._check(k, shape, name="k"), self._check(v, shape, name="v")
        _call("kvc_prefill_attn", self.handle, layer, qp, kp, vp, op, start, t, float(sm_scale),
              _stream(self.device))

    def mla_decode(self, layer, q_nope, q_rope, w_uk, w_uv, out, valid_lens=None, cache_index=None,
                   sm_scale=None):
        d = self.desc
        B, H, dn, dc, dr = d.batch, d.n_heads, d.head_dim, d.latent_dim, d.rope_dim
        args = [self._check(q_nope, (B, H, dn), name="q_nope"),
                self._check(q_rope, (B, H, dr), name="q_rope"),
                self._check(w_uk, (H, dn, dc), name="w_uk"),
                self._check(w_uv, (H, dc, dn), name="w_uv"),
                self._check(out, (B, H, dn), name="out")]
        if sm_scale is None:
            raise ValueError("sm_scale is required")
        _call("kvc_mla_decode", self.handle, layer, *args, self._idx(valid_lens, "valid_lens"),
              self._idx(cache_index, "cache_index"), float(sm_scale), _stream(self.device))

    # -- live-prefix image (kvc_prefix_bytes / kvc_save_prefix / kvc_load_prefix) --
    def _host_lens(self, valid_lens):
        v = np.ascontiguousarray(valid_lens, dtype=np.int32)
        if v.shape != (self.desc.batch,):
            raise ValueError("valid_lens must have shape [B]")
        return v

    def _image_ptr(self, image):
        torch = _torch()
        if image.dtype != torch.uint8 or image.dim() != 1 or not image.is_contiguous():
            raise ValueError("image must be a contiguous 1-D uint8 tensor")
        if image.device.type == "cpu" and not image.is_pinned():
            raise ValueError("a host image must be pinned memory")
        if image.device.type != "cpu" and image.device != self.device:
            raise ValueError(f"image must be on {self.device} or pinned host memory")
        if image.data_ptr() % 16 != 0:
            raise ValueError("image must be 16-byte aligned")
        return ctypes.c_void_p(image.data_ptr()), image.numel()

    def prefix_bytes(self, valid_lens):
        v = self._host_lens(valid_lens)
        out = ctypes.c_uint64(0)
        _call("kvc_prefix_bytes", self.handle, v.ctypes.data_as(ctypes.c_void_p), ctypes.byref(out))
        return out.value

    def save_prefix(self, valid_lens, dst=None):
        """Image of rows [0, valid_lens[b]) of every layer and sequence (kvc_save_prefix), as a uint8
        tensor: `dst` if given (device or pinned host), else a new device tensor."""
        torch = _torch()
        v = self._host_lens(valid_lens)
        n = self.prefix_bytes(v)
        if dst is None:
            dst = torch.empty(n, dtype=torch.uint8, device=self.device)
        ptr, size = self._image_ptr(dst)
        _call("kvc_save_prefix", self.handle, v.ctypes.data_as(ctypes.c_void_p), ptr, size, _stream(self.device))
        return dst

    def load_prefix(self, image, src_seq=None, valid_lens=None):
        """Load an image (kvc_load_prefix): sequence b gets saved sequence src_seq[b] (-1: untouched;
        default b -> b). Returns the valid lengths: the loaded ones, and valid_lens[b] (default -1)
        where src_seq[b] = -1."""
        B = self.desc.batch
        src = np.arange(B, dtype=np.int32) if src_seq is None else self._host_lens(src_seq)
        lens = np.full(B, -1, dtype=np.int32) if valid_lens is None else self._host_lens(valid_lens).copy()
        ptr, size = self._image_ptr(image)
        _call("kvc_load_prefix", self.handle, ptr, size, src.ctypes.data_as(ctypes.c_void_p),
              lens.ctypes.data_as(ctypes.c_void_p), _stream(self.device))
        return lens

    def set_workgroups(self, n):
        """Force the persistent attention grid size (0 = device default)."""
        _call("kvc_set_workgroups", self.handle, n)

    def workgroups(self):
        """(forced count or 0, largest accepted count)."""
        n, mx = ctypes.c_int32(0), ctypes.c_int32(0)
        _call("kvc_get_workgroups", self.handle, ctypes.byref(n), ctypes.byref(mx))
        return n.value, mx.value

    def check(self):
        """Synchronise the current stream; raise KvcError on a device-range or HIP error."""
        _call("kvc_check", self.handle, _stream(self.device))

    def check_status(self):
        """Like check() but return the status code instead of raising."""
        return load().kvc_check(self.handle, _stream(self.device))

    def free(self):
        if self._h is not None:
            _call("kvc_free", self._h)
            self._h = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def decode_attn_noalloc(desc, k_layer, v_layer, q, out, valid_lens=None, cache_index=None, sm_scale=None,
                        err_flag=None):
    """kvc_decode_attn_noalloc: decode attention over one GQA layer the caller
    holds (k_layer, v_layer [B][H_kv][max_context][d_h], bf16 or fp32), with
    the library's static workspace (no allocation). err_flag: optional device
    int32 tensor of one element that the kernels set on an out-of-range
    length."""
    torch = _torch()
    dtype = {KVC_F32: "f32", KVC_BF16: "bf16"}.get(desc.dtype)
    if dtype is None:
        raise ValueError("decode_attn_noalloc takes bf16 or fp32 GQA shapes")
    want = torch_dtype(dtype)
    dev = q.device

    def ptr(t, shape, dt, name):
        if t is None:
            return None
        if t.device != dev or t.dtype != dt or tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must be {dt} of shape {tuple(shape)} on {dev}")
        if not t.is_contiguous() or t.data_ptr() % 16 != 0:
            raise ValueError(f"{name} must be contiguous and 16-byte aligned")
        return ctypes.c_void_p(t.data_ptr())

    kv = (desc.batch, desc.n_kv_heads, desc.max_context, desc.head_dim)
    qo = (desc.batch, desc.n_heads, desc.head_dim)
    if sm_scale is None:
        raise ValueError("sm_scale is required")
    _call("kvc_decode_attn_noalloc", ctypes.byref(desc), ptr(k_layer, kv, want, "k_layer"),
          ptr(v_layer, kv, want, "v_layer"), ptr(q, qo, want, "q"), ptr(out, qo, want, "out"),
          ptr(valid_lens, (desc.batch,), torch.int32, "valid_lens"),
          ptr(cache_index, (desc.batch,), torch.int32, "cache_index"), float(sm_scale),
          ptr(err_flag, (1,), torch.int32, "err_flag"), _stream(dev))


def paged_cache_bytes(desc, block_size, num_blocks):
    out = ctypes.c_uint64(0)
    _call("kvc_bytes_paged", ctypes.byref(desc), block_size, num_blocks, ctypes.byref(out))
    return out.value


class PagedCache(Cache):
    """A block-table cache (kvc_alloc_paged): per layer, K and V pools
    [num_blocks, H_kv, block_size, D] (bf16); block tables [B, max_context // block_size]
    int32 are passed per call. Only the paged calls (and the shared ones: layer
    pointers, workgroups, check, free) apply."""

    def __init__(self, desc, block_size, num_blocks, external=None):
        torch = _torch()
        self.desc = desc
        self.dtype = {KVC_F32: "f32", KVC_BF16: "bf16", KVC_I8: "i8"}[desc.dtype]
        self.io_dtype = io_dtype(self.dtype)
        self.device = torch.device("cuda", torch.cuda.current_device())
        self.block_size = block_size
        self.num_blocks = num_blocks
        self.table_width = desc.max_context // block_size
        self.nbytes = paged_cache_bytes(desc, block_size, num_blocks)
        self._external = external
        ext = None
        if external is not None:
            if not (external.is_cuda and external.is_contiguous()
                    and external.numel() * external.element_size() >= self.nbytes):
                raise ValueError("external buffer must be a contiguous device tensor of >= kvc_bytes_paged")
            ext = ctypes.c_void_p(external.data_ptr())
        h = ctypes.c_void_p()
        _call("kvc_alloc_paged", ctypes.byref(desc), block_size, num_blocks, ext, ctypes.byref(h))
        self._h = h

    def layer_tensors(self, layer):
        """Copies of one layer's pools (K, V) as [num_blocks, H_kv, block_size, D] tensors."""
        torch = _torch()
        d = self.desc
        shape = (self.num_blocks, d.n_kv_heads, self.block_size, d.head_dim)
        out = []
        for ptr in self.layer_ptrs(layer):
            t = torch.empty(shape, dtype=torch_dtype(self.dtype), device=self.device)
            _memcpy_d2d(t.data_ptr(), ptr, t.numel() * t.element_size(), self.device)
            out.append(t)
        return tuple(out)

    def _table(self, table):
        return self._check(table, (self.desc.batch, self.table_width), _torch().int32, "block_table")

    def paged_append(self, layer, k_new, v_new, block_table, cache_index):
        """Write rows [cache_index[b], cache_index[b] + t) of each sequence through its table
        (kvc_paged_append): k_new, v_new [B, H_kv, t, D]."""
        d = self.desc
        t = k_new.shape[2]
        shape = (d.batch, d.n_kv_heads, t, d.head_dim)
        kp, vp = self._check(k_new, shape, name="k_new"), self._check(v_new, shape, name="v_new")
        _call("kvc_paged_append", self.handle, layer, kp, vp, self._table(block_table),
              self._idx(cache_index, "cache_index"), t, _stream(self.device))

    def paged_decode_attn(self, layer, q, out, block_table, valid_lens=None, cache_index=None, sm_scale=None):
        """Decode attention over the rows the tables map (kvc_paged_decode_attn)."""
        d = self.desc
        qp = self._check(q, (d.batch, d.n_heads, d.head_dim), name="q")
        op = self._check(out, (d.batch, d.n_heads, d.head_dim), name="out")
        if sm_scale is None:
            raise ValueError("sm_scale is required")
        _call("kvc_paged_decode_attn", self.handle, layer, qp, op, self._table(block_table),
              self._idx(valid_lens, "valid_lens"), self._idx(cache_index, "cache_index"), float(sm_scale),
              _stream(self.device))


    def paged_append_decode_attn(self, layer, k_new, v_new, q, out, block_table, cache_index, sm_scale):
        """One launch: the new row at cache_index through the table, then attention over rows
        [0, cache_index + 1) (kvc_paged_append_decode_attn)."""
        d = self.desc
        shape = (d.batch, d.n_kv_heads, 1, d.head_dim)
        kp, vp = self._check(k_new, shape, name="k_new"), self._check(v_new, shape, name="v_new")
        qp = self._check(q, (d.batch, d.n_heads, d.head_dim), name="q")
        op = self._check(out, (d.batch, d.n_heads, d.head_dim), name="out")
        _call("kvc_paged_append_decode_attn", self.handle, layer, kp, vp, qp, op, self._table(block_table),
              self._idx(cache_index, "cache_index"), float(sm_scale), _stream(self.device))


def _memcpy_d2d(dst, src, nbytes, device):
    """Device-to-device byte copy on the current stream, through the HIP
    runtime that libkvc.so itself is bound to; waits for completion."""
    st = load().hipMemcpyAsync(ctypes.c_void_p(dst), ctypes.c_void_p(src), ctypes.c_size_t(nbytes),
                               ctypes.c_int(3), _stream(device))
    if st != 0:
        raise RuntimeError(f"hipMemcpyAsync failed ({st})")
    _torch().cuda.current_stream(device).synchronize()
