"""Block-sparse attention forward for MI355X (gfx950): Python binding.

Thin ctypes binding of ``libbsa.so`` (C ABI declared in include/bsa.h).  It
only marshals arguments: every step of the request path (mask state, plan
selection, launch preparation, attention, split-K merge) runs in the
library's host code and gfx950 kernels.  torch is used for device memory and
the current stream only.  There is no fallback: if the library is not built
the import of any entry point raises.
"""

import ctypes
import os

__all__ = ["BsaError", "Plan", "plan", "run", "run_timed", "catalog", "select", "eligible", "base_plan",
           "table_load", "table_version", "catalog_hash", "library_path"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libbsa.so")
_lib = None

BSA_DTYPE_BF16 = 1
BSA_LAYOUT_HND = 0
BSA_LAYOUT_NHD = 1
SPLIT_STREAM = -2  # force_split value of the stream organization (BSA_SPLIT_STREAM)
_LAYOUTS = {"HND": BSA_LAYOUT_HND, "NHD": BSA_LAYOUT_NHD}


class BsaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{status}: {msg}")
        self.status = status


class Request(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("N", ctypes.c_int32), ("d", ctypes.c_int32),
                ("block_q", ctypes.c_int32), ("block_kv", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("force_plan", ctypes.c_int32), ("force_split", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("workspace_limit", ctypes.c_int64),
                ("mask", ctypes.c_void_p)]


class PlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "plan_id", "regime", "tile_q", "tile_kv", "coarsen_q", "coarsen_kv", "refine_q",
        "refine_kv", "split_items", "max_row_nnz")] + \
        [(n, ctypes.c_int64) for n in (
            "nnz_blocks", "n_tile_rows", "n_items", "n_tasks", "grid", "workspace_bytes",
            "long_run_blocks")] + \
        [(n, ctypes.c_double) for n in ("density", "run_coverage", "row_skew", "host_select_us")] + \
        [("tasks_predicted", ctypes.c_int32), ("split_threshold", ctypes.c_int32)]


class CatalogEntry(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("id", "tile_q", "tile_kv", "d", "split", "xcd_remap",
                                              "order")] + \
        [("name", ctypes.c_char * 48)]


def library_path():
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"libbsa.so is not built at {_LIB_PATH}; run "
                          "`python -m dynamic_block_sparse_bsa_amd.build` (or __graft_entry__.build())")
    L = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    L.bsa_plan_create.argtypes = [ctypes.POINTER(Request), P, ctypes.POINTER(P)]
    L.bsa_run.argtypes = [P, P, P, P, P, P]
    L.bsa_run_timed.argtypes = [P, P, P, P, P, P, ctypes.POINTER(ctypes.c_float),
                                ctypes.POINTER(ctypes.c_float)]
    L.bsa_plan_destroy.argtypes = [P]
    L.bsa_plan_get_info.argtypes = [P, ctypes.POINTER(PlanInfo)]
    L.bsa_plan_export_tiles.argtypes = [P, P, P, P, P, i64, ctypes.POINTER(i64)]
    L.bsa_plan_export_csr.argtypes = [P, P, P, i64]
    L.bsa_plan_export_tasks.argtypes = [P, P, P, P, P, P, i64, ctypes.POINTER(i64)]
    L.bsa_catalog_size.restype = i32
    L.bsa_catalog_get.argtypes = [i32, ctypes.POINTER(CatalogEntry)]
    L.bsa_plan_eligible.argtypes = [i32, ctypes.POINTER(Request), ctypes.POINTER(i32)]
    L.bsa_select.argtypes = [ctypes.POINTER(Request), ctypes.c_double, ctypes.c_double,
                             ctypes.c_double, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.bsa_table_load.argtypes = [ctypes.c_char_p]
    L.bsa_base_plan.argtypes = [ctypes.POINTER(Request), ctypes.POINTER(i32)]
    L.bsa_plan_cache_create.argtypes = [i32, i64, ctypes.POINTER(P)]
    L.bsa_plan_cache_get.argtypes = [P, ctypes.POINTER(Request), P, ctypes.POINTER(P), ctypes.POINTER(i32)]
    L.bsa_plan_cache_destroy.argtypes = [P]
    L.bsa_plan_cache_run.argtypes = [P, ctypes.POINTER(Request), P, P, P, P, P, ctypes.POINTER(i32)]
    L.bsa_attention_noalloc.argtypes = [ctypes.POINTER(Request), P, P, P, P, P]
    for f in ("bsa_table_version", "bsa_catalog_hash", "bsa_status_string", "bsa_last_error"):
        getattr(L, f).restype = ctypes.c_char_p
    L.bsa_status_string.argtypes = [i32]
    for f in ("bsa_plan_create", "bsa_run", "bsa_run_timed", "bsa_plan_destroy",
              "bsa_plan_get_info", "bsa_plan_export_tiles", "bsa_plan_export_csr",
              "bsa_plan_export_tasks",
              "bsa_catalog_get", "bsa_plan_eligible", "bsa_select", "bsa_table_load",
              "bsa_base_plan", "bsa_plan_cache_create", "bsa_plan_cache_get", "bsa_plan_cache_destroy",
              "bsa_plan_cache_run", "bsa_attention_noalloc"):
        getattr(L, f).restype = i32
    _lib = L
    return L


def _check(st):
    if st != 0:
        L = _load()
        raise BsaError(L.bsa_status_string(st).decode(), L.bsa_last_error().decode())


def _layout(layout):
    if layout not in _LAYOUTS:
        raise BsaError("BSA_ERR_INVALID_ARG", f"layout must be one of {sorted(_LAYOUTS)}, got {layout!r}")
    return _LAYOUTS[layout]


def _request(H, N, d, block, mask_ptr=None, force_plan=-1, force_split=-1, workspace_limit=0, batch=1,
             layout="HND"):
    return Request(H=H, N=N, d=d, block_q=block[0], block_kv=block[1], dtype=BSA_DTYPE_BF16,
                   layout=_layout(layout), force_plan=force_plan, force_split=force_split,
                   batch=batch, workspace_limit=workspace_limit, mask=mask_ptr)


def tensor_shapes(H, N, d, batch=1, layout="HND"):
    """Accepted Q/K/V/O shapes: [batch][H][N][d] (HND) or [batch][N][H][d]
    (NHD); with batch 1 the leading dimension may be left out."""
    inner = (H, N, d) if _layout(layout) == BSA_LAYOUT_HND else (N, H, d)
    return [(batch,) + inner] + ([inner] if batch == 1 else [])


def _stream(stream):
    import torch
    if stream is None:
        # the raw handle of the current stream without building a Stream
        # object (a few microseconds per call on the request path)
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:
            return ctypes.c_void_p(raw(torch.cuda.current_device()))
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Plan:
    """A prepared plan (owns device metadata until destroyed or collected;
    a plan returned by a PlanCache belongs to the cache instead)."""

    def __init__(self, handle, H, N, d, block, owned=True, batch=1, layout="HND"):
        self._h = handle
        self._owned = owned
        self.H, self.N, self.d, self.block = H, N, d, block
        self.batch, self.layout = batch, layout

    @property
    def handle(self):
        if self._h is None:
            raise BsaError("BSA_ERR_INVALID_ARG", "plan was destroyed")
        return self._h

    @property
    def info(self):
        out = PlanInfo()
        _check(_load().bsa_plan_get_info(self.handle, ctypes.byref(out)))
        return {k: getattr(out, k) for k, _ in PlanInfo._fields_}

    def export_tiles(self):
        """numpy arrays (head, q_tile, kv_tile, bits) of the tiles in task order."""
        import numpy as np
        L = _load()
        cnt = ctypes.c_int64(0)
        st = L.bsa_plan_export_tiles(self.handle, None, None, None, None, 0, ctypes.byref(cnt))
        n = cnt.value
        if st != 0 and n == 0:
            _check(st)
        arrs = [np.empty(n, np.int32), np.empty(n, np.int32), np.empty(n, np.int32),
                np.empty(n, np.uint32)]
        ptrs = [a.ctypes.data_as(ctypes.c_void_p) for a in arrs]
        _check(L.bsa_plan_export_tiles(self.handle, *ptrs, n, ctypes.byref(cnt)))
        return tuple(arrs)

    def export_tasks(self):
        """numpy arrays (head, q_tile, begin, end, slot) of the tasks in dispatch order."""
        import numpy as np
        L = _load()
        cnt = ctypes.c_int64(0)
        st = L.bsa_plan_export_tasks(self.handle, None, None, None, None, None, 0, ctypes.byref(cnt))
        n = cnt.value
        if st != 0 and n == 0:
            _check(st)
        arrs = [np.empty(n, np.int32) for _ in range(5)]
        ptrs = [a.ctypes.data_as(ctypes.c_void_p) for a in arrs]
        _check(L.bsa_plan_export_tasks(self.handle, *ptrs, n, ctypes.byref(cnt)))
        return tuple(arrs)

    def export_csr(self):
        import numpy as np
        info = self.info
        nrows = self.batch * self.H * (-(-self.N // self.block[0]))
        rp = np.empty(nrows + 1, np.int32)
        cols = np.empty(max(1, info["nnz_blocks"]), np.int32)
        _check(_load().bsa_plan_export_csr(self.handle, rp.ctypes.data_as(ctypes.c_void_p),
                                           cols.ctypes.data_as(ctypes.c_void_p), cols.size))
        return rp, cols[:info["nnz_blocks"]]

    def destroy(self):
        if self._h is not None:
            h, self._h = self._h, None
            if self._owned:
                _check(_load().bsa_plan_destroy(h))

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def _mask_request(mask, block, H, N, d, force_plan, force_split, workspace_limit, batch, layout):
    import torch
    nq, nk = -(-N // block[0]), -(-N // block[1])
    if not (isinstance(mask, torch.Tensor) and mask.is_cuda and mask.dtype == torch.uint8):
        raise BsaError("BSA_ERR_INVALID_ARG", "mask must be a CUDA uint8 tensor")
    ok = [(batch * H, nq, nk), (batch, H, nq, nk)]
    if tuple(mask.shape) not in ok or not mask.is_contiguous():
        raise BsaError("BSA_ERR_INVALID_ARG", f"mask must be contiguous {ok[0]} or {ok[1]}, got {tuple(mask.shape)}")
    return _request(H, N, d, block, mask.data_ptr(), force_plan, force_split, workspace_limit, batch, layout)


def plan(mask, block, H, N, d, force_plan=-1, force_split=-1, workspace_limit=0, stream=None, batch=1,
         layout="HND"):
    """Create a plan. mask: CUDA uint8 tensor [batch*H, ceil(N/B_Q), ceil(N/B_KV)]
    (or with batch and head dimensions apart); layout "HND" or "NHD" for the
    tensors the plan will run on."""
    req = _mask_request(mask, block, H, N, d, force_plan, force_split, workspace_limit, batch, layout)
    h = ctypes.c_void_p()
    _check(_load().bsa_plan_create(ctypes.byref(req), _stream(stream), ctypes.byref(h)))
    return Plan(h, H, N, d, block, batch=batch, layout=layout)


class PlanCache:
    """bsa_plan_cache: prepared plans reused for exact repeats of a request
    (same geometry and options, byte-identical mask)."""

    def __init__(self, capacity=4, max_mask_bytes=0):
        h = ctypes.c_void_p()
        _check(_load().bsa_plan_cache_create(int(capacity), int(max_mask_bytes), ctypes.byref(h)))
        self._h = h

    def get(self, mask, block, H, N, d, force_plan=-1, force_split=-1, workspace_limit=0, stream=None, batch=1,
            layout="HND"):
        """(Plan, hit): the cached plan of an identical earlier request, or a new one."""
        if self._h is None:
            raise BsaError("BSA_ERR_INVALID_ARG", "cache was destroyed")
        req = _mask_request(mask, block, H, N, d, force_plan, force_split, workspace_limit, batch, layout)
        h = ctypes.c_void_p()
        hit = ctypes.c_int32(0)
        _check(_load().bsa_plan_cache_get(self._h, ctypes.byref(req), _stream(stream), ctypes.byref(h),
                                          ctypes.byref(hit)))
        return Plan(h, H, N, d, block, owned=False, batch=batch, layout=layout), bool(hit.value)

    def run(self, mask, block, H, N, d, q, k, v, out=None, force_plan=-1, force_split=-1, workspace_limit=0,
            stream=None, batch=1, layout="HND"):
        """(out, hit): O = BSA(Q, K, V) for the request through the cache, the
        repeat check overlapped with the speculative run of the most recently
        used matching-geometry plan (bsa_plan_cache_run)."""
        import types
        if self._h is None:
            raise BsaError("BSA_ERR_INVALID_ARG", "cache was destroyed")
        req = _mask_request(mask, block, H, N, d, force_plan, force_split, workspace_limit, batch, layout)
        out = _tensors(types.SimpleNamespace(H=H, N=N, d=d, batch=batch, layout=layout), q, k, v, out)
        hit = ctypes.c_int32(0)
        _check(_load().bsa_plan_cache_run(self._h, ctypes.byref(req), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                          out.data_ptr(), _stream(stream), ctypes.byref(hit)))
        return out, bool(hit.value)

    def destroy(self):
        if self._h is not None:
            h, self._h = self._h, None
            _check(_load().bsa_plan_cache_destroy(h))

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def _tensors(p, q, k, v, out):
    import torch
    shapes = tensor_shapes(p.H, p.N, p.d, p.batch, p.layout)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == torch.bfloat16
                and tuple(t.shape) in shapes and t.is_contiguous()):
            raise BsaError("BSA_ERR_INVALID_ARG", f"{name} must be a contiguous CUDA bf16 tensor {shapes[-1]}")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    elif not (out.is_cuda and out.dtype == torch.bfloat16 and tuple(out.shape) in shapes
              and out.is_contiguous()):
        raise BsaError("BSA_ERR_INVALID_ARG", f"out must be a contiguous CUDA bf16 tensor {shapes[-1]}")
    return out


def run(p, q, k, v, out=None, stream=None):
    out = _tensors(p, q, k, v, out)
    _check(_load().bsa_run(p.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                           _stream(stream)))
    return out


def attention_noalloc(mask, block, H, N, d, q, k, v, out, force_plan=-1, force_split=-1, workspace_limit=0,
                      stream=None, batch=1, layout="HND"):
    """bsa_attention_noalloc: O = BSA(Q, K, V) for the request in one call,
    every device buffer carved from the library's fixed per-device scratch
    (no device allocation; `out` must be given).  Returns out."""
    import types
    req = _mask_request(mask, block, H, N, d, force_plan, force_split, workspace_limit, batch, layout)
    if out is None:
        raise BsaError("BSA_ERR_INVALID_ARG", "out must be given (this entry point allocates nothing)")
    out = _tensors(types.SimpleNamespace(H=H, N=N, d=d, batch=batch, layout=layout), q, k, v, out)
    _check(_load().bsa_attention_noalloc(ctypes.byref(req), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                         out.data_ptr(), _stream(stream)))
    return out


def run_timed(p, q, k, v, out=None, stream=None):
    """run() plus the attention and merge kernel durations (ms, HIP events)."""
    out = _tensors(p, q, k, v, out)
    a, m = ctypes.c_float(0), ctypes.c_float(0)
    _check(_load().bsa_run_timed(p.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                 out.data_ptr(), _stream(stream), ctypes.byref(a), ctypes.byref(m)))
    return out, a.value, m.value


def catalog():
    L = _load()
    res = []
    for i in range(L.bsa_catalog_size()):
        e = CatalogEntry()
        _check(L.bsa_catalog_get(i, ctypes.byref(e)))
        res.append(dict(id=e.id, tile_q=e.tile_q, tile_kv=e.tile_kv, d=e.d, split=e.split,
                        xcd_remap=e.xcd_remap, order=e.order, name=e.name.decode()))
    return res


def eligible(plan_id, H, N, d, block, workspace_limit=0, batch=1, layout="HND"):
    r = _request(H, N, d, block, None, workspace_limit=workspace_limit, batch=batch, layout=layout)
    out = ctypes.c_int32(0)
    _check(_load().bsa_plan_eligible(plan_id, ctypes.byref(r), ctypes.byref(out)))
    return bool(out.value)


def select(H, N, d, block, density, run_coverage, row_skew=1.0, batch=1, layout="HND"):
    """Host-only regime lookup + ranked fallback: (plan_id, regime)."""
    r = _request(H, N, d, block, None, batch=batch, layout=layout)
    pid, reg = ctypes.c_int32(-1), ctypes.c_int32(-1)
    _check(_load().bsa_select(ctypes.byref(r), density, run_coverage, row_skew, ctypes.byref(pid),
                              ctypes.byref(reg)))
    return pid.value, reg.value


def base_plan(H, N, d, block, batch=1, layout="HND"):
    """Catalog id of the request key's base plan (host only)."""
    r = _request(H, N, d, block, None, batch=batch, layout=layout)
    pid = ctypes.c_int32(-1)
    _check(_load().bsa_base_plan(ctypes.byref(r), ctypes.byref(pid)))
    return pid.value


def table_load(path):
    _check(_load().bsa_table_load(None if path is None else os.fsencode(path)))


def table_version():
    return _load().bsa_table_version().decode()


def catalog_hash():
    return _load().bsa_catalog_hash().decode()
