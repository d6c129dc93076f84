"""Thin ctypes binding over libhyb.so (the C ABI in include/hyb.h).

Argument marshalling only: torch tensors supply device memory and the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  There is no CPU fallback -- if libhyb.so is missing or a call
fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# The in-tree library; HYB_LIB names another build of the same ABI (the
# sanitizer test's host-only build).
LIB_PATH = os.environ.get("HYB_LIB") or os.path.join(PKG_DIR, "libhyb.so")

HYB_OK = 0
HYB_F16, HYB_BF16, HYB_F32 = 1, 2, 3
HYB_META_IDX2, HYB_META_MASK4, HYB_META_MASK8 = 1, 2, 3
HYB_MAGIC = 0x31425948
HYB_VERSION = 1
MAX_GEMV_M = 16

META_CODES = {"idx2": HYB_META_IDX2, "mask4": HYB_META_MASK4, "mask8": HYB_META_MASK8}
DTYPE_CODES = {"f16": HYB_F16, "bf16": HYB_BF16}

EXPORTED = ("hyb_plan", "hyb_layout_check", "hyb_pack", "hyb_unpack", "hyb_gemv", "hyb_gemv_grouped", "hyb_lowrank_project",
            "hyb_gemv_lowrank", "hyb_gemm_lowrank", "hyb_gemm_lowrank_ws", "hyb_gemm", "hyb_gemm_mfma", "hyb_gemm_ws", "hyb_gemm_workspace_size", "hyb_gemm_noalloc",
            "hyb_gemm_shape",
            "hyb_stream_read",
            "hyb_status_str", "hyb_last_error", "hyb_abi_version")
KERNEL_NAMES = {1: "decode", 2: "register", 3: "lds", 4: "split"}   # HYB_KERNEL_* of hyb_gemm_shape
MAX_GROUP = 16
MAX_RANK = 256


class HybLayout(ctypes.Structure):
    _fields_ = [
        ("magic", ctypes.c_uint32), ("version", ctypes.c_uint32),
        ("n", ctypes.c_int64), ("k", ctypes.c_int64),
        ("b1", ctypes.c_int32), ("b2", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("meta", ctypes.c_int32),
        ("tiles_n", ctypes.c_int64), ("tiles_k", ctypes.c_int64),
        ("n_dense", ctypes.c_int64), ("n_sparse", ctypes.c_int64),
        ("dense_bytes", ctypes.c_int64), ("val_bytes", ctypes.c_int64),
        ("meta_bytes", ctypes.c_int64), ("tidx_bytes", ctypes.c_int64),
    ]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class HybPacked(ctypes.Structure):
    _fields_ = [("dense", ctypes.c_void_p), ("val", ctypes.c_void_p),
                ("meta", ctypes.c_void_p), ("tidx", ctypes.c_void_p)]


class HybError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)}: {detail}")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libhyb.so (built in-tree by matmul_pack_b1_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m matmul_pack_b1_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.hyb_plan.argtypes = [I64, I64, I32, I32, I32, I32, P, ctypes.POINTER(HybLayout), P]
    L.hyb_plan.restype = I32
    L.hyb_layout_check.argtypes = [ctypes.POINTER(HybLayout)]
    L.hyb_layout_check.restype = I32
    L.hyb_pack.argtypes = [ctypes.POINTER(HybLayout), P, I64, ctypes.POINTER(HybPacked), P]
    L.hyb_pack.restype = I32
    L.hyb_unpack.argtypes = [ctypes.POINTER(HybLayout), ctypes.POINTER(HybPacked), P, I64, P]
    L.hyb_unpack.restype = I32
    for name in ("hyb_gemv", "hyb_gemm", "hyb_gemm_mfma", "hyb_gemm_noalloc"):
        f = getattr(L, name)
        f.argtypes = [ctypes.POINTER(HybLayout), ctypes.POINTER(HybPacked), P, I32, I64, P, I32, I64, P]
        f.restype = I32
    L.hyb_gemm_ws.argtypes = [ctypes.POINTER(HybLayout), ctypes.POINTER(HybPacked), P, I32, I64, P, I32, I64, P,
                              ctypes.c_size_t, P]
    L.hyb_gemm_ws.restype = I32
    L.hyb_gemm_workspace_size.argtypes = [ctypes.POINTER(HybLayout), I32, ctypes.POINTER(ctypes.c_size_t)]
    L.hyb_gemm_workspace_size.restype = I32
    L.hyb_gemv_grouped.argtypes = [I32, ctypes.POINTER(HybLayout), ctypes.POINTER(HybPacked), P, I32, I64,
                                   ctypes.POINTER(ctypes.c_void_p), I32, ctypes.POINTER(I64), P]
    L.hyb_gemv_grouped.restype = I32
    for f in (L.hyb_gemv_lowrank, L.hyb_gemm_lowrank):
        f.argtypes = [ctypes.POINTER(HybLayout), ctypes.POINTER(HybPacked), P, I32, I64, P, I64, P, I64, I32, P,
                      I32, I64, P]
        f.restype = I32
    L.hyb_gemm_lowrank_ws.argtypes = [ctypes.POINTER(HybLayout), ctypes.POINTER(HybPacked), P, I32, I64, P, I64, P,
                                      I64, I32, P, I32, I64, P, ctypes.c_size_t, P]
    L.hyb_gemm_lowrank_ws.restype = I32
    L.hyb_lowrank_project.argtypes = [P, I64, I32, I64, I32, P, I32, I64, P, I64, P]
    L.hyb_lowrank_project.restype = I32
    L.hyb_gemm_shape.argtypes = [ctypes.POINTER(HybLayout), I32, ctypes.POINTER(I32 * 4)]
    L.hyb_gemm_shape.restype = I32
    L.hyb_stream_read.argtypes = [P, I64, P, I32, P]
    L.hyb_stream_read.restype = I32
    L.hyb_status_str.argtypes = [I32]
    L.hyb_status_str.restype = ctypes.c_char_p
    L.hyb_last_error.argtypes = []
    L.hyb_last_error.restype = ctypes.c_char_p
    L.hyb_abi_version.argtypes = []
    L.hyb_abi_version.restype = I32
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().hyb_status_str(int(status)).decode()


def last_error() -> str:
    return lib().hyb_last_error().decode()


def check(status: int, where: str) -> None:
    if status != HYB_OK:
        raise HybError(status, where, last_error())


# ------------------------------------------------------------------ plan ----

def plan(n: int, k: int, b1: int, b2: int, dtype: str, meta: str, tile_map) -> tuple[HybLayout, np.ndarray]:
    """Host-only layout planning.  Returns (layout, int32 tile index)."""
    tm = np.ascontiguousarray(np.asarray(tile_map, dtype=np.uint8).reshape(-1))
    tidx = np.zeros(max(tm.size, 1), dtype=np.int32)
    L = HybLayout()
    st = lib().hyb_plan(int(n), int(k), int(b1), int(b2), DTYPE_CODES.get(dtype, -1),
                        META_CODES.get(meta, -1), tm.ctypes.data if tm.size else None,
                        ctypes.byref(L), tidx.ctypes.data)
    check(st, "hyb_plan")
    return L, tidx[: L.tiles_n * L.tiles_k]


# ------------------------------------------------------- torch plumbing -----

def _torch():
    import torch
    return torch


def _dtype_name(t) -> str:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return "bf16"
    if t.dtype == torch.float16:
        return "f16"
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return t.data_ptr() if t is not None and t.numel() > 0 else None


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_2d(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor")
    if t.numel() and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")


def _check_gpu(t, name, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _check_rows(t, name):
    _check_2d(t, name)
    _check_gpu(t, name)


def _check_x(P: "PackedWeight", x, name="x"):
    """x must be m x k of the weight's dtype (checked before any device test,
    so shape and type errors never reach the library)."""
    _check_2d(x, name)
    torch = _torch()
    want = torch.bfloat16 if P.dtype == "bf16" else torch.float16
    if x.dtype != want:
        raise TypeError(f"{name} is {x.dtype}, the weight is {P.dtype}")
    if x.shape[1] != P.shape[1]:
        raise ValueError(f"{name} has {x.shape[1]} columns, the weight has k = {P.shape[1]}")


def _check_out(out, shape, tdt, name="out"):
    """A caller-supplied output must have exactly the shape and dtype the
    library will write (it only knows the row stride)."""
    _check_2d(out, name)
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"{name} is {tuple(out.shape)}, expected {tuple(shape)}")
    if out.dtype != tdt:
        raise TypeError(f"{name} is {out.dtype}, expected {tdt}")


def _check_same_device(P: "PackedWeight", device, what="x"):
    for name in ("dense", "val", "meta", "tidx"):
        t = getattr(P, name)
        if t.numel() and t.device != device:
            raise ValueError(f"packed {name} is on {t.device}, {what} on {device}")


@dataclass
class PackedWeight:
    """One packed matrix: its layout plus four device buffers."""
    layout: HybLayout
    dense: object
    val: object
    meta: object
    tidx: object
    dtype: str
    meta_kind: str

    @property
    def shape(self):
        return (self.layout.n, self.layout.k)

    @property
    def device(self):
        return self.tidx.device

    def packed_struct(self) -> HybPacked:
        return HybPacked(_ptr(self.dense), _ptr(self.val), _ptr(self.meta), _ptr(self.tidx))

    def weight_bytes(self) -> int:
        L = self.layout
        return L.dense_bytes + L.val_bytes + L.meta_bytes


def allocate(layout: HybLayout, tidx_host: np.ndarray, device, dtype: str, meta: str) -> PackedWeight:
    torch = _torch()
    def buf(nbytes):
        return torch.empty(int(nbytes), dtype=torch.uint8, device=device)
    tidx = torch.from_numpy(np.ascontiguousarray(tidx_host, dtype=np.int32)).to(device)
    return PackedWeight(layout, buf(layout.dense_bytes), buf(layout.val_bytes), buf(layout.meta_bytes),
                        tidx, dtype, meta)


# ------------------------------------------------------------ save / load --
#
# A saved packed weight is the layout header -- the hyb_layout struct as laid
# out in memory (104 bytes, little-endian, fixed-width fields) -- followed by
# the dense, value, metadata and tile-index streams, each exactly the size
# the header gives.  Loading checks the header with hyb_layout_check before
# anything is allocated.

DTYPE_NAMES = {v: k for k, v in DTYPE_CODES.items()}
META_NAMES = {v: k for k, v in META_CODES.items()}


def save(P: PackedWeight, path) -> None:
    """Write a packed weight to `path` (header, then the four streams)."""
    with open(path, "wb") as f:
        f.write(bytes(P.layout))
        for t in (P.dense, P.val, P.meta, P.tidx):
            f.write(t.detach().cpu().contiguous().numpy().tobytes())


def load(path, device) -> PackedWeight:
    """Read a packed weight written by `save` onto `device`.  A header that
    fails hyb_layout_check (bad magic, version, counts or sizes) raises
    HybError with that status; a file of the wrong length raises ValueError."""
    torch = _torch()
    with open(path, "rb") as f:
        head = f.read(ctypes.sizeof(HybLayout))
        if len(head) != ctypes.sizeof(HybLayout):
            raise ValueError(f"{path}: shorter than a layout header")
        L = HybLayout.from_buffer_copy(head)
        check(lib().hyb_layout_check(ctypes.byref(L)), "hyb_layout_check")
        parts = []
        for nbytes in (L.dense_bytes, L.val_bytes, L.meta_bytes, L.tidx_bytes):
            b = f.read(int(nbytes))
            if len(b) != nbytes:
                raise ValueError(f"{path}: truncated stream ({len(b)} of {nbytes} bytes)")
            parts.append(b)
        if f.read(1):
            raise ValueError(f"{path}: trailing bytes after the streams")
    def dev_u8(b):
        return torch.frombuffer(bytearray(b), dtype=torch.uint8).to(device) if b else \
            torch.empty(0, dtype=torch.uint8, device=device)
    tidx = torch.frombuffer(bytearray(parts[3]), dtype=torch.int32).to(device) if parts[3] else \
        torch.empty(0, dtype=torch.int32, device=device)
    return PackedWeight(L, dev_u8(parts[0]), dev_u8(parts[1]), dev_u8(parts[2]), tidx,
                        DTYPE_NAMES[L.dtype], META_NAMES[L.meta])


def pack(w, tile_map, b1: int, b2: int, meta: str = "idx2", out: PackedWeight | None = None) -> PackedWeight:
    """Pack a device matrix w (n x k, bf16 or fp16) with the given tile map
    (uint8 [n/b1, k/b2], 1 = sparse: 2:4, or 4:8 with meta "mask8").  `out`
    reuses existing buffers."""
    _check_2d(w, "w")
    dtype = _dtype_name(w)
    n, k = w.shape
    if out is None:
        _check_gpu(w, "w")
        L, tidx = plan(n, k, b1, b2, dtype, meta, tile_map)
        out = allocate(L, tidx, w.device, dtype, meta)
    else:
        # out's streams were planned for one matrix and map; w and the map
        # must match them (the tile index on the device is not re-read: the
        # map is checked through its tile counts)
        L = out.layout
        if (n, k) != (L.n, L.k) or (b1, b2) != (L.b1, L.b2):
            raise ValueError(f"w is {n}x{k} with {b1}x{b2} tiles, out holds {L.n}x{L.k} with {L.b1}x{L.b2}")
        if dtype != out.dtype or meta != out.meta_kind:
            raise TypeError(f"w/meta are {dtype}/{meta}, out holds {out.dtype}/{out.meta_kind}")
        L2, _ = plan(n, k, b1, b2, dtype, meta, tile_map)
        if (L2.n_dense, L2.n_sparse) != (L.n_dense, L.n_sparse):
            raise ValueError("the tile map does not match out's layout")
        _check_gpu(w, "w")
        _check_same_device(out, w.device, "w")
    P = out.packed_struct()
    st = lib().hyb_pack(ctypes.byref(out.layout), _ptr(w), int(w.stride(0)) if w.numel() else int(k),
                        ctypes.byref(P), _stream(w.device))
    check(st, "hyb_pack")
    return out


def unpack(P: PackedWeight, out=None):
    """W' (n x k, same dtype) rebuilt on the device from the packed streams."""
    torch = _torch()
    n, k = P.shape
    tdt = torch.bfloat16 if P.dtype == "bf16" else torch.float16
    if out is None:
        out = torch.empty((n, k), dtype=tdt, device=P.device)
    _check_out(out, (n, k), tdt)
    _check_gpu(out, "out")
    _check_same_device(P, out.device, "out")
    st = lib().hyb_unpack(ctypes.byref(P.layout), ctypes.byref(P.packed_struct()), _ptr(out),
                          int(out.stride(0)) if out.numel() else int(k), _stream(P.device))
    check(st, "hyb_unpack")
    return out


def _out_code(P: PackedWeight, out_dtype) -> int:
    torch = _torch()
    if out_dtype in (None, torch.float32):
        return HYB_F32
    if out_dtype == torch.bfloat16 and P.dtype == "bf16":
        return HYB_BF16
    if out_dtype == torch.float16 and P.dtype == "f16":
        return HYB_F16
    raise TypeError(f"output dtype {out_dtype} must be float32 or the weight dtype")


def _product(fn_name: str, P: PackedWeight, x, out_dtype=None, out=None, workspace=None):
    torch = _torch()
    _check_x(P, x)
    m = x.shape[0]
    n, k = P.shape
    if out is not None and out_dtype is None:
        out_dtype = out.dtype
    code = _out_code(P, out_dtype)
    tdt = {HYB_F32: torch.float32, HYB_BF16: torch.bfloat16, HYB_F16: torch.float16}[code]
    if out is None:
        out = torch.empty((m, n), dtype=tdt, device=x.device)
    _check_out(out, (m, n), tdt)
    _check_gpu(x, "x")
    _check_gpu(out, "out", x.device)
    _check_same_device(P, x.device)
    fn = getattr(lib(), fn_name)
    args = [ctypes.byref(P.layout), ctypes.byref(P.packed_struct()), _ptr(x), int(m),
            int(x.stride(0)) if x.numel() else int(k), _ptr(out), code,
            int(out.stride(0)) if out.numel() else int(n)]
    if fn_name == "hyb_gemm_ws":
        # split-K workspace from torch's allocator on the current stream (so
        # that graph capture takes it from the graph's pool); kept alive by
        # the stream order of the allocator until the launches complete
        if workspace is None:
            need = workspace_bytes(P, m)
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device) if need else None
        if workspace is not None:
            _check_gpu(workspace, "workspace", x.device)
            if not workspace.is_contiguous():
                raise ValueError("workspace must be contiguous")
        args += [_ptr(workspace) if workspace is not None else None,
                 workspace.numel() * workspace.element_size() if workspace is not None else 0]
    st = fn(*args, _stream(x.device))
    check(st, fn_name)
    return out


def gemv(P: PackedWeight, x, out_dtype=None, out=None):
    """Decode product Y = X W'^T for 1..16 tokens (rows of x)."""
    return _product("hyb_gemv", P, x, out_dtype, out)


def gemv_grouped(Ps, x, out_dtype=None, outs=None):
    """Decode products of the same x with several packed matrices (same k,
    b2, dtype and metadata kind) in one launch; returns one output per
    matrix."""
    torch = _torch()
    Ps = list(Ps)
    _check_2d(x, "x")
    for i, P in enumerate(Ps):
        _check_x(P, x, f"x (matrix {i})")
    m = x.shape[0]
    count = len(Ps)
    if outs is not None and out_dtype is None and len(outs):
        out_dtype = outs[0].dtype
    codes = {_out_code(P, out_dtype) for P in Ps} or {HYB_F32}
    if len(codes) != 1:
        raise TypeError("all matrices must share one output type")
    code = codes.pop()
    tdt = {HYB_F32: torch.float32, HYB_BF16: torch.bfloat16, HYB_F16: torch.float16}[code]
    if outs is None:
        outs = [torch.empty((m, P.shape[0]), dtype=tdt, device=x.device) for P in Ps]
    if len(outs) != count:
        raise ValueError("one output per matrix")
    for i, (o, P) in enumerate(zip(outs, Ps)):
        _check_out(o, (m, P.shape[0]), tdt, f"outs[{i}]")
    _check_gpu(x, "x")
    for i, (o, P) in enumerate(zip(outs, Ps)):
        _check_gpu(o, f"outs[{i}]", x.device)
        _check_same_device(P, x.device)
    layouts = (HybLayout * max(count, 1))(*[P.layout for P in Ps])
    packed = (HybPacked * max(count, 1))(*[P.packed_struct() for P in Ps])
    ys = (ctypes.c_void_p * max(count, 1))(*[_ptr(o) for o in outs])
    ldys = (ctypes.c_int64 * max(count, 1))(*[int(o.stride(0)) if o.numel() else int(P.shape[0])
                                               for o, P in zip(outs, Ps)])
    k = Ps[0].shape[1] if Ps else x.shape[1]
    st = lib().hyb_gemv_grouped(count, layouts, packed, _ptr(x), int(m),
                                int(x.stride(0)) if x.numel() else int(k), ys, code, ldys, _stream(x.device))
    check(st, "hyb_gemv_grouped")
    return outs


def lowrank_project(v, x, out=None):
    """T = X V (fp32, m x rank) for a low-rank factor V (k x rank) held
    transposed: `v` is rank x k with unit column stride, of x's dtype."""
    torch = _torch()
    _check_2d(v, "v")
    _check_2d(x, "x")
    if v.dtype != x.dtype or v.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("v and x must share one dtype, bfloat16 or float16")
    rank, k = v.shape
    m = x.shape[0]
    if x.shape[1] != k:
        raise ValueError(f"x must have {k} columns")
    if out is None:
        out = torch.empty((m, rank), dtype=torch.float32, device=x.device)
    _check_out(out, (m, rank), torch.float32)
    _check_gpu(x, "x")
    _check_gpu(v, "v", x.device)
    _check_gpu(out, "out", x.device)
    code = HYB_BF16 if v.dtype == torch.bfloat16 else HYB_F16
    st = lib().hyb_lowrank_project(_ptr(v), int(v.stride(0)) if v.numel() else int(k), int(rank), int(k), code,
                                   _ptr(x), int(m), int(x.stride(0)) if x.numel() else int(k), _ptr(out),
                                   int(out.stride(0)) if out.numel() else int(rank), _stream(x.device))
    check(st, "hyb_lowrank_project")
    return out


def _lowrank(fn_name: str, P: PackedWeight, x, t, u, out_dtype, out, workspace=None):
    torch = _torch()
    _check_x(P, x)
    _check_2d(t, "t")
    _check_2d(u, "u")
    m = x.shape[0]
    n, k = P.shape
    rank = t.shape[1]
    if t.shape[0] != m or tuple(u.shape) != (n, rank):
        raise ValueError(f"t must be {m} x rank and u {n} x rank")
    if t.dtype != torch.float32:
        raise TypeError("t must be float32")
    if u.dtype != (torch.bfloat16 if P.dtype == "bf16" else torch.float16):
        raise TypeError(f"u is {u.dtype}, the weight is {P.dtype}")
    if out is not None and out_dtype is None:
        out_dtype = out.dtype
    code = _out_code(P, out_dtype)
    tdt = {HYB_F32: torch.float32, HYB_BF16: torch.bfloat16, HYB_F16: torch.float16}[code]
    if out is None:
        out = torch.empty((m, n), dtype=tdt, device=x.device)
    _check_out(out, (m, n), tdt)
    _check_gpu(x, "x")
    for name, tt in (("t", t), ("u", u), ("out", out)):
        _check_gpu(tt, name, x.device)
    _check_same_device(P, x.device)
    args = [ctypes.byref(P.layout), ctypes.byref(P.packed_struct()), _ptr(x), int(m),
            int(x.stride(0)) if x.numel() else int(k), _ptr(t), int(t.stride(0)) if t.numel() else int(rank),
            _ptr(u), int(u.stride(0)) if u.numel() else int(rank), int(rank), _ptr(out), code,
            int(out.stride(0)) if out.numel() else int(n)]
    if fn_name == "hyb_gemm_lowrank_ws":
        # split-K workspace from torch's allocator, as for gemm()
        if workspace is None:
            need = workspace_bytes(P, m)
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device) if need else None
        if workspace is not None:
            _check_gpu(workspace, "workspace", x.device)
            if not workspace.is_contiguous():
                raise ValueError("workspace must be contiguous")
        args += [_ptr(workspace) if workspace is not None else None,
                 workspace.numel() * workspace.element_size() if workspace is not None else 0]
    st = getattr(lib(), fn_name)(*args, _stream(x.device))
    check(st, fn_name)
    return out


def gemv_lowrank(P: PackedWeight, x, t, u, out_dtype=None, out=None):
    """Decode product of a sparse + low-rank weight (1..16 tokens): Y = X W'^T
    + T U^T, with t = X V (fp32, m x rank) given and u (n x rank, weight
    dtype)."""
    return _lowrank("hyb_gemv_lowrank", P, x, t, u, out_dtype, out)


def gemm_lowrank(P: PackedWeight, x, t, u, out_dtype=None, out=None, workspace=None):
    """Sparse + low-rank product for any number of tokens, through
    hyb_gemm_lowrank_ws: a route that splits K gets its workspace from torch's
    allocator (so graph capture works) unless `workspace` is given."""
    return _lowrank("hyb_gemm_lowrank_ws", P, x, t, u, out_dtype, out, workspace)


def gemm_lowrank_held(P: PackedWeight, x, t, u, out_dtype=None, out=None):
    """The same through hyb_gemm_lowrank (workspace held by the library per
    device and stream)."""
    return _lowrank("hyb_gemm_lowrank", P, x, t, u, out_dtype, out)


def sparse_lowrank_gemv(P: PackedWeight, v, u, x, out_dtype=None, out=None, t=None):
    """Y = X (W' + U V^T)^T in two launches: T = X V (hyb_lowrank_project,
    v = V^T, rank x k), then the sparse product with T U^T added in the
    decode kernel.  `t` optionally gives the m x rank fp32 buffer for T."""
    t = lowrank_project(v, x, out=t)
    return gemv_lowrank(P, x, t, u, out_dtype, out)


def sparse_lowrank_gemm(P: PackedWeight, v, u, x, out_dtype=None, out=None, t=None):
    """As sparse_lowrank_gemv for any number of tokens (hyb_gemm_lowrank)."""
    t = lowrank_project(v, x, out=t)
    return gemm_lowrank(P, x, t, u, out_dtype, out)


def gemm(P: PackedWeight, x, out_dtype=None, out=None, workspace=None):
    """Y = X W'^T for any number of tokens (decode kernel up to 8, matrix cores
    above), through hyb_gemm_ws: a product whose route splits K gets its
    workspace from torch's allocator unless `workspace` (a contiguous device
    tensor of at least workspace_bytes(P, m) bytes) is given."""
    return _product("hyb_gemm_ws", P, x, out_dtype, out, workspace)


def gemm_noalloc(P: PackedWeight, x, out_dtype=None, out=None):
    """hyb_gemm with no device allocation: a split product uses the library's
    static device scratch (calls that overlap on one GPU race)."""
    return _product("hyb_gemm_noalloc", P, x, out_dtype, out)


def workspace_bytes(P: PackedWeight, m: int) -> int:
    """Workspace bytes of hyb_gemm_ws for m tokens on the current device."""
    nbytes = ctypes.c_size_t(0)
    check(lib().hyb_gemm_workspace_size(ctypes.byref(P.layout), int(m), ctypes.byref(nbytes)),
          "hyb_gemm_workspace_size")
    return int(nbytes.value)


def gemm_mfma(P: PackedWeight, x, out_dtype=None, out=None):
    """Y = X W'^T on the matrix-core kernel regardless of the token count."""
    return _product("hyb_gemm_mfma", P, x, out_dtype, out)


def gemm_shape(layout: HybLayout, m: int) -> dict:
    """The kernel and workgroup shape hyb_gemm would launch for m tokens on
    this layout's matrix on the current device (hyb_gemm_shape; host only)."""
    out = (ctypes.c_int32 * 4)()
    check(lib().hyb_gemm_shape(ctypes.byref(layout), int(m), ctypes.byref(out)), "hyb_gemm_shape")
    return {"kernel": KERNEL_NAMES[out[0]], "token_blocks": out[1], "waves": out[2], "row_groups": out[3]}


def stream_read(buf, nbytes: int, sink, grid: int) -> None:
    """Measurement aid: read `nbytes` of the device tensor `buf` with the
    decode kernel's load pattern (hyb_stream_read); `sink` holds grid*256
    uint32/int32 entries."""
    if sink.numel() < grid * 256:
        raise ValueError("sink too small")
    st = lib().hyb_stream_read(_ptr(buf), int(nbytes), _ptr(sink), int(grid), _stream(buf.device))
    check(st, "hyb_stream_read")


def bits_to_tensor(bits: np.ndarray, dtype: str, device):
    """Upload uint16 bit patterns as a bf16 / fp16 device tensor."""
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    return t.to(device).view(tdt)


def tensor_to_bits(t) -> np.ndarray:
    """Download a 16-bit device tensor as uint16 bit patterns."""
    torch = _torch()
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
