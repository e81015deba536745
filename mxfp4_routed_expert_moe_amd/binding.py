"""Python binding of libmoe.so: argument marshalling only.

Every step of the layer runs in the library's HIP kernels; this module checks
tensor dtypes/devices, allocates outputs and workspaces as torch tensors on
the current device, passes raw pointers and the current HIP stream, and turns
a non-zero status into an exception.  The names follow the C ABI in
include/moe.h.  If the library is missing the import fails loudly: there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_ABI_VERSION = 1
MOE_LAYOUT_CANONICAL_MXFP4 = 0x4D584330
MOE_LAYOUT_GFX950_TILED_V1 = 0x4D584731
MOE_FFN_SPLIT_FP8 = 1  # moe_experts.flags: prefill expert FFN on the scaled FP4 matrix cores
MOE_SHARED_MXFP8 = 2   # moe_experts.flags: the shared expert is MXFP8
MOE_ROUTED_AFFINE2 = 4  # moe_experts.flags: the routed experts are 2-bit affine (JANG recipe)
MOE_MAX_TOKENS = 262144  # largest T any call accepts
MOE_MAX_DIM = 65536  # largest H or I any call accepts
MOE_DISPATCH_NOALLOC_SCRATCH_BYTES = 8 << 20  # static scratch of moe_dispatch_noalloc, per GPU
STATUS = {0: "MOE_OK", 1: "MOE_EINVAL", 2: "MOE_EALIGN", 3: "MOE_ELAYOUT", 4: "MOE_ESHAPE",
          5: "MOE_EWORKSPACE", 6: "MOE_EHIP"}

EXPORTED = ("moe_status_str", "moe_abi_version", "moe_expert_bytes", "moe_experts_init", "moe_pack_mxfp4",
            "moe_unpack_mxfp4", "moe_expert_bytes_mxfp8", "moe_pack_mxfp8", "moe_unpack_mxfp8",
            "moe_expert_bytes_affine2", "moe_pack_affine2", "moe_unpack_affine2", "moe_route_workspace_size", "moe_route",
            "moe_dispatch_workspace_size",
            "moe_dispatch", "moe_dispatch_noalloc", "moe_ffn_workspace_size", "moe_expert_ffn", "moe_expert_ffn_phase",
            "moe_combine")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


class moe_experts(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint32), ("layout", ctypes.c_uint32), ("n_experts", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("expert_bytes", ctypes.c_uint64), ("base", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmoe.so (built by mxfp4_routed_expert_moe_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mxfp4_routed_expert_moe_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    c_i32, c_u64, c_sz, vp = ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_void_p
    sig = {
        "moe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_abi_version": (ctypes.c_uint32, []),
        "moe_expert_bytes": (c_u64, [c_i32, c_i32]),
        "moe_experts_init": (ctypes.c_int, [ctypes.POINTER(moe_experts), vp, c_i32, c_i32, c_i32]),
        "moe_pack_mxfp4": (ctypes.c_int, [vp, c_u64, c_i32, c_i32, c_i32, vp, c_u64]),
        "moe_unpack_mxfp4": (ctypes.c_int, [vp, c_u64, c_i32, c_i32, c_i32, vp, c_u64]),
        "moe_expert_bytes_mxfp8": (c_u64, [c_i32, c_i32]),
        "moe_pack_mxfp8": (ctypes.c_int, [vp, c_u64, c_i32, c_i32, vp, c_u64]),
        "moe_unpack_mxfp8": (ctypes.c_int, [vp, c_u64, c_i32, c_i32, vp, c_u64]),
        "moe_expert_bytes_affine2": (c_u64, [c_i32, c_i32]),
        "moe_pack_affine2": (ctypes.c_int, [vp, c_u64, c_i32, c_i32, c_i32, vp, c_u64]),
        "moe_unpack_affine2": (ctypes.c_int, [vp, c_u64, c_i32, c_i32, c_i32, vp, c_u64]),
        "moe_route_workspace_size": (c_sz, [c_i32, c_i32, c_i32]),
        "moe_route": (ctypes.c_int, [vp, c_i32, c_i32, vp, vp, vp, vp, c_i32, c_i32, c_i32, ctypes.c_float,
                                     vp, vp, vp, c_sz, vp]),
        "moe_dispatch_workspace_size": (c_sz, [c_i32, c_i32, c_i32]),
        "moe_dispatch": (ctypes.c_int, [vp, c_i32, c_i32, c_i32, vp, vp, vp, vp, c_sz, vp]),
        "moe_dispatch_noalloc": (ctypes.c_int, [vp, c_i32, c_i32, c_i32, vp, vp, vp, vp]),
        "moe_ffn_workspace_size": (c_sz, [c_i32, ctypes.POINTER(moe_experts), c_i32]),
        "moe_expert_ffn": (ctypes.c_int, [vp, c_i32, ctypes.POINTER(moe_experts), c_i32, vp, vp, ctypes.c_float,
                                          vp, vp, c_sz, vp]),
        "moe_expert_ffn_phase": (ctypes.c_int, [vp, c_i32, ctypes.POINTER(moe_experts), c_i32, vp, vp,
                                                ctypes.c_float, vp, vp, c_sz, c_i32, vp]),
        "moe_combine": (ctypes.c_int, [vp, vp, vp, c_i32, c_i32, c_i32, vp, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(fn: str, st: int):
    if st != 0:
        raise MoeError(fn, st)


# ---------------------------------------------------------------- host helpers
def expert_bytes(hidden: int, inter: int) -> int:
    return int(lib().moe_expert_bytes(hidden, inter))


def pack_mxfp4(canonical: np.ndarray, n_total: int, hidden: int, inter: int) -> np.ndarray:
    """Canonical MXFP4 blob (uint8, host) -> device-layout blob (uint8, host)."""
    src = np.ascontiguousarray(canonical, dtype=np.uint8)
    dst = np.empty_like(src)
    _check("moe_pack_mxfp4", lib().moe_pack_mxfp4(src.ctypes.data, src.nbytes, n_total, hidden, inter,
                                                  dst.ctypes.data, dst.nbytes))
    return dst


def unpack_mxfp4(device_layout: np.ndarray, n_total: int, hidden: int, inter: int) -> np.ndarray:
    src = np.ascontiguousarray(device_layout, dtype=np.uint8)
    dst = np.empty_like(src)
    _check("moe_unpack_mxfp4", lib().moe_unpack_mxfp4(src.ctypes.data, src.nbytes, n_total, hidden, inter,
                                                      dst.ctypes.data, dst.nbytes))
    return dst


def pack_mxfp8(canonical: np.ndarray, hidden: int, inter: int) -> np.ndarray:
    """One canonical MXFP8 expert (uint8, host) -> its device layout (uint8, host)."""
    src = np.ascontiguousarray(canonical, dtype=np.uint8)
    dst = np.empty_like(src)
    _check("moe_pack_mxfp8", lib().moe_pack_mxfp8(src.ctypes.data, src.nbytes, hidden, inter, dst.ctypes.data,
                                                  dst.nbytes))
    return dst


def unpack_mxfp8(device_layout: np.ndarray, hidden: int, inter: int) -> np.ndarray:
    src = np.ascontiguousarray(device_layout, dtype=np.uint8)
    dst = np.empty_like(src)
    _check("moe_unpack_mxfp8", lib().moe_unpack_mxfp8(src.ctypes.data, src.nbytes, hidden, inter, dst.ctypes.data,
                                                      dst.nbytes))
    return dst


def pack_affine2(canonical: np.ndarray, n_experts: int, hidden: int, inter: int) -> np.ndarray:
    """Canonical 2-bit affine routed experts (uint8, host) -> device layout (uint8, host)."""
    src = np.ascontiguousarray(canonical, dtype=np.uint8)
    dst = np.empty_like(src)
    _check("moe_pack_affine2", lib().moe_pack_affine2(src.ctypes.data, src.nbytes, n_experts, hidden, inter,
                                                      dst.ctypes.data, dst.nbytes))
    return dst


def unpack_affine2(device_layout: np.ndarray, n_experts: int, hidden: int, inter: int) -> np.ndarray:
    src = np.ascontiguousarray(device_layout, dtype=np.uint8)
    dst = np.empty_like(src)
    _check("moe_unpack_affine2", lib().moe_unpack_affine2(src.ctypes.data, src.nbytes, n_experts, hidden, inter,
                                                          dst.ctypes.data, dst.nbytes))
    return dst


# ---------------------------------------------------------------- device calls
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _dev(t, dtypes, name):
    if t is None:
        return None
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be one of {dtypes}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


class Experts:
    """A device-layout expert blob on the GPU and its C descriptor."""

    def __init__(self, blob_device, n_experts: int, hidden: int, inter: int, split_fp8: bool = False,
                 shared_mxfp8: bool = False, routed_affine2: bool = False):
        torch = _torch()
        _dev(blob_device, torch.uint8, "blob")
        self.blob = blob_device
        self.n_experts, self.hidden, self.inter = n_experts, hidden, inter
        self.desc = moe_experts()
        _check("moe_experts_init", lib().moe_experts_init(ctypes.byref(self.desc), _ptr(blob_device), n_experts,
                                                          hidden, inter))
        self.desc.flags = ((MOE_FFN_SPLIT_FP8 if split_fp8 else 0) | (MOE_SHARED_MXFP8 if shared_mxfp8 else 0)
                           | (MOE_ROUTED_AFFINE2 if routed_affine2 else 0))
        if routed_affine2:
            self.desc.expert_bytes = int(lib().moe_expert_bytes_affine2(hidden, inter))

    @classmethod
    def from_canonical(cls, canonical: np.ndarray, n_experts: int, hidden: int, inter: int, device="cuda",
                       split_fp8: bool = False, shared_mxfp8: bool = False, routed_affine2: bool = False):
        """canonical: n_experts routed experts (MXFP4, or 2-bit affine with
        routed_affine2) followed by the shared expert (MXFP4, or MXFP8 with
        shared_mxfp8)."""
        torch = _torch()
        if routed_affine2:
            nb = n_experts * int(lib().moe_expert_bytes_affine2(hidden, inter))
            routed = pack_affine2(canonical[:nb], n_experts, hidden, inter)
        else:
            nb = n_experts * int(lib().moe_expert_bytes(hidden, inter))
            routed = pack_mxfp4(canonical[:nb], n_experts, hidden, inter)
        shared = pack_mxfp8(canonical[nb:], hidden, inter) if shared_mxfp8 else pack_mxfp4(canonical[nb:], 1, hidden,
                                                                                           inter)
        packed = np.concatenate([routed, shared])
        return cls(torch.from_numpy(packed).to(device), n_experts, hidden, inter, split_fp8, shared_mxfp8,
                   routed_affine2)


def route(x, T: int, E: int, top_k: int, route_scale: float, w_router=None, sel_bias=None, token_ids=None,
          hash_table=None):
    """moe_route -> (ids int32 [T,k], weights float32 [T,k])."""
    torch = _torch()
    dev = (x if x is not None else token_ids).device
    ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    w = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    ws = None
    H = 0
    V = 0
    if hash_table is None:
        _dev(x, (torch.int16, torch.bfloat16), "x")
        _dev(w_router, torch.float32, "w_router")
        _dev(sel_bias, torch.float32, "sel_bias")
        H = x.shape[1]
        nbytes = int(lib().moe_route_workspace_size(T, H, E))
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    else:
        _dev(token_ids, torch.int32, "token_ids")
        _dev(hash_table, torch.int32, "hash_table")
        V = hash_table.shape[0]
    st = lib().moe_route(_ptr(x) if hash_table is None else None, T, H, _ptr(w_router), _ptr(sel_bias),
                         _ptr(token_ids), _ptr(hash_table), V, E, top_k, route_scale, _ptr(ids), _ptr(w),
                         _ptr(ws), 0 if ws is None else ws.numel(), _stream())
    _check("moe_route", st)
    return ids, w


def dispatch(ids, E: int):
    """moe_dispatch -> (offsets [E+2], row_token [T*(k+1)], slot_row [T, k+1]), int32."""
    torch = _torch()
    _dev(ids, torch.int32, "ids")
    T, k = ids.shape
    dev = ids.device
    offsets = torch.empty(E + 2, dtype=torch.int32, device=dev)
    row_token = torch.empty(T * (k + 1), dtype=torch.int32, device=dev)
    slot_row = torch.empty((T, k + 1), dtype=torch.int32, device=dev)
    nbytes = int(lib().moe_dispatch_workspace_size(T, E, k))
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check("moe_dispatch", lib().moe_dispatch(_ptr(ids), T, E, k, _ptr(offsets), _ptr(row_token), _ptr(slot_row),
                                              _ptr(ws), ws.numel(), _stream()))
    return offsets, row_token, slot_row


def dispatch_noalloc(ids, E: int, offsets=None, row_token=None, slot_row=None):
    """moe_dispatch_noalloc (no workspace): the outputs of dispatch(), written
    into the given tensors or new ones."""
    torch = _torch()
    _dev(ids, torch.int32, "ids")
    T, k = ids.shape
    dev = ids.device
    offsets = torch.empty(E + 2, dtype=torch.int32, device=dev) if offsets is None else offsets
    row_token = torch.empty(T * (k + 1), dtype=torch.int32, device=dev) if row_token is None else row_token
    slot_row = torch.empty((T, k + 1), dtype=torch.int32, device=dev) if slot_row is None else slot_row
    _check("moe_dispatch_noalloc", lib().moe_dispatch_noalloc(_ptr(ids), T, E, k, _ptr(offsets), _ptr(row_token),
                                                              _ptr(slot_row), _stream()))
    return offsets, row_token, slot_row


def ffn_workspace_size(T: int, experts: Experts, top_k: int) -> int:
    return int(lib().moe_ffn_workspace_size(T, ctypes.byref(experts.desc), top_k))


def expert_ffn(x, experts: Experts, top_k: int, offsets, row_token, clamp_limit: float, out_rows=None, ws=None):
    """moe_expert_ffn -> out_rows bf16 [T*(k+1), H]."""
    torch = _torch()
    T = x.shape[0]
    H = experts.hidden
    if out_rows is None:
        out_rows = torch.empty((T * (top_k + 1), H), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = torch.empty(max(ffn_workspace_size(T, experts, top_k), 1), dtype=torch.uint8, device=x.device)
    _check("moe_expert_ffn", lib().moe_expert_ffn(_ptr(x), T, ctypes.byref(experts.desc), top_k, _ptr(offsets),
                                                  _ptr(row_token), clamp_limit, _ptr(out_rows), _ptr(ws),
                                                  ws.numel(), _stream()))
    return out_rows


def combine(out_rows, slot_row, weights, T: int, H: int, top_k: int, y=None):
    """moe_combine -> y bf16 bits (int16) [T, H]."""
    torch = _torch()
    if y is None:
        y = torch.empty((T, H), dtype=torch.int16, device=out_rows.device)
    _check("moe_combine", lib().moe_combine(_ptr(out_rows), _ptr(slot_row), _ptr(weights), T, H, top_k, _ptr(y),
                                            _stream()))
    return y


class MoeLayer:
    """One MoE layer on the GPU with preallocated outputs and workspaces: the
    four C-ABI calls in order on the current stream."""

    def __init__(self, experts: Experts, T: int, top_k: int, route_scale: float, clamp_limit: float,
                 w_router=None, sel_bias=None, hash_table=None):
        torch = _torch()
        dev = experts.blob.device
        self.experts, self.T, self.k = experts, T, top_k
        self.E, self.H = experts.n_experts, experts.hidden
        self.route_scale, self.limit = route_scale, clamp_limit
        self.w_router, self.sel_bias, self.hash_table = w_router, sel_bias, hash_table
        E, k, H = self.E, top_k, self.H
        self.ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.weights = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.offsets = torch.empty(E + 2, dtype=torch.int32, device=dev)
        self.row_token = torch.empty(T * (k + 1), dtype=torch.int32, device=dev)
        self.slot_row = torch.empty((T, k + 1), dtype=torch.int32, device=dev)
        self.out_rows = torch.empty((T * (k + 1), H), dtype=torch.bfloat16, device=dev)
        self.y = torch.empty((T, H), dtype=torch.int16, device=dev)
        L = lib()
        self.ws_route = torch.empty(max(int(L.moe_route_workspace_size(T, H, E)), 256), dtype=torch.uint8, device=dev)
        self.ws_disp = torch.empty(max(int(L.moe_dispatch_workspace_size(T, E, k)), 256), dtype=torch.uint8, device=dev)
        self.ws_ffn = torch.empty(max(ffn_workspace_size(T, experts, k), 256), dtype=torch.uint8, device=dev)

    def set_experts(self, experts: Experts):
        self.experts = experts

    def route(self, x, token_ids=None):
        L = lib()
        s = _stream()
        T, k, E = self.T, self.k, self.E
        _check("moe_route", L.moe_route(_ptr(x) if self.hash_table is None else None, T, self.H,
                                        _ptr(self.w_router), _ptr(self.sel_bias), _ptr(token_ids),
                                        _ptr(self.hash_table), 0 if self.hash_table is None else self.hash_table.shape[0],
                                        E, k, self.route_scale, _ptr(self.ids), _ptr(self.weights),
                                        _ptr(self.ws_route), self.ws_route.numel(), s))

    def dispatch(self):
        _check("moe_dispatch", lib().moe_dispatch(_ptr(self.ids), self.T, self.E, self.k, _ptr(self.offsets),
                                                  _ptr(self.row_token), _ptr(self.slot_row), _ptr(self.ws_disp),
                                                  self.ws_disp.numel(), _stream()))

    def expert_ffn(self, x):
        _check("moe_expert_ffn", lib().moe_expert_ffn(_ptr(x), self.T, ctypes.byref(self.experts.desc), self.k,
                                                      _ptr(self.offsets), _ptr(self.row_token), self.limit,
                                                      _ptr(self.out_rows), _ptr(self.ws_ffn), self.ws_ffn.numel(),
                                                      _stream()))

    def expert_ffn_phase(self, x, phase: int):
        _check("moe_expert_ffn_phase", lib().moe_expert_ffn_phase(
            _ptr(x), self.T, ctypes.byref(self.experts.desc), self.k, _ptr(self.offsets), _ptr(self.row_token),
            self.limit, _ptr(self.out_rows), _ptr(self.ws_ffn), self.ws_ffn.numel(), phase, _stream()))

    def combine(self):
        _check("moe_combine", lib().moe_combine(_ptr(self.out_rows), _ptr(self.slot_row), _ptr(self.weights),
                                                self.T, self.H, self.k, _ptr(self.y), _stream()))

    def forward(self, x, token_ids=None):
        self.route(x, token_ids)
        self.dispatch()
        self.expert_ffn(x)
        self.combine()
        return self.y
