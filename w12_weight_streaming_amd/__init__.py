"""w12_weight_streaming_amd -- lossless 12-bit weight streaming for the
verification pass of greedy speculative decoding on MI355X (gfx950).

Thin ctypes binding over libw12.so (C ABI in include/w12.h), with the same
names as the C entry points: w12_pack, w12_decode, w12_check, w12_gemm,
w12_head_argmax, tree_accept. Every step of the path runs in the library's
HIP kernels; this module only checks tensor dtypes/devices, passes device
pointers and the current HIP stream, and keeps zero-filled workspaces.
There is no CPU fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw12.so")

W12_OK, W12_EINVAL, W12_ENOSPC, W12_EHIP, W12_ECORRUPT = 0, -1, -2, -3, -4
W12_Y_F32, W12_Y_BF16 = 0, 1
MFMA_MIN_ROWS = 5  # rows from which w12_gemm multiplies on the matrix cores (fewer: VALU path)
MAX_ROWS = 512

_lib = None


class W12Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib().w12_strerror(status).decode()}")


class W12Matrix(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("records", ctypes.c_void_p), ("e_top", ctypes.c_void_p),
                ("esc_off", ctypes.c_void_p), ("esc", ctypes.c_void_p)]


class W12Cert8(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("q", ctypes.c_void_p), ("qexp", ctypes.c_void_p), ("cbound", ctypes.c_void_p)]


def lib() -> ctypes.CDLL:
    """The loaded libw12.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m w12_weight_streaming_amd.build`"
                " (hipcc, gfx950). There is no fallback path.")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        mp = ctypes.POINTER(W12Matrix)
        sig = {
            "w12_strerror": (ctypes.c_char_p, [ctypes.c_int]),
            "w12_abi_version": (ctypes.c_int, []),
            "w12_num_blocks": (i64, [i64, i64]),
            "w12_pack_plan": (ctypes.c_int, [vp, i64, i64, vp, vp, vp]),
            "w12_pack": (ctypes.c_int, [vp, i64, i64, vp, vp, vp, vp, i64, vp]),
            "w12_decode": (ctypes.c_int, [mp, vp, vp]),
            "w12_check": (ctypes.c_int, [mp, vp, vp, vp]),
            "w12_gemm_workspace": (ctypes.c_int, [i64, i64, i64, ctypes.POINTER(sz)]),
            "w12_gemm": (ctypes.c_int, [mp, vp, i64, vp, ctypes.c_int, vp, sz, vp]),
            "w12_head_argmax_workspace": (ctypes.c_int, [i64, i64, i64, ctypes.POINTER(sz)]),
            "w12_head_argmax": (ctypes.c_int, [mp, vp, i64, vp, vp, vp, sz, vp]),
            "w12_gemm_qpass": (ctypes.c_int, [mp, vp, i64, vp, ctypes.c_int, vp, sz, vp]),
            "w12_gemm_noalloc": (ctypes.c_int, [mp, vp, i64, vp, ctypes.c_int, vp]),
            "w12_cert8_pack": (ctypes.c_int, [vp, i64, i64, vp, vp, vp, vp, vp]),
            "w12_head_argmax_certified_workspace": (ctypes.c_int, [i64, i64, i64, ctypes.POINTER(sz)]),
            "w12_head_argmax_certified": (ctypes.c_int, [mp, ctypes.POINTER(W12Cert8), vp, i64, vp, vp, vp, vp,
                                                         sz, vp]),
            "w12_head_argmax_qpass": (ctypes.c_int, [mp, vp, i64, vp, vp, vp, sz, vp]),
            "tree_accept": (ctypes.c_int, [i32, vp, i32, vp, vp, vp, vp, vp, vp, vp]),
            "w12_tree_build_workspace": (ctypes.c_int, [i32, i32, ctypes.POINTER(sz)]),
            "w12_tree_build": (ctypes.c_int, [i32, i32, i32, vp, vp, vp, vp, i32, vp, sz, vp, vp, vp, vp,
                                              vp, vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    return ["w12_strerror", "w12_abi_version", "w12_num_blocks", "w12_pack_plan", "w12_pack",
            "w12_decode", "w12_check", "w12_gemm_workspace", "w12_gemm",
            "w12_head_argmax_workspace", "w12_head_argmax", "w12_gemm_qpass",
            "w12_head_argmax_qpass", "tree_accept", "w12_tree_build_workspace", "w12_tree_build",
            "w12_gemm_noalloc", "w12_cert8_pack", "w12_head_argmax_certified_workspace",
            "w12_head_argmax_certified"]


def _ok(status: int, what: str):
    if status != W12_OK:
        raise W12Error(status, what)


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t: torch.Tensor, dtype, name: str, ndim: int | None = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got {t.dim()})")


@dataclass
class PackedW12:
    """Device-resident W12 matrix: the five buffers of include/w12.h."""
    n: int
    k: int
    records: torch.Tensor   # uint8 [n*k*3/2]
    e_top: torch.Tensor     # uint8 [n]
    esc_off: torch.Tensor   # int32 view of u32 [n*k/1024 + 1]
    esc: torch.Tensor       # int32 view of u32 [n_esc] (at least 1 element)
    n_esc: int

    def desc(self) -> W12Matrix:
        return W12Matrix(self.n, self.k, self.records.data_ptr(), self.e_top.data_ptr(),
                         self.esc_off.data_ptr(), self.esc.data_ptr())

    @property
    def device(self):
        return self.records.device

    def nbytes(self) -> int:
        """Packed bytes: records + e_top + esc_off + escape entries."""
        return (self.records.numel() + self.e_top.numel() + 4 * self.esc_off.numel()
                + 4 * self.n_esc)


# ------------------------------------------------------------------ workspaces

_ws_cache: dict = {}


def workspace(nbytes: int, device: torch.device, tag: str = "gemm") -> torch.Tensor:
    """Zero-filled device workspace, grown on demand and kept per (device,
    stream, tag). The library leaves it zero-filled after every call."""
    key = (device.index, torch.cuda.current_stream(device).cuda_stream, tag)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


# ------------------------------------------------------------------ entry points

def w12_pack(w: torch.Tensor, check: bool = True) -> PackedW12:
    """Pack bf16 weights [n, k] (on the GPU) into W12; with check=True run the
    load-time bit-for-bit check and raise if any weight fails to restore."""
    _need(w, torch.bfloat16, "w", 2)
    n, k = w.shape
    dev = w.device
    s = _stream(dev)
    L = lib()
    nb = L.w12_num_blocks(n, k)
    if nb < 0:
        raise W12Error(W12_EINVAL, f"w12_pack: shape {n}x{k}")
    e_top = torch.empty(n, dtype=torch.uint8, device=dev)
    esc_off = torch.empty(nb + 1, dtype=torch.int32, device=dev)
    _ok(L.w12_pack_plan(_ptr(w), n, k, _ptr(e_top), _ptr(esc_off), s), "w12_pack_plan")
    n_esc = int(esc_off[-1].item()) & 0xFFFFFFFF
    records = torch.empty(n * k * 3 // 2, dtype=torch.uint8, device=dev)
    esc = torch.empty(max(n_esc, 1), dtype=torch.int32, device=dev)
    _ok(L.w12_pack(_ptr(w), n, k, _ptr(e_top), _ptr(esc_off), _ptr(records), _ptr(esc),
                   n_esc, s), "w12_pack")
    pw = PackedW12(n, k, records, e_top, esc_off, esc, n_esc)
    if check:
        bad = w12_check(pw, w)
        if bad:
            raise W12Error(W12_ECORRUPT, f"w12_pack load-time check: {bad} weights differ")
    return pw


def w12_require_exact(pw: PackedW12, ref: torch.Tensor) -> None:
    """The load-time refusal: raise W12Error(W12_ECORRUPT) unless every
    weight of pw restores bit-for-bit to ref."""
    bad = w12_check(pw, ref)
    if bad:
        raise W12Error(W12_ECORRUPT, f"w12_check: {bad} weights differ")


def w12_decode(pw: PackedW12) -> torch.Tensor:
    out = torch.empty(pw.n, pw.k, dtype=torch.bfloat16, device=pw.device)
    d = pw.desc()
    _ok(lib().w12_decode(ctypes.byref(d), _ptr(out), _stream(pw.device)), "w12_decode")
    return out


def w12_check(pw: PackedW12, ref: torch.Tensor) -> int:
    """Number of weights whose restore differs from ref (0 = bit-exact)."""
    _need(ref, torch.bfloat16, "ref", 2)
    if tuple(ref.shape) != (pw.n, pw.k):
        raise ValueError("ref shape does not match the packed matrix")
    cnt = torch.zeros(1, dtype=torch.int64, device=pw.device)
    d = pw.desc()
    _ok(lib().w12_check(ctypes.byref(d), _ptr(ref), _ptr(cnt), _stream(pw.device)), "w12_check")
    return int(cnt.item())


def gemm_workspace_bytes(n: int, k: int, m: int) -> int:
    out = ctypes.c_size_t(0)
    _ok(lib().w12_gemm_workspace(n, k, m, ctypes.byref(out)), "w12_gemm_workspace")
    return out.value


def w12_gemm(pw: PackedW12, x: torch.Tensor, out: torch.Tensor | None = None,
             out_dtype=torch.float32, ws: torch.Tensor | None = None,
             qpass: bool = False) -> torch.Tensor:
    """y[m, n] = x[m, :] . W[n, :] with W streamed from W12 (fp32 accumulate).
    qpass=True runs w12_gemm_qpass (8-bit view, midpoint low nibbles)."""
    _need(x, torch.bfloat16, "x", 2)
    m, k = x.shape
    if k != pw.k:
        raise ValueError(f"x has k={k}, matrix has k={pw.k}")
    if out is None:
        out = torch.empty(m, pw.n, dtype=out_dtype, device=x.device)
    if out.dtype not in (torch.float32, torch.bfloat16) or tuple(out.shape) != (m, pw.n):
        raise ValueError("out must be [m, n] float32 or bfloat16")
    _need(out, out.dtype, "out", 2)
    yt = W12_Y_F32 if out.dtype == torch.float32 else W12_Y_BF16
    need = gemm_workspace_bytes(pw.n, pw.k, m)
    if ws is None:
        ws = workspace(need, x.device)
    d = pw.desc()
    fn, name = (lib().w12_gemm_qpass, "w12_gemm_qpass") if qpass else (lib().w12_gemm, "w12_gemm")
    _ok(fn(ctypes.byref(d), _ptr(x), m, _ptr(out), yt, _ptr(ws), ws.numel(), _stream(x.device)), name)
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20


def w12_gemm_noalloc(pw: PackedW12, x: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """w12_gemm with the library's own static scratch as workspace: no
    device allocation in the call (out is the caller's). Calls that overlap
    on one device race."""
    _need(x, torch.bfloat16, "x", 2)
    m, k = x.shape
    if k != pw.k:
        raise ValueError(f"x has k={k}, matrix has k={pw.k}")
    if out.dtype not in (torch.float32, torch.bfloat16) or tuple(out.shape) != (m, pw.n):
        raise ValueError("out must be [m, n] float32 or bfloat16")
    _need(out, out.dtype, "out", 2)
    yt = W12_Y_F32 if out.dtype == torch.float32 else W12_Y_BF16
    d = pw.desc()
    _ok(lib().w12_gemm_noalloc(ctypes.byref(d), _ptr(x), m, _ptr(out), yt, _stream(x.device)),
        "w12_gemm_noalloc")
    return out


def w12_head_argmax(pw: PackedW12, x: torch.Tensor, ws: torch.Tensor | None = None,
                    with_max: bool = True, qpass: bool = False):
    """Greedy token per row: (idx int32 [m], max logit float32 [m] or None).
    qpass=True runs w12_head_argmax_qpass (8-bit view, midpoint low nibbles)."""
    _need(x, torch.bfloat16, "x", 2)
    m, k = x.shape
    if k != pw.k:
        raise ValueError(f"x has k={k}, head has k={pw.k}")
    idx = torch.empty(m, dtype=torch.int32, device=x.device)
    mx = torch.empty(m, dtype=torch.float32, device=x.device) if with_max else None
    need = ctypes.c_size_t(0)
    _ok(lib().w12_head_argmax_workspace(pw.n, pw.k, m, ctypes.byref(need)),
        "w12_head_argmax_workspace")
    if ws is None:
        ws = workspace(need.value, x.device, "head")
    d = pw.desc()
    fn, name = ((lib().w12_head_argmax_qpass, "w12_head_argmax_qpass") if qpass
                else (lib().w12_head_argmax, "w12_head_argmax"))
    _ok(fn(ctypes.byref(d), _ptr(x), m, _ptr(idx), _ptr(mx), _ptr(ws), ws.numel(),
           _stream(x.device)), name)
    return idx, mx


@dataclass
class Cert8Head:
    """Device-resident INT8 copy of an LM head for the certified argmax."""
    n: int
    k: int
    q: torch.Tensor        # int8 [n*k], 8 KB records
    qexp: torch.Tensor     # uint8 [n*k/32] block scale codes
    cbound: torch.Tensor   # float32 [n] per-row bound constants

    def desc(self) -> W12Cert8:
        return W12Cert8(self.n, self.k, self.q.data_ptr(), self.qexp.data_ptr(), self.cbound.data_ptr())

    def nbytes(self) -> int:
        return self.q.numel() + self.qexp.numel() + 4 * self.cbound.numel()


def w12_cert8_pack(w: torch.Tensor, pw: PackedW12) -> Cert8Head:
    """INT8 copy of the bf16 head w [n, k], using the window tops of its
    W12 pack pw (the weights W12 escapes are left to its escape list)."""
    _need(w, torch.bfloat16, "w", 2)
    n, k = w.shape
    if (n, k) != (pw.n, pw.k):
        raise ValueError("w and its W12 pack differ in shape")
    dev = w.device
    q = torch.empty(n * k, dtype=torch.int8, device=dev)
    qexp = torch.empty(n * k // 32, dtype=torch.uint8, device=dev)
    cb = torch.empty(n, dtype=torch.float32, device=dev)
    _ok(lib().w12_cert8_pack(_ptr(w), n, k, _ptr(pw.e_top), _ptr(q), _ptr(qexp), _ptr(cb), _stream(dev)),
        "w12_cert8_pack")
    return Cert8Head(n, k, q, qexp, cb)


def w12_head_argmax_certified(pw: PackedW12, cert: Cert8Head, x: torch.Tensor, ws: torch.Tensor | None = None,
                              with_max: bool = True):
    """Certified head argmax of 1 <= m <= 64 rows: (idx int32 [m], max
    logit float32 [m] or None, rescored vocabulary rows int32 [m])."""
    _need(x, torch.bfloat16, "x", 2)
    m, k = x.shape
    if k != pw.k or (cert.n, cert.k) != (pw.n, pw.k):
        raise ValueError("x, the head and its INT8 copy must agree in shape")
    dev = x.device
    idx = torch.empty(m, dtype=torch.int32, device=dev)
    mx = torch.empty(m, dtype=torch.float32, device=dev) if with_max else None
    cnt = torch.empty(m, dtype=torch.int32, device=dev)
    need = ctypes.c_size_t(0)
    _ok(lib().w12_head_argmax_certified_workspace(pw.n, pw.k, m, ctypes.byref(need)),
        "w12_head_argmax_certified_workspace")
    if ws is None:
        ws = workspace(need.value, dev, "cert")
    d, c = pw.desc(), cert.desc()
    _ok(lib().w12_head_argmax_certified(ctypes.byref(d), ctypes.byref(c), _ptr(x), m, _ptr(idx), _ptr(mx),
                                        _ptr(cnt), _ptr(ws), ws.numel(), _stream(dev)),
        "w12_head_argmax_certified")
    return idx, mx, cnt


def tree_accept(node_off: torch.Tensor, parent: torch.Tensor, token: torch.Tensor,
                argmax: torch.Tensor):
    """Greedy tree acceptance; returns (accept_len [T], path [sum n], bonus [T])."""
    for t, nm in ((node_off, "node_off"), (parent, "parent"), (token, "token"),
                  (argmax, "argmax")):
        _need(t, torch.int32, nm, 1)
    T = node_off.numel() - 1
    total = parent.numel()
    if T < 0 or token.numel() != total or argmax.numel() != total:
        raise ValueError("tree_accept: inconsistent array sizes")
    dev = parent.device
    acc = torch.empty(max(T, 0), dtype=torch.int32, device=dev)
    path = torch.empty(total, dtype=torch.int32, device=dev)
    bonus = torch.empty(max(T, 0), dtype=torch.int32, device=dev)
    _ok(lib().tree_accept(T, _ptr(node_off), total, _ptr(parent), _ptr(token), _ptr(argmax),
                          _ptr(acc), _ptr(path), _ptr(bonus), _stream(dev)), "tree_accept")
    return acc, path, bonus


def w12_tree_build(lp: torch.Tensor, tok: torch.Tensor, depth: torch.Tensor, root: torch.Tensor,
                   budget: int, ws: torch.Tensor | None = None):
    """Best-first draft trees of R requests under one shared row budget.

    lp [R, D, K, K] fp32 edge scores, tok [R, D, K] int32, depth [R] int32,
    root [R] int32 (device tensors). Returns (node_off [R+1], parent, token,
    node_depth, score), the row arrays trimmed to node_off[R] rows."""
    _need(lp, torch.float32, "lp", 4)
    _need(tok, torch.int32, "tok", 3)
    _need(depth, torch.int32, "depth", 1)
    _need(root, torch.int32, "root", 1)
    R, D, K, K2 = lp.shape
    if K2 != K or tuple(tok.shape) != (R, D, K) or depth.numel() != R or root.numel() != R:
        raise ValueError("w12_tree_build: inconsistent shapes")
    dev = lp.device
    need = ctypes.c_size_t(0)
    _ok(lib().w12_tree_build_workspace(R, budget, ctypes.byref(need)), "w12_tree_build_workspace")
    if ws is None:
        ws = torch.empty(max(int(need.value), 16), dtype=torch.uint8, device=dev)
    node_off = torch.empty(R + 1, dtype=torch.int32, device=dev)
    parent = torch.empty(budget, dtype=torch.int32, device=dev)
    token = torch.empty(budget, dtype=torch.int32, device=dev)
    ndepth = torch.empty(budget, dtype=torch.int32, device=dev)
    score = torch.empty(budget, dtype=torch.float32, device=dev)
    _ok(lib().w12_tree_build(R, D, K, _ptr(lp), _ptr(tok), _ptr(depth), _ptr(root), budget, _ptr(ws),
                             ws.numel(), _ptr(node_off), _ptr(parent), _ptr(token), _ptr(ndepth),
                             _ptr(score), _stream(dev)), "w12_tree_build")
    n = int(node_off[-1].item())
    return node_off, parent[:n], token[:n], ndepth[:n], score[:n]
