"""Python binding of libmoe, the MI355X (gfx950) sparse mixture-of-experts experts forward pass.

Argument marshalling only: every step runs in the HIP kernels of ``libmoe.so`` behind the C ABI
declared in ``include/moe.h``. PyTorch provides device memory and the current HIP stream. There is
no fallback: if the library is missing, using any op raises.

The functions carry the names of the C entry points: ``moe_route``, ``moe_permute``,
``fp8_quantize_act``, ``fp8_quantize_weight``, ``moe_experts_forward``, ``moe_combine``; plus
``moe_layer`` which chains them into one layer forward.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_LIBRARY names another build of the same library (the host-sanitized one, for CPU checks)
LIB_PATH = os.environ.get("MOE_LIBRARY") or os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL, \
    MOE_ERR_DEVICE = range(5)
MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_FP4_E2M1 = range(4)
MOE_Y_PERMUTED, MOE_Y_SLOTS, MOE_Y_ACC_F32 = range(3)

_LAYOUTS = {"permuted": MOE_Y_PERMUTED, "slots": MOE_Y_SLOTS, "acc_f32": MOE_Y_ACC_F32}

# Every symbol include/moe.h declares.
EXPORTED_SYMBOLS = (
    "moe_status_string", "moe_route", "moe_permute", "moe_permute_workspace_size",
    "fp8_quantize_act", "fp8_quantize_weight", "fp8_quantize_act_ue8m0",
    "fp8_quantize_weight_ue8m0", "fp4_quantize_weight_mx", "fp4_tile_weight",
    "moe_experts_forward",
    "moe_experts_workspace_size", "moe_combine", "moe_fused_forward", "moe_fused_workspace_size",
    "moe_fused_forward_noalloc", "moe_experts_small_batch",
)
NOALLOC_SCRATCH_BYTES = 32 << 20   # MOE_NOALLOC_SCRATCH_BYTES


class MoeError(RuntimeError):
    """A device-side failure reported by libmoe (MOE_ERR_DEVICE)."""


class moe_experts_args(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int), ("d", ctypes.c_int), ("f", ctypes.c_int), ("E", ctypes.c_int),
        ("k", ctypes.c_int),
        ("act_dtype", ctypes.c_int), ("w_dtype", ctypes.c_int), ("y_dtype", ctypes.c_int),
        ("y_layout", ctypes.c_int),
        ("x", ctypes.c_void_p), ("x_scales", ctypes.c_void_p),
        ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
        ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p),
        ("offsets", ctypes.c_void_p), ("sorted_pair", ctypes.c_void_p),
        ("topk_w", ctypes.c_void_p), ("y", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("scale_fmt", ctypes.c_int), ("phase", ctypes.c_int),
    ]


class moe_fused_args(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int), ("d", ctypes.c_int), ("f", ctypes.c_int), ("E", ctypes.c_int),
        ("k", ctypes.c_int),
        ("x_dtype", ctypes.c_int), ("w_dtype", ctypes.c_int), ("scale_fmt", ctypes.c_int),
        ("x", ctypes.c_void_p), ("logits", ctypes.c_void_p), ("w_router", ctypes.c_void_p),
        ("logits_out", ctypes.c_void_p),
        ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
        ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("out_dtype", ctypes.c_int),
        ("topk_ids", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


_SCALE_FMTS = {"f32": 0, "ue8m0": 1}   # moe_scale_fmt
MOE_SCALE_F32, MOE_SCALE_UE8M0 = 0, 1
MOE_PHASE_ALL, MOE_PHASE_GATE_UP, MOE_PHASE_DOWN = 0, 1, 2
_PHASES = {"all": MOE_PHASE_ALL, "gate_up": MOE_PHASE_GATE_UP, "down": MOE_PHASE_DOWN}


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libmoe.so not found at %s; build it with "
                          "`python -m mixture_experts_ffn_softmax_amd.build`" % path)
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    st = ctypes.c_int
    sig = {
        "moe_status_string": ([st], ctypes.c_char_p),
        "moe_route": ([vp, vp, i32, vp, i32, i32, i32, i32, vp, vp, vp, vp], st),
        "moe_permute": ([vp, i32, i32, i32, vp, vp, vp, vp, vp, i32, vp, i32, vp, vp, vp, sz, vp],
                        st),
        "moe_permute_workspace_size": ([i32, i32, i32], sz),
        "fp8_quantize_act": ([vp, i32, i32, i32, i32, vp, vp, vp, vp], st),
        "fp8_quantize_weight": ([vp, i32, i32, i32, i32, i32, vp, vp, vp], st),
        "fp8_quantize_act_ue8m0": ([vp, i32, i32, i32, i32, vp, vp, vp, vp], st),
        "fp8_quantize_weight_ue8m0": ([vp, i32, i32, i32, i32, i32, vp, vp, vp], st),
        "fp4_quantize_weight_mx": ([vp, i32, i32, i32, i32, vp, vp, vp], st),
        "fp4_tile_weight": ([vp, i32, i32, i32, vp, vp], st),
        "moe_experts_forward": ([ctypes.POINTER(moe_experts_args), vp], st),
        "moe_experts_workspace_size": ([i32, i32, i32, i32, i32, i32, i32], sz),
        "moe_combine": ([vp, i32, i32, vp, vp, i32, i32, i32, vp, i32, vp], st),
        "moe_fused_forward": ([ctypes.POINTER(moe_fused_args), vp], st),
        "moe_fused_workspace_size": ([i32, i32, i32, i32, i32, i32, i32], sz),
        "moe_fused_forward_noalloc": ([ctypes.POINTER(moe_fused_args), vp], st),
        "moe_experts_small_batch": ([i32, i32, i32, i32, i32, i32, i32], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(status: int):
    if status == MOE_OK:
        return
    name = load_library().moe_status_string(status).decode()
    if status == MOE_ERR_DEVICE:
        raise MoeError(name)
    raise ValueError(name)


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return MOE_FP8_E4M3
    raise TypeError("unsupported dtype %s" % t.dtype)


def _torch_dtype(code: int):
    return {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16}[code]


def _contig(t):
    if t is not None and not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return t


# ---- the C entry points ---------------------------------------------------------------------

def moe_route(k: int, logits=None, x=None, w_router=None, logits_out=None):
    """Softmax top-k routing. Give ``logits`` [T, E] fp32, or ``x`` [T, d] and ``w_router`` [E, d]
    to compute fp32 logits on the device. Returns (topk_ids [T,k] int32, topk_w [T,k] fp32,
    logits [T,E] fp32)."""
    lib = load_library()
    for t in (logits, x, w_router, logits_out):
        _contig(t)
    if logits is not None:
        T, E = logits.shape
        d = 0
        dev = logits.device
    else:
        T, d = x.shape
        E = w_router.shape[0]
        dev = x.device
        if logits_out is None:
            logits_out = torch.empty((T, E), dtype=torch.float32, device=dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _check(lib.moe_route(_ptr(logits), _ptr(x), _dtype_code(x) if x is not None else MOE_F32,
                         _ptr(w_router), T, d, E, k, _ptr(logits_out), _ptr(ids), _ptr(w),
                         _stream()))
    return ids, w, (logits if logits is not None else logits_out)


@dataclass
class Permutation:
    counts: torch.Tensor
    offsets: torch.Tensor
    sorted_pair: torch.Tensor
    pair_pos: torch.Tensor
    x_perm: torch.Tensor | None = None
    x_perm_scales: torch.Tensor | None = None


def moe_permute(topk_ids: torch.Tensor, E: int, x=None, x_scales=None, workspace=None):
    """Group the T*k pairs by expert (stable). Optionally gather x rows into sorted order."""
    lib = load_library()
    _contig(topk_ids)
    T, k = topk_ids.shape
    P = T * k
    dev = topk_ids.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sp = torch.empty(P, dtype=torch.int32, device=dev)
    pp = torch.empty(P, dtype=torch.int32, device=dev)
    nbytes = lib.moe_permute_workspace_size(T, k, E)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    x_perm = xps = None
    d = 0
    xdt = MOE_F32
    if x is not None:
        _contig(x)
        d = x.shape[1]
        xdt = _dtype_code(x)
        x_perm = torch.empty((P, d), dtype=x.dtype, device=dev)
        if xdt == MOE_FP8_E4M3:
            xps = torch.empty((P, d // 128), dtype=torch.float32, device=dev)
    _check(lib.moe_permute(_ptr(topk_ids), T, k, E, _ptr(counts), _ptr(offsets), _ptr(sp),
                           _ptr(pp), _ptr(x), xdt, _ptr(x_scales), d, _ptr(x_perm), _ptr(xps),
                           _ptr(workspace), workspace.numel(), _stream()))
    return Permutation(counts, offsets, sp, pp, x_perm, xps)


def fp8_quantize_act(x: torch.Tensor, group: int = 128, row_index=None, scale_fmt: str = "f32"):
    """Per-row, per-128-channel dynamic e4m3 quantisation. Returns (q uint8 [M,K], scales):
    fp32 scales, or e8m0 bytes (uint8) for scale_fmt="ue8m0"."""
    lib = load_library()
    _contig(x)
    M = row_index.numel() if row_index is not None else x.shape[0]
    K = x.shape[1]
    ue = _SCALE_FMTS[scale_fmt] == 1
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    s = torch.empty((M, max(K // group, 1)), dtype=torch.uint8 if ue else torch.float32,
                    device=x.device)
    fn = lib.fp8_quantize_act_ue8m0 if ue else lib.fp8_quantize_act
    _check(fn(_ptr(x), _dtype_code(x), M, K, group, _ptr(row_index), _ptr(q), _ptr(s), _stream()))
    return q, s


def fp8_quantize_weight(w: torch.Tensor, block: int = 128, scale_fmt: str = "f32"):
    """128x128 block e4m3 quantisation of [batch, N, K] (or [N, K]) weights; scales fp32, or
    e8m0 bytes for scale_fmt="ue8m0"."""
    lib = load_library()
    _contig(w)
    shape = w.shape
    batch = 1 if w.dim() == 2 else int(torch.tensor(shape[:-2]).prod())
    N, K = shape[-2], shape[-1]
    ue = _SCALE_FMTS[scale_fmt] == 1
    q = torch.empty(shape, dtype=torch.uint8, device=w.device)
    s = torch.empty(tuple(shape[:-2]) + (max(N // block, 1), max(K // block, 1)),
                    dtype=torch.uint8 if ue else torch.float32, device=w.device)
    fn = lib.fp8_quantize_weight_ue8m0 if ue else lib.fp8_quantize_weight
    _check(fn(_ptr(w), _dtype_code(w), batch, N, K, block, _ptr(q), _ptr(s), _stream()))
    return q, s


def fp4_quantize_weight_mx(w: torch.Tensor, tiled: bool = False):
    """E2M1 quantisation of [batch, N, K] (or [N, K]) weights with one e8m0 scale per row per 32
    input channels. Returns (q uint8 [..., N, K/2] packed, element 2j in the low nibble of byte
    j; scales uint8 [..., N, K/32]). ``tiled``: q in the matrix-fragment order that
    moe_experts_forward takes (see fp4_tile_weight)."""
    lib = load_library()
    _contig(w)
    shape = w.shape
    batch = 1 if w.dim() == 2 else int(torch.tensor(shape[:-2]).prod())
    N, K = shape[-2], shape[-1]
    q = torch.empty(tuple(shape[:-1]) + (max(K // 2, 1),), dtype=torch.uint8, device=w.device)
    s = torch.empty(tuple(shape[:-1]) + (max(K // 32, 1),), dtype=torch.uint8, device=w.device)
    _check(lib.fp4_quantize_weight_mx(_ptr(w), _dtype_code(w), batch, N, K, _ptr(q), _ptr(s),
                                      _stream()))
    if tiled:
        q = fp4_tile_weight(q)
    return q, s


def fp4_tile_weight(q: torch.Tensor) -> torch.Tensor:
    """Packed E2M1 rows [..., N, K/2] -> the same bytes in matrix-fragment order (a new tensor
    of the same shape): for each 16-row group and 128-wide K block, 1 KB holding 16 bytes per
    lane l = r + 16 g (row r of the group, K = 32 g .. 32 g + 31 of the block)."""
    lib = load_library()
    _contig(q)
    N, K = q.shape[-2], 2 * q.shape[-1]
    batch = 1 if q.dim() == 2 else int(torch.tensor(q.shape[:-2]).prod())
    out = torch.empty_like(q)
    _check(lib.fp4_tile_weight(_ptr(q), batch, N, K, _ptr(out), _stream()))
    return out


def experts_small_batch(T, d, f, E, k, act_dtype: int, w_dtype: int) -> int:
    """1 if moe_experts_forward takes the small-batch kernels for these sizes, 0 for the tiled
    grouped GEMMs, -1 if it has no kernel for them (moe_experts_small_batch)."""
    return load_library().moe_experts_small_batch(T, d, f, E, k, act_dtype, w_dtype)


def experts_workspace_bytes(T, d, f, E, k, act_dtype: int, w_dtype: int) -> int:
    return load_library().moe_experts_workspace_size(T, d, f, E, k, act_dtype, w_dtype)


def moe_experts_forward(x, w_gate, w_up, w_down, offsets, sorted_pair, topk_w, k: int,
                        y_layout: str = "slots", y_dtype=None, x_scales=None, s_gate=None,
                        s_up=None, s_down=None, y=None, workspace=None, phase: str = "all",
                        scale_fmt: str = "f32", w_fp4: bool = False):
    """Both grouped projections. Returns y in ``y_layout`` ("permuted" [P,d], "slots" [T,k,d],
    "acc_f32" [T,d] fp32). ``phase``: "all", or "gate_up" then "down" as two calls on one
    ``workspace`` (pass the same workspace and y to both).
    ``scale_fmt``: fp8 block scales as fp32 values ("f32") or e8m0 bytes ("ue8m0").
    ``w_fp4``: the uint8 weights are packed E2M1 in matrix-fragment order (fp4_quantize_weight_mx
    with tiled=True) with MX scales."""
    lib = load_library()
    for t in (x, w_gate, w_up, w_down, offsets, sorted_pair, topk_w, x_scales, s_gate, s_up,
              s_down):
        _contig(t)
    T, d = x.shape
    E, f, _ = w_gate.shape
    act = _dtype_code(x)
    wdt = _dtype_code(w_gate)
    if w_fp4:
        if w_gate.dtype != torch.uint8 or 2 * w_gate.shape[2] != d:
            raise ValueError("E2M1 weights are uint8 [E, f, d/2]")
        wdt = MOE_FP4_E2M1
    layout = _LAYOUTS[y_layout]
    if y_dtype is None:
        y_dtype = torch.float32 if act == MOE_F32 else torch.bfloat16
    if layout == MOE_Y_ACC_F32:
        y_dtype = torch.float32
    P = T * k
    if y is None:
        shape = {MOE_Y_PERMUTED: (P, d), MOE_Y_SLOTS: (T, k, d), MOE_Y_ACC_F32: (T, d)}[layout]
        y = torch.empty(shape, dtype=y_dtype, device=x.device)
    nbytes = lib.moe_experts_workspace_size(T, d, f, E, k, act, wdt)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    a = moe_experts_args(T, d, f, E, k, act, wdt, _dtype_code(y), layout, x.data_ptr(),
                         x_scales.data_ptr() if x_scales is not None else None,
                         w_gate.data_ptr(), w_up.data_ptr(), w_down.data_ptr(),
                         s_gate.data_ptr() if s_gate is not None else None,
                         s_up.data_ptr() if s_up is not None else None,
                         s_down.data_ptr() if s_down is not None else None,
                         offsets.data_ptr(), sorted_pair.data_ptr(),
                         topk_w.data_ptr() if topk_w is not None else None, y.data_ptr(),
                         workspace.data_ptr(), workspace.numel(), _SCALE_FMTS[scale_fmt],
                         _PHASES[phase])
    _check(lib.moe_experts_forward(ctypes.byref(a), _stream()))
    return y


def moe_combine(y, layout: str, T: int, k: int, d: int, pair_pos=None, topk_w=None,
                out_dtype=torch.bfloat16, out=None):
    """Weighted sum of each token's k expert outputs -> out [T, d]."""
    lib = load_library()
    _contig(y)
    if out is None:
        out = torch.empty((T, d), dtype=out_dtype, device=y.device)
    _check(lib.moe_combine(_ptr(y), _dtype_code(y), _LAYOUTS[layout], _ptr(pair_pos),
                           _ptr(topk_w), T, k, d, _ptr(out), _dtype_code(out), _stream()))
    return out


def moe_fused_forward(x, w_gate, w_up, w_down, k: int, logits=None, w_router=None, s_gate=None,
                      s_up=None, s_down=None, w_fp4: bool = False, out_dtype=None,
                      workspace=None, out=None, logits_out=None, noalloc: bool = False,
                      topk_ids=None, topk_w=None):
    """The whole layer for small batches (T*k <= 256) in one call (moe_fused_forward).
    Weights as for moe_layer (bf16; uint8 e4m3 codes with fp32 or uint8 (UE8M0) block scales; with
    w_fp4, E2M1 codes in fragment order with MX scales). Returns (out [T, d], topk_ids, topk_w).
    ``noalloc``: call moe_fused_forward_noalloc (the library's own device scratch array instead of
    a workspace); with ``out``, ``topk_ids`` and ``topk_w`` given, nothing is allocated here
    either."""
    lib = load_library()
    for t in (x, w_gate, w_up, w_down, logits, w_router, s_gate, s_up, s_down):
        _contig(t)
    T, d = x.shape
    E, f = w_gate.shape[0], w_gate.shape[1]
    if w_fp4:
        wdt = MOE_FP4_E2M1
    elif w_gate.dtype in (torch.uint8, torch.float8_e4m3fn):
        wdt = MOE_FP8_E4M3
    else:
        wdt = _dtype_code(w_gate)
    fmt = "ue8m0" if s_gate is not None and s_gate.dtype == torch.uint8 else "f32"
    if out_dtype is None:
        out_dtype = torch.float32 if x.dtype == torch.float32 else torch.bfloat16
    if out is None:
        out = torch.empty((T, d), dtype=out_dtype, device=x.device)
    ids = topk_ids if topk_ids is not None else \
        torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = topk_w if topk_w is not None else torch.empty((T, k), dtype=torch.float32, device=x.device)
    _contig(ids)
    _contig(w)
    if not noalloc and workspace is None:
        nbytes = lib.moe_fused_workspace_size(T, d, f, E, k, wdt, _dtype_code(out))
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    p = lambda t: t.data_ptr() if t is not None else None
    a = moe_fused_args(T, d, f, E, k, _dtype_code(x), wdt, _SCALE_FMTS[fmt], p(x), p(logits),
                       p(w_router), p(logits_out), p(w_gate), p(w_up), p(w_down), p(s_gate),
                       p(s_up), p(s_down), p(out), _dtype_code(out), p(ids), p(w),
                       p(workspace), workspace.numel() if workspace is not None else 0)
    fn = lib.moe_fused_forward_noalloc if noalloc else lib.moe_fused_forward
    _check(fn(ctypes.byref(a), _stream()))
    return out, ids, w


# ---- the whole layer ------------------------------------------------------------------------

@dataclass
class LayerResult:
    out: torch.Tensor
    topk_ids: torch.Tensor
    topk_w: torch.Tensor
    logits: torch.Tensor
    perm: Permutation


def moe_layer(x, w_gate, w_up, w_down, k: int, logits=None, w_router=None, y_layout="slots",
              s_gate=None, s_up=None, s_down=None, out_dtype=None,
              w_fp4: bool = False) -> LayerResult:
    """route -> permute -> (fp8: quantise x) -> experts -> combine, all on the device.

    For fp8 weights (uint8 e4m3 codes with block scales s_*), x is given in bf16/fp32 and quantised
    per token per 128 channels here; uint8 scales select the UE8M0 scale format. ``w_fp4``:
    packed E2M1 weights in matrix-fragment order with MX scales (e4m3 activations, UE8M0 scales).
    """
    E = w_gate.shape[0]
    T, d = x.shape
    ids, w, lg = moe_route(k, logits=logits, x=None if logits is not None else x,
                           w_router=w_router)
    perm = moe_permute(ids, E)
    if out_dtype is None:
        out_dtype = torch.float32 if x.dtype == torch.float32 else torch.bfloat16
    x_in, xs = x, None
    fmt = "ue8m0" if s_gate is not None and s_gate.dtype == torch.uint8 else "f32"
    if w_gate.dtype in (torch.uint8, torch.float8_e4m3fn):
        x_in, xs = fp8_quantize_act(x, scale_fmt=fmt)
    y = moe_experts_forward(x_in, w_gate, w_up, w_down, perm.offsets, perm.sorted_pair, w, k,
                            y_layout=y_layout, x_scales=xs, s_gate=s_gate, s_up=s_up,
                            s_down=s_down,
                            y_dtype=torch.float32 if out_dtype == torch.float32 else None,
                            scale_fmt=fmt, w_fp4=w_fp4)
    out = moe_combine(y, y_layout, T, k, d, pair_pos=perm.pair_pos, topk_w=w,
                      out_dtype=out_dtype)
    return LayerResult(out, ids, w, lg, perm)
