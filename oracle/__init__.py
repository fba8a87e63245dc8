"""CPU oracle for the sparse MoE experts forward pass (ctypes front end of ``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the benchmark's CPU
baseline leg are the only callers. It shares no code with the GPU library and never imports it.

Every function restates what the layer computes, in double precision, with a plain per-token loop
over the selected experts; see ``moe_oracle.c`` for the passages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_LIB_SAN = os.path.join(_HERE, "liboracle_san.so")
_lib = None

F32, BF16, E4M3, E2M1 = 0, 1, 2, 3
SCALE_FMTS = {"f32": 0, "ue8m0": 1}   # block scales: fp32 values, or UE8M0 bytes (2^(b-127))


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` with gcc (plain -O2, OpenMP over tokens, IEEE arithmetic)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(clang: str = "/opt/rocm/llvm/bin/clang") -> str:
    """Compile ``liboracle_san.so``: the same source under AddressSanitizer and
    UndefinedBehaviorSanitizer (clang, serial: the OpenMP pragmas are ignored). Loaded instead of
    ``liboracle.so`` when MOE_ORACLE_LIBRARY names it, with clang's ASan runtime preloaded."""
    tmp = _LIB_SAN + ".tmp%d" % os.getpid()
    subprocess.check_call(
        [clang, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=undefined", "-Wno-unknown-pragmas", "-shared-libsan", "-shared",
         "-fPIC", "-o", tmp, _SRC, "-lm"]
    )
    os.replace(tmp, _LIB_SAN)
    return _LIB_SAN


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("MOE_ORACLE_LIBRARY") or _LIB
        if path == _LIB and not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(path)
        vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_value.restype = ctypes.c_double
        lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_encode.argtypes = [f32]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e2m1_value.restype = ctypes.c_double
        lib.oracle_e2m1_encode.argtypes = [f32]
        lib.oracle_e2m1_encode.restype = ctypes.c_uint8
        lib.oracle_quantize_weight_mxfp4.argtypes = [vp, i32, i32, vp, vp]
        lib.oracle_quantize_weight_mxfp4.restype = None
        lib.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e8m0_value.restype = ctypes.c_double
        lib.oracle_ue8m0_scale.argtypes = [f32]
        lib.oracle_ue8m0_scale.restype = ctypes.c_uint8
        lib.oracle_quantize_act.argtypes = [vp, i32, i32, i32, i32, vp, vp]
        lib.oracle_quantize_weight.argtypes = [vp, i32, i32, i32, vp, vp]
        lib.oracle_quantize_act_ue8m0.argtypes = [vp, i32, i32, i32, i32, vp, vp]
        lib.oracle_quantize_weight_ue8m0.argtypes = [vp, i32, i32, i32, vp, vp]
        lib.oracle_router_logits.argtypes = [vp, i32, vp, i32, i32, i32, vp]
        lib.oracle_route.argtypes = [vp, i32, i32, i32, vp, vp]
        lib.oracle_permute.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
        lib.oracle_expert_pairs.argtypes = [i32, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, i32,
                                            i32, i32, vp, vp, vp, vp]
        lib.oracle_moe_forward.argtypes = [i32, i32, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp,
                                           vp, i32, i32, vp, vp, i32, vp, vp]
        lib.oracle_combine_permuted.argtypes = [vp, vp, vp, i32, i32, i32, vp]
        lib.oracle_router_logits_f32.argtypes = [vp, i32, vp, i32, i32, i32, vp]
        lib.oracle_moe_forward_f32.argtypes = [i32, i32, i32, i32, i32, vp, i32, vp, vp, vp, vp,
                                               vp, i32, vp, vp]
        for fn in ("oracle_quantize_act", "oracle_quantize_weight", "oracle_quantize_act_ue8m0",
                   "oracle_quantize_weight_ue8m0", "oracle_router_logits",
                   "oracle_route", "oracle_permute", "oracle_expert_pairs", "oracle_moe_forward",
                   "oracle_combine_permuted", "oracle_router_logits_f32",
                   "oracle_moe_forward_f32"):
            getattr(lib, fn).restype = None
        _lib = lib
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16          # bf16 bit patterns
    if a.dtype == np.uint8:
        return E4M3          # e4m3 codes
    raise TypeError("unsupported oracle dtype %s" % a.dtype)


def _c(a: np.ndarray, dtype=None) -> np.ndarray:
    return np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))


def _ptr(a):
    return None if a is None else a.ctypes.data


# ---- number formats -------------------------------------------------------------------------

def bf16_value(bits: int) -> float:
    return _load().oracle_bf16_value(bits)


def e4m3_value(code: int) -> float:
    return _load().oracle_e4m3_value(code)


def e4m3_encode(v: float) -> int:
    return _load().oracle_e4m3_encode(v)


def e4m3_decode_array(q: np.ndarray) -> np.ndarray:
    table = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(q, dtype=np.uint8)]


def e8m0_value(b: int) -> float:
    return _load().oracle_e8m0_value(b)


def ue8m0_scale(amax: float) -> int:
    return _load().oracle_ue8m0_scale(amax)


def e8m0_decode_array(b: np.ndarray) -> np.ndarray:
    table = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(b, dtype=np.uint8)]


def e2m1_value(code: int) -> float:
    return _load().oracle_e2m1_value(code)


def e2m1_encode(v: float) -> int:
    return _load().oracle_e2m1_encode(v)


def e2m1_decode_packed(q: np.ndarray) -> np.ndarray:
    """Packed FP4 [..., K/2] bytes -> float64 [..., K] (element 2j in the low nibble of byte j)."""
    table = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
    q = np.asarray(q, dtype=np.uint8)
    out = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), np.float64)
    out[..., 0::2] = table[q & 0xF]
    out[..., 1::2] = table[q >> 4]
    return out


def quantize_weight_mxfp4(W: np.ndarray):
    """W [..., N, K] fp32 -> (q [..., N, K/2] packed e2m1, s [..., N, K/32] UE8M0 bytes)."""
    if not np.issubdtype(np.asarray(W).dtype, np.floating):
        raise TypeError("quantize_weight_mxfp4 takes float values (decode bf16 bits first)")
    W = _c(W, np.float32)
    lead, (N, K) = W.shape[:-2], W.shape[-2:]
    assert K % 32 == 0
    Wf = W.reshape(-1, N, K)
    q = np.empty((Wf.shape[0], N, K // 2), np.uint8)
    s = np.empty((Wf.shape[0], N, K // 32), np.uint8)
    lib = _load()
    for e in range(Wf.shape[0]):
        lib.oracle_quantize_weight_mxfp4(Wf[e].ctypes.data, N, K, q[e].ctypes.data,
                                         s[e].ctypes.data)
    return q.reshape(lead + (N, K // 2)), s.reshape(lead + (N, K // 32))


def scale_values(s: np.ndarray, scale_fmt: str = "f32") -> np.ndarray:
    """Block scales as float64 values (fp32 scales as they are, UE8M0 bytes decoded)."""
    return e8m0_decode_array(s) if scale_fmt == "ue8m0" else np.asarray(s, np.float64)


# ---- fine-grained FP8 rule --------------------------------------------------------------------

def quantize_act(x: np.ndarray, group: int = 128, scale_fmt: str = "f32"):
    """x [M, K] fp32 or bf16 bits -> (q [M, K] uint8 e4m3, s [M, K/group]): fp32 scales, or
    UE8M0 bytes for scale_fmt="ue8m0"."""
    x = _c(x)
    M, K = x.shape
    assert K % group == 0
    q = np.empty((M, K), np.uint8)
    lib = _load()
    if scale_fmt == "ue8m0":
        s = np.empty((M, K // group), np.uint8)
        lib.oracle_quantize_act_ue8m0(x.ctypes.data, _dtype_code(x), M, K, group, q.ctypes.data,
                                      s.ctypes.data)
    else:
        s = np.empty((M, K // group), np.float32)
        lib.oracle_quantize_act(x.ctypes.data, _dtype_code(x), M, K, group, q.ctypes.data,
                                s.ctypes.data)
    return q, s


def quantize_weight(W: np.ndarray, block: int = 128, scale_fmt: str = "f32"):
    """W [..., N, K] fp32 -> (q [..., N, K] e4m3, s [..., N/block, K/block]): fp32 scales, or
    UE8M0 bytes for scale_fmt="ue8m0"."""
    W = _c(W, np.float32)
    lead, (N, K) = W.shape[:-2], W.shape[-2:]
    assert N % block == 0 and K % block == 0
    Wf = W.reshape(-1, N, K)
    q = np.empty(Wf.shape, np.uint8)
    ue = scale_fmt == "ue8m0"
    s = np.empty((Wf.shape[0], N // block, K // block), np.uint8 if ue else np.float32)
    lib = _load()
    fn = lib.oracle_quantize_weight_ue8m0 if ue else lib.oracle_quantize_weight
    for e in range(Wf.shape[0]):
        fn(Wf[e].ctypes.data, N, K, block, q[e].ctypes.data, s[e].ctypes.data)
    return q.reshape(W.shape), s.reshape(lead + (N // block, K // block))


# ---- router ----------------------------------------------------------------------------------

def router_logits(x: np.ndarray, Wr: np.ndarray) -> np.ndarray:
    x = _c(x)
    Wr = _c(Wr, np.float32)
    T, d = x.shape
    E = Wr.shape[0]
    out = np.empty((T, E), np.float32)
    _load().oracle_router_logits(x.ctypes.data, _dtype_code(x), Wr.ctypes.data, T, d, E,
                                 out.ctypes.data)
    return out


def route(logits: np.ndarray, k: int):
    """logits [T, E] fp32 -> (ids [T, k] int32, w [T, k] fp32)."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    assert 1 <= k <= E
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _load().oracle_route(logits.ctypes.data, T, E, k, ids.ctypes.data, w.ctypes.data)
    return ids, w


def permute(ids: np.ndarray, E: int):
    """ids [T, k] -> (counts [E], offsets [E+1], sorted_pair [T*k], pair_pos [T*k]) int32."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    P = T * k
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sp = np.empty(P, np.int32)
    pp = np.empty(P, np.int32)
    _load().oracle_permute(ids.ctypes.data, T, k, E, counts.ctypes.data, offsets.ctypes.data,
                           sp.ctypes.data, pp.ctypes.data)
    return counts, offsets, sp, pp


# ---- experts and the layer ---------------------------------------------------------------------

class Experts:
    """Expert weights: W_gate, W_up [E, f, d]; W_down [E, d, f] (fp32, bf16 bits or e4m3 codes).

    For e4m3 weights the block scales s_gate, s_up [E, f/128, d/128] and s_down
    [E, d/128, f/128] are required: fp32, or UE8M0 bytes with ``scale_fmt="ue8m0"`` (then the
    activation rule uses UE8M0 scales too). ``quant_act`` applies the fp8 activation rule to x
    and h.
    """

    def __init__(self, w_gate, w_up, w_down, s_gate=None, s_up=None, s_down=None,
                 quant_act=False, scale_fmt="f32", w_fp4=False):
        self.w_gate, self.w_up, self.w_down = _c(w_gate), _c(w_up), _c(w_down)
        self.E, self.f, self.d = self.w_gate.shape
        if w_fp4:  # packed FP4: two input channels per byte, MX scales [.., rows, cols/32]
            self.d *= 2
            assert self.w_down.shape == (self.E, self.d, self.f // 2) and scale_fmt == "ue8m0"
        else:
            assert self.w_down.shape == (self.E, self.d, self.f)
        assert self.w_up.shape == self.w_gate.shape
        self.w_dtype = E2M1 if w_fp4 else _dtype_code(self.w_gate)
        self.scale_fmt = scale_fmt
        sdt = np.uint8 if scale_fmt == "ue8m0" else np.float32
        self.s_gate = None if s_gate is None else _c(s_gate, sdt)
        self.s_up = None if s_up is None else _c(s_up, sdt)
        self.s_down = None if s_down is None else _c(s_down, sdt)
        if self.w_dtype in (E4M3, E2M1):
            assert self.s_gate is not None and self.s_up is not None and self.s_down is not None
        self.quant_act = bool(quant_act)

    def _wargs(self):
        return (self.w_dtype, _ptr(self.w_gate), _ptr(self.w_up), _ptr(self.w_down),
                _ptr(self.s_gate), _ptr(self.s_up), _ptr(self.s_down), int(self.quant_act),
                SCALE_FMTS[self.scale_fmt])


def expert_pairs(x: np.ndarray, experts: Experts, tok: np.ndarray, exp_of: np.ndarray,
                 want_h=True, want_y=True):
    """Per (token, expert) pair: h [n, f] (before any h quantisation) and unweighted y [n, d]."""
    x = _c(x)
    tok = _c(tok, np.int32)
    exp_of = _c(exp_of, np.int32)
    n = tok.size
    h = np.empty((n, experts.f), np.float64) if want_h else None
    y = np.empty((n, experts.d), np.float64) if want_y else None
    _load().oracle_expert_pairs(experts.d, experts.f, _dtype_code(x), x.ctypes.data,
                                *experts._wargs(), n, tok.ctypes.data, exp_of.ctypes.data,
                                _ptr(h), _ptr(y))
    return h, y


def moe_forward(x: np.ndarray, experts: Experts, ids: np.ndarray, w: np.ndarray,
                tokens=None) -> np.ndarray:
    """out[t] = sum_j w[t,j] * expert_{ids[t,j]}(x[t]) for the listed tokens (all if None).

    Returns float64 [n_tok, d] in the order of ``tokens``.
    """
    x = _c(x)
    ids = _c(ids, np.int32)
    w = _c(w, np.float32)
    T, d = x.shape
    k = ids.shape[1]
    assert d == experts.d and ids.shape == (T, k) and w.shape == (T, k)
    tl = None if tokens is None else _c(np.asarray(tokens), np.int32)
    n_tok = T if tl is None else tl.size
    out = np.empty((n_tok, d), np.float64)
    _load().oracle_moe_forward(T, d, experts.f, k, _dtype_code(x), x.ctypes.data,
                               *experts._wargs(), ids.ctypes.data, w.ctypes.data, n_tok, _ptr(tl),
                               out.ctypes.data)
    return out


def router_logits_f32(x: np.ndarray, Wr: np.ndarray) -> np.ndarray:
    """router_logits with the sum in fp32 (ascending i) instead of fp64."""
    x = _c(x)
    Wr = _c(Wr, np.float32)
    T, d = x.shape
    E = Wr.shape[0]
    out = np.empty((T, E), np.float32)
    _load().oracle_router_logits_f32(x.ctypes.data, _dtype_code(x), Wr.ctypes.data, T, d, E,
                                     out.ctypes.data)
    return out


def moe_forward_f32(x: np.ndarray, experts: Experts, ids: np.ndarray, w: np.ndarray,
                    tokens=None) -> np.ndarray:
    """moe_forward with every sum in fp32 (fp32 or bf16 inputs and weights only): the plain fp32
    per-token loop. Returns float32 [n_tok, d]."""
    assert experts.w_dtype in (F32, BF16) and not experts.quant_act
    x = _c(x)
    ids = _c(ids, np.int32)
    w = _c(w, np.float32)
    T, d = x.shape
    k = ids.shape[1]
    tl = None if tokens is None else _c(np.asarray(tokens), np.int32)
    n_tok = T if tl is None else tl.size
    out = np.empty((n_tok, d), np.float32)
    _load().oracle_moe_forward_f32(T, d, experts.f, k, _dtype_code(x), x.ctypes.data,
                                   experts.w_dtype, _ptr(experts.w_gate), _ptr(experts.w_up),
                                   _ptr(experts.w_down), ids.ctypes.data, w.ctypes.data, n_tok,
                                   _ptr(tl), out.ctypes.data)
    return out


def combine_permuted(y: np.ndarray, pair_pos: np.ndarray, w: np.ndarray) -> np.ndarray:
    """out[t] = sum_j w[t,j] * y[pair_pos[t*k+j]] with y [T*k, d] in sorted-pair order."""
    y = _c(y, np.float64)
    pair_pos = _c(pair_pos, np.int32)
    w = _c(w, np.float32)
    T, k = w.shape
    d = y.shape[1]
    out = np.empty((T, d), np.float64)
    _load().oracle_combine_permuted(y.ctypes.data, pair_pos.ctypes.data, w.ctypes.data, T, k, d,
                                    out.ctypes.data)
    return out


def layer(x: np.ndarray, experts: Experts, k: int, logits=None, Wr=None, tokens=None):
    """Full layer on the CPU: logits (given, or x . Wr^T), route, experts, combine.

    Returns dict with logits, ids, w, counts, offsets, sorted_pair, pair_pos, out.
    """
    if logits is None:
        logits = router_logits(x, Wr)
    ids, w = route(logits, k)
    counts, offsets, sp, pp = permute(ids, experts.E)
    out = moe_forward(x, experts, ids, w, tokens)
    return dict(logits=logits, ids=ids, w=w, counts=counts, offsets=offsets, sorted_pair=sp,
                pair_pos=pp, out=out)
