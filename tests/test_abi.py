"""The C ABI library: it loads without a GPU, exports every symbol include/moe.h declares, and
rejects bad arguments on the host before anything is enqueued (no compute calls here)."""
import ctypes
import os
import re
import subprocess

import pytest

import mixture_experts_ffn_softmax_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

# A non-null address that is never dereferenced: every call below fails validation first.
FAKE = ctypes.c_void_p(0x1000)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        from mixture_experts_ffn_softmax_amd import build
        build.build()
    return moe.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "sizeof")))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("moe_route", "moe_permute", "moe_experts_forward", "moe_combine",
              "fp8_quantize_act"):
        assert n in names
    assert sorted(moe.EXPORTED_SYMBOLS) == names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for n in _declared_functions():
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_status_strings(lib):
    assert lib.moe_status_string(0) == b"MOE_OK"
    assert lib.moe_status_string(3) == b"MOE_ERR_WORKSPACE_TOO_SMALL"
    assert lib.moe_status_string(99) == b"MOE_ERR_UNKNOWN"


def test_route_validation(lib):
    INV, UNS = moe.MOE_ERR_INVALID_ARGUMENT, moe.MOE_ERR_UNSUPPORTED
    # k > E, k < 1, T < 1
    assert lib.moe_route(FAKE, None, 0, None, 4, 0, 2, 3, None, FAKE, FAKE, None) == INV
    assert lib.moe_route(FAKE, None, 0, None, 4, 0, 8, 0, None, FAKE, FAKE, None) == INV
    assert lib.moe_route(FAKE, None, 0, None, 0, 0, 8, 2, None, FAKE, FAKE, None) == INV
    # too many experts / too large k
    assert lib.moe_route(FAKE, None, 0, None, 4, 0, 2048, 2, None, FAKE, FAKE, None) == UNS
    assert lib.moe_route(FAKE, None, 0, None, 4, 0, 64, 33, None, FAKE, FAKE, None) == UNS
    # missing outputs
    assert lib.moe_route(FAKE, None, 0, None, 4, 0, 8, 2, None, None, FAKE, None) == INV
    # computing logits needs x, w_router and logits_out
    assert lib.moe_route(None, FAKE, moe.MOE_BF16, None, 4, 64, 8, 2, FAKE, FAKE, FAKE,
                         None) == INV
    assert lib.moe_route(None, FAKE, moe.MOE_BF16, FAKE, 4, 64, 8, 2, None, FAKE, FAKE,
                         None) == INV
    assert lib.moe_route(None, FAKE, moe.MOE_FP8_E4M3, FAKE, 4, 64, 8, 2, FAKE, FAKE, FAKE,
                         None) == UNS


def test_permute_validation(lib):
    INV = moe.MOE_ERR_INVALID_ARGUMENT
    ws = lib.moe_permute_workspace_size(16, 2, 8)
    assert ws > 0
    assert lib.moe_permute_workspace_size(16, 9, 8) == 0
    args = [FAKE, 16, 2, 8, FAKE, FAKE, FAKE, FAKE, None, 0, None, 0, None, None]
    assert lib.moe_permute(*args, FAKE, ws - 1, None) == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    assert lib.moe_permute(*args, None, ws, None) == INV
    bad = list(args)
    bad[4] = None  # counts
    assert lib.moe_permute(*bad, FAKE, ws, None) == INV
    # gather needs both x and x_perm; fp8 gather needs scales and d % 128 == 0
    g = list(args)
    g[8] = FAKE
    assert lib.moe_permute(*g, FAKE, ws, None) == INV
    g[9], g[11], g[12] = moe.MOE_FP8_E4M3, 100, FAKE
    assert lib.moe_permute(*g, FAKE, ws, None) == moe.MOE_ERR_UNSUPPORTED
    g[11] = 128
    assert lib.moe_permute(*g, FAKE, ws, None) == INV


def test_quantize_validation(lib):
    UNS, INV = moe.MOE_ERR_UNSUPPORTED, moe.MOE_ERR_INVALID_ARGUMENT
    assert lib.fp8_quantize_act(FAKE, moe.MOE_BF16, 4, 100, 128, None, FAKE, FAKE, None) == UNS
    assert lib.fp8_quantize_act(FAKE, moe.MOE_BF16, 4, 256, 64, None, FAKE, FAKE, None) == UNS
    assert lib.fp8_quantize_act(FAKE, moe.MOE_FP8_E4M3, 4, 256, 128, None, FAKE, FAKE,
                                None) == INV
    assert lib.fp8_quantize_act(None, moe.MOE_BF16, 4, 256, 128, None, FAKE, FAKE, None) == INV
    assert lib.fp8_quantize_act(ctypes.c_void_p(0x1002), moe.MOE_BF16, 4, 256, 128, None, FAKE,
                                FAKE, None) == UNS  # misaligned
    assert lib.fp8_quantize_weight(FAKE, moe.MOE_F32, 2, 128, 200, 128, FAKE, FAKE, None) == UNS
    assert lib.fp8_quantize_weight(FAKE, moe.MOE_F32, 0, 128, 256, 128, FAKE, FAKE, None) == INV
    # the UE8M0 variants validate the same way
    assert lib.fp8_quantize_act_ue8m0(FAKE, moe.MOE_BF16, 4, 100, 128, None, FAKE, FAKE,
                                      None) == UNS
    assert lib.fp8_quantize_act_ue8m0(FAKE, moe.MOE_FP8_E4M3, 4, 256, 128, None, FAKE, FAKE,
                                      None) == INV
    assert lib.fp8_quantize_act_ue8m0(FAKE, moe.MOE_BF16, 4, 256, 128, None, FAKE, None,
                                      None) == INV
    assert lib.fp8_quantize_weight_ue8m0(FAKE, moe.MOE_F32, 2, 128, 200, 128, FAKE, FAKE,
                                         None) == UNS
    assert lib.fp8_quantize_weight_ue8m0(FAKE, moe.MOE_F32, 0, 128, 256, 128, FAKE, FAKE,
                                         None) == INV
    # FP4 with MX scales: K % 32, float input, 16-byte aligned codes
    assert lib.fp4_quantize_weight_mx(FAKE, moe.MOE_F32, 2, 128, 200, FAKE, FAKE, None) == UNS
    assert lib.fp4_quantize_weight_mx(FAKE, moe.MOE_F32, 0, 128, 256, FAKE, FAKE, None) == INV
    assert lib.fp4_quantize_weight_mx(FAKE, moe.MOE_FP8_E4M3, 2, 128, 256, FAKE, FAKE,
                                      None) == INV
    assert lib.fp4_quantize_weight_mx(FAKE, moe.MOE_BF16, 2, 128, 256, ctypes.c_void_p(0x1008), FAKE,
                                      None) == UNS
    assert lib.fp4_quantize_weight_mx(FAKE, moe.MOE_BF16, 2, 128, 256, FAKE, None, None) == INV
    # tiling: N % 16, K % 128, 16-byte alignment, no overlap
    OTHER = ctypes.c_void_p(0x100000)
    assert lib.fp4_tile_weight(FAKE, 2, 24, 256, OTHER, None) == UNS
    assert lib.fp4_tile_weight(FAKE, 2, 32, 192, OTHER, None) == UNS
    assert lib.fp4_tile_weight(FAKE, 2, 32, 256, ctypes.c_void_p(0x100008), None) == UNS
    assert lib.fp4_tile_weight(FAKE, 2, 32, 256, FAKE, None) == INV          # in place
    assert lib.fp4_tile_weight(FAKE, 0, 32, 256, OTHER, None) == INV


def _args(**kw):
    base = dict(T=32, d=256, f=512, E=8, k=2, act_dtype=moe.MOE_BF16, w_dtype=moe.MOE_BF16,
                y_dtype=moe.MOE_BF16, y_layout=moe.MOE_Y_SLOTS, x=0x1000, x_scales=None,
                w_gate=0x1000, w_up=0x1000, w_down=0x1000, s_gate=None, s_up=None, s_down=None,
                offsets=0x1000, sorted_pair=0x1000, topk_w=0x1000, y=0x1000, workspace=0x1000,
                workspace_bytes=1 << 40, scale_fmt=moe.MOE_SCALE_F32, phase=moe.MOE_PHASE_ALL)
    base.update(kw)
    return moe.moe_experts_args(**base)


def _fwd(lib, **kw):
    a = _args(**kw)
    return lib.moe_experts_forward(ctypes.byref(a), None)


def test_experts_validation(lib):
    INV, UNS = moe.MOE_ERR_INVALID_ARGUMENT, moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_experts_forward(None, None) == INV
    assert _fwd(lib, k=9) == INV
    assert _fwd(lib, d=0) == INV
    assert _fwd(lib, x=None) == INV
    assert _fwd(lib, topk_w=None) == INV                      # slots need routing weights
    assert _fwd(lib, y_layout=7) == INV
    assert _fwd(lib, w_dtype=moe.MOE_FP8_E4M3) == UNS          # mixed bf16 act / fp8 weights
    assert _fwd(lib, act_dtype=moe.MOE_F32, w_dtype=moe.MOE_F32) == UNS  # f32 needs f32 y
    assert _fwd(lib, d=200) == UNS                             # bf16 path needs d % 64 == 0
    fp8 = dict(act_dtype=moe.MOE_FP8_E4M3, w_dtype=moe.MOE_FP8_E4M3)
    assert _fwd(lib, d=192, **fp8) == UNS                      # fp8 needs d % 128 == 0
    assert _fwd(lib, **fp8) == INV                             # fp8 needs the scales
    assert _fwd(lib, scale_fmt=moe.MOE_SCALE_UE8M0) == INV     # UE8M0 scales only on fp8
    assert _fwd(lib, scale_fmt=7, **fp8) == INV                # unknown scale format
    fp4 = dict(act_dtype=moe.MOE_FP8_E4M3, w_dtype=moe.MOE_FP4_E2M1, x_scales=0x1000,
               s_gate=0x1000, s_up=0x1000, s_down=0x1000)
    assert _fwd(lib, **fp4) == UNS                             # E2M1 needs UE8M0 scales
    fp4_ue = dict(fp4, scale_fmt=moe.MOE_SCALE_UE8M0)
    assert _fwd(lib, **dict(fp4_ue, s_down=0x1002)) == UNS          # MX scales read as dwords
    assert _fwd(lib, act_dtype=moe.MOE_BF16, w_dtype=moe.MOE_FP4_E2M1) == UNS
    # 16-byte vector loads / LDS DMA of x and weights, vector stores of y; fp32 scales as dwords
    for name in ("x", "w_gate", "w_up", "w_down", "y"):
        assert _fwd(lib, **{name: 0x1008}) == UNS, name
    fp8_s = dict(fp8, x_scales=0x1000, s_gate=0x1000, s_up=0x1000, s_down=0x1000)
    assert _fwd(lib, **dict(fp8_s, s_up=0x1002)) == UNS
    assert _fwd(lib, **dict(fp8_s, x=0x1008)) == UNS
    # the fp32 path takes any alignment: a misaligned x gets as far as the workspace check
    f32 = dict(act_dtype=moe.MOE_F32, w_dtype=moe.MOE_F32, y_dtype=moe.MOE_F32)
    assert _fwd(lib, x=0x1004, workspace_bytes=1, **f32) == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    assert (lib.moe_experts_workspace_size(32, 256, 512, 8, 2, moe.MOE_FP8_E4M3,
                                           moe.MOE_FP4_E2M1) ==
            lib.moe_experts_workspace_size(32, 256, 512, 8, 2, moe.MOE_FP8_E4M3,
                                           moe.MOE_FP8_E4M3))
    need = lib.moe_experts_workspace_size(32, 256, 512, 8, 2, moe.MOE_BF16, moe.MOE_BF16)
    assert need >= 32 * 2 * 512 * 2
    assert _fwd(lib, workspace_bytes=need - 1) == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    assert _fwd(lib, workspace=None) == INV
    assert lib.moe_experts_workspace_size(32, 256, 512, 8, 9, moe.MOE_BF16, moe.MOE_BF16) == 0


def _fz(lib, **kw):
    base = dict(T=32, d=256, f=512, E=8, k=2, x_dtype=moe.MOE_BF16, w_dtype=moe.MOE_BF16,
                scale_fmt=moe.MOE_SCALE_F32, x=0x1000, logits=0x1000, w_router=None,
                logits_out=None, w_gate=0x1000, w_up=0x1000, w_down=0x1000, s_gate=None,
                s_up=None, s_down=None, out=0x1000, out_dtype=moe.MOE_BF16, topk_ids=0x1000,
                topk_w=0x1000, workspace=0x1000, workspace_bytes=1 << 40)
    base.update(kw)
    a = moe.moe_fused_args(**base)
    return lib.moe_fused_forward(ctypes.byref(a), None)


def test_fused_validation(lib):
    INV, UNS = moe.MOE_ERR_INVALID_ARGUMENT, moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_fused_forward(None, None) == INV
    assert _fz(lib, T=129) == UNS                                  # 258 pairs > 256
    assert _fz(lib, d=192) == UNS                                  # d % 128
    assert _fz(lib, out=None) == INV
    assert _fz(lib, topk_ids=None) == INV
    assert _fz(lib, logits=None) == INV                            # neither logits nor router
    assert _fz(lib, x=0x1008) == UNS                               # x alignment
    for name in ("w_gate", "w_up", "w_down"):
        assert _fz(lib, **{name: 0x1008}) == UNS, name
    assert _fz(lib, w_dtype=moe.MOE_F32) == UNS
    assert _fz(lib, x_dtype=moe.MOE_F32) == UNS                    # bf16 experts take bf16 x
    assert _fz(lib, out_dtype=moe.MOE_FP8_E4M3) == INV
    fp8 = dict(w_dtype=moe.MOE_FP8_E4M3, s_gate=0x1000, s_up=0x1000, s_down=0x1000)
    assert _fz(lib, w_dtype=moe.MOE_FP8_E4M3) == INV               # fp8 needs the scales
    assert _fz(lib, w_dtype=moe.MOE_FP4_E2M1, s_gate=0x1000, s_up=0x1000,
               s_down=0x1000) == UNS                               # FP4 needs UE8M0
    assert _fz(lib, scale_fmt=5, **fp8) == INV
    assert _fz(lib, **dict(fp8, s_down=0x1002)) == UNS             # fp32 scales read as dwords
    assert _fz(lib, workspace=None, **fp8) == INV
    need = lib.moe_fused_workspace_size(32, 256, 512, 8, 2, moe.MOE_FP8_E4M3, moe.MOE_BF16)
    assert need > 64 * 512 * 4                                     # at least h in fp32
    assert _fz(lib, workspace_bytes=need - 1, **fp8) == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    assert lib.moe_fused_workspace_size(129, 256, 512, 8, 2, moe.MOE_BF16, moe.MOE_BF16) == 0


def test_combine_validation(lib):
    INV = moe.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_combine(FAKE, moe.MOE_BF16, moe.MOE_Y_PERMUTED, None, FAKE, 4, 2, 64, FAKE,
                           moe.MOE_BF16, None) == INV
    assert lib.moe_combine(FAKE, moe.MOE_BF16, moe.MOE_Y_ACC_F32, None, None, 4, 2, 64, FAKE,
                           moe.MOE_BF16, None) == INV
    assert lib.moe_combine(FAKE, moe.MOE_FP8_E4M3, moe.MOE_Y_SLOTS, None, None, 4, 2, 64, FAKE,
                           moe.MOE_BF16, None) == INV
    assert lib.moe_combine(FAKE, moe.MOE_BF16, 5, None, None, 4, 2, 64, FAKE, moe.MOE_BF16,
                           None) == INV


def test_experts_phase_validation(lib):
    assert _fwd(lib, phase=3) == moe.MOE_ERR_INVALID_ARGUMENT
    assert _fwd(lib, phase=-1) == moe.MOE_ERR_INVALID_ARGUMENT


def test_enum_values_outside_the_declared_ones(lib):
    # any int32 is a value of each enum type (range markers in the header): rejected, never UB
    INV = moe.MOE_ERR_INVALID_ARGUMENT
    lo, hi = -2 ** 31, 2 ** 31 - 1
    for v in (lo, -1, 4, hi):
        assert _fwd(lib, act_dtype=v) in (INV, moe.MOE_ERR_UNSUPPORTED), v
        assert _fwd(lib, w_dtype=v) in (INV, moe.MOE_ERR_UNSUPPORTED), v
        assert _fwd(lib, y_dtype=v) in (INV, moe.MOE_ERR_UNSUPPORTED), v
        assert _fwd(lib, y_layout=v) == INV, v
        assert _fwd(lib, scale_fmt=v) == INV, v
        assert _fwd(lib, phase=v) == INV, v
        assert _fz(lib, out_dtype=v) == INV, v
        assert _fz(lib, scale_fmt=v) == INV, v
        assert lib.moe_combine(FAKE, moe.MOE_BF16, v, None, None, 4, 2, 64, FAKE, moe.MOE_BF16,
                               None) == INV, v
        assert lib.moe_combine(FAKE, v, moe.MOE_Y_SLOTS, None, None, 4, 2, 64, FAKE,
                               moe.MOE_BF16, None) == INV, v
    for v in (lo, -1, 5, hi):
        assert lib.moe_status_string(v) == b"MOE_ERR_UNKNOWN"


def test_fused_noalloc_validation(lib):
    # host-side checks before anything touches a device: the same argument checks as
    # moe_fused_forward, and requests whose workspace exceeds the fixed scratch array
    def fused(**kw):
        base = dict(T=32, d=4096, f=14336, E=8, k=2, x_dtype=moe.MOE_BF16, w_dtype=moe.MOE_BF16,
                    scale_fmt=moe.MOE_SCALE_F32, x=0x1000, logits=None, w_router=0x1000,
                    logits_out=None, w_gate=0x1000, w_up=0x1000, w_down=0x1000, s_gate=None,
                    s_up=None, s_down=None, out=0x1000, out_dtype=moe.MOE_BF16, topk_ids=0x1000,
                    topk_w=0x1000, workspace=None, workspace_bytes=0)
        base.update(kw)
        return lib.moe_fused_forward_noalloc(ctypes.byref(moe.moe_fused_args(**base)), None)
    assert lib.moe_fused_forward_noalloc(None, None) == moe.MOE_ERR_INVALID_ARGUMENT
    assert fused(k=9) == moe.MOE_ERR_INVALID_ARGUMENT
    assert fused(x=None) == moe.MOE_ERR_INVALID_ARGUMENT
    assert fused(T=129) == moe.MOE_ERR_UNSUPPORTED            # more than 256 pairs
    # 256 pairs of a d = f = 32768 bf16 layer with fp32 output need 48 MiB of workspace: beyond
    # the array
    need = lib.moe_fused_workspace_size(128, 32768, 32768, 8, 2, moe.MOE_BF16, moe.MOE_F32)
    assert need > moe.NOALLOC_SCRATCH_BYTES
    assert fused(T=128, d=32768, f=32768, out_dtype=moe.MOE_F32) == moe.MOE_ERR_UNSUPPORTED
    # the Mixtral-shaped decode layer fits at every batch the fused path takes, in every format
    for wdt in (moe.MOE_BF16, moe.MOE_FP8_E4M3, moe.MOE_FP4_E2M1):
        n = lib.moe_fused_workspace_size(128, 4096, 14336, 8, 2, wdt, moe.MOE_BF16)
        assert 0 < n <= moe.NOALLOC_SCRATCH_BYTES, (wdt, n)


def test_small_batch_switch(lib):
    # the switch on mean rows per expert (host logic only)
    sb = lib.moe_experts_small_batch
    BF, F8, F4, F32 = moe.MOE_BF16, moe.MOE_FP8_E4M3, moe.MOE_FP4_E2M1, moe.MOE_F32
    assert sb(32, 4096, 14336, 8, 2, BF, BF) == 1           # Mixtral decode: 8 rows per expert
    assert sb(48, 4096, 14336, 8, 2, BF, BF) == 1           # 12 rows per expert
    assert sb(49, 4096, 14336, 8, 2, BF, BF) == 0
    assert sb(4096, 4096, 14336, 8, 2, BF, BF) == 0         # prefill
    assert sb(40, 192, 320, 8, 2, BF, BF) == 0              # bf16 small-batch needs d, f % 128
    assert sb(512, 7168, 2048, 256, 8, F8, F8) == 1         # 16 rows per expert
    assert sb(513, 7168, 2048, 256, 8, F8, F4) == 0
    assert sb(8192, 7168, 2048, 256, 8, F8, F8) == 0
    assert sb(64, 4096, 14336, 8, 2, F8, F4) == 1
    assert sb(64, 128, 256, 8, 2, F32, F32) == 0
    assert sb(64, 128, 256, 8, 2, BF, F8) == -1
    assert sb(0, 128, 256, 8, 2, BF, BF) == -1
