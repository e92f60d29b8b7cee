"""Host-side tests of the C ABI that need no GPU: the library loads, exports every function
include/moe.h declares, the ctypes structs match the C layout, and invalid calls fail with
the documented status before anything is launched.
"""

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from mixture_experts_layer_renorm_amd import abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
HEADERS = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    return abi.load_library()


def test_header_declares_the_five_stages_and_helpers():
    names = _declared_functions()
    for n in ("moe_route", "moe_dispatch", "moe_experts", "moe_combine", "moe_forward",
              "moe_route_logits", "moe_workspace_size", "moe_status_string", "moe_last_error"):
        assert n in names
    assert set(names) == set(abi.SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for n in _declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", abi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)", out))
    assert set(_declared_functions()) <= exported


def test_struct_layout_matches_c(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "moe.h"\n'
        "int main(void){printf(\"%zu %zu %zu %zu %zu %zu %zu %zu %zu\\n\", sizeof(moe_problem),"
        " offsetof(moe_problem, flags), offsetof(moe_problem, out_dtype), sizeof(moe_weights),"
        " sizeof(moe_routing), offsetof(moe_routing, shared_gate),"
        " offsetof(moe_problem, gemm_kernel), offsetof(moe_problem, dispatch_kernel),"
        " offsetof(moe_routing, select_keys));return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                    str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    want = [ctypes.sizeof(abi.moe_problem), abi.moe_problem.flags.offset,
            abi.moe_problem.out_dtype.offset, ctypes.sizeof(abi.moe_weights),
            ctypes.sizeof(abi.moe_routing), abi.moe_routing.shared_gate.offset,
            abi.moe_problem.gemm_kernel.offset, abi.moe_problem.dispatch_kernel.offset,
            abi.moe_routing.select_keys.offset]
    assert got == want


def _prob(dtype="f32", **kw):
    base = dict(T=64, D=256, E=8, K=2, F=128)
    base.update(kw)
    import torch
    return abi.make_problem(**base, dtype=torch.float32 if dtype == "f32" else torch.bfloat16)


def _plan(**kw):
    return abi.describe_plan(_prob(**kw))


def test_plan_choices_and_32bit_offset_limits():
    """The plan moe_forward launches, read through moe_describe_plan (no GPU).  The matrix-core
    GEMM addresses operands with 32-bit byte offsets, so a bf16 operand of 4 GiB or more must
    send that GEMM to the 64-bit tile GEMM: the grouped GEMMs when T*K*max(D,F) or one expert's
    weights reach 4 GiB, the shared expert's when x [T,D], Hs [T,F_s] or its weights do."""
    sig = dict(dtype="bf16", T=16384, D=4096, E=256, K=6, F=2048, F_shared=2048)
    text = _plan(**sig)
    assert "grouped gate_up/down: mfma 256x256" in text and "shared: mfma 256x256" in text
    assert "fp16 rows" in text
    # x is [2^19, 4096] bf16 = 4 GiB exactly: both GEMM kinds leave the matrix-core kernel
    big = dict(dtype="bf16", T=1 << 19, D=4096, E=8, K=1, F=256, F_shared=1024)
    text = _plan(**big)
    assert "grouped gate_up/down: tile 256x128" in text, text
    assert "shared: tile 256x128" in text, text
    # one token fewer fits both
    text = _plan(**dict(big, T=(1 << 19) - 1))
    assert "grouped gate_up/down: mfma" in text and "shared: mfma" in text, text
    # shared weights [2 F_s, D] of 4 GiB (F_s = 2^18, D = 4096) with a small batch of tokens that
    # still fills the chip
    text = _plan(dtype="bf16", T=4096, D=4096, E=8, K=1, F=256, F_shared=1 << 18)
    assert "shared: tile 256x128" in text, text
    # fp32 layers never take the matrix-core GEMM; forced tiles are reported
    assert "grouped gate_up/down: tile 32x128" in _plan(T=64)
    assert "grouped gate_up/down: tile 256x128" in _plan(T=64, gemm_kernel="tile256")
    assert "grouped gate_up/down: tile 32x128" in _plan(dtype="bf16", T=64, gemm_kernel="tile32")
    assert "one work-group" in _plan(T=64)
    assert "scan+scatter" in _plan(T=64, dispatch_kernel="multi")
    assert "one work-group" in _plan(T=100000, dispatch_kernel="one_workgroup")


def test_router_plan():
    """Router choice (moe_describe_plan, no GPU): the split-K router for bf16 batches of up to
    1024 tokens; the matrix-core GEMM with the reduction split until about one work-group per
    CU (at most 8 slices of at least 4 stages) for longer bf16 batches of at least 32 output
    tiles, the shared-gate logit
    then computed in the top-K kernel; the tile GEMM when E is not a multiple of 4, when x
    reaches 4 GiB, and for fp32 layers."""
    sig = dict(dtype="bf16", T=16384, D=4096, E=256, K=6, F=2048, F_shared=2048)
    assert "router: mfma 256x256, 4 K slice(s);" in _plan(**sig)      # 64 tiles x 4
    gated = dict(dtype="bf16", T=8192, D=4096, E=512, K=10, F=1024, F_shared=1024,
                 shared_gated=1)
    assert "router: mfma 256x256, 4 K slice(s), gate logit in top-K;" in _plan(**gated)
    # 32 tiles: 8 slices of 4 stages (D = 2048)
    assert "router: mfma 256x256, 8 K slice(s);" in _plan(dtype="bf16", T=8192, D=2048, E=256,
                                                           K=8, F=512)
    # D = 256 has 4 stages: no split
    assert "router: mfma 256x256, 1 K slice(s);" in _plan(dtype="bf16", T=8192, D=256, E=8, K=2,
                                                           F=64)
    # fewer than 32 output tiles (4096 tokens, 256 experts: 16) stay on the tile GEMM
    assert "router: tile 32x128" in _plan(dtype="bf16", T=4096, D=2048, E=256, K=8, F=512)
    assert "router: split-K mfma 16x64" in _plan(dtype="bf16", T=1024, D=4096, E=256, K=6, F=256)
    assert "router: tile" in _plan(dtype="bf16", T=8192, D=256, E=6, K=2, F=64)   # E % 4
    assert "router: tile" in _plan(dtype="bf16", T=1 << 19, D=4096, E=8, K=1, F=256)  # 4 GiB x
    assert "router: tile" in _plan(T=4096)                                          # fp32


def _ws_size(lib, p):
    n = ctypes.c_size_t(0)
    st = lib.moe_workspace_size(ctypes.byref(p), ctypes.byref(n))
    return st, n.value


def test_workspace_size_and_validation(lib):
    st, n = _ws_size(lib, _prob())
    assert st == abi.MOE_OK and n > 0
    assert _ws_size(lib, _prob(K=9))[0] == abi.MOE_ERR_INVALID_ARG      # K > E
    assert _ws_size(lib, _prob(K=0))[0] == abi.MOE_ERR_INVALID_ARG      # K < 1
    assert _ws_size(lib, _prob(T=-1))[0] == abi.MOE_ERR_INVALID_ARG
    assert _ws_size(lib, _prob(D=100))[0] == abi.MOE_ERR_UNSUPPORTED    # D % 64
    assert _ws_size(lib, _prob(F=96))[0] == abi.MOE_ERR_UNSUPPORTED
    assert _ws_size(lib, _prob(E=2000, K=4))[0] == abi.MOE_ERR_UNSUPPORTED
    assert _ws_size(lib, _prob(E=128, K=65))[0] == abi.MOE_ERR_UNSUPPORTED
    p = _prob()
    p.scoring = 7
    assert _ws_size(lib, p)[0] == abi.MOE_ERR_INVALID_ARG
    p = _prob()
    p.flags = 0x80
    assert _ws_size(lib, p)[0] == abi.MOE_ERR_INVALID_ARG
    # capacity: negative or NaN factor, negative floor
    assert _ws_size(lib, _prob(capacity_factor=-1.0))[0] == abi.MOE_ERR_INVALID_ARG
    assert _ws_size(lib, _prob(capacity_factor=float("nan")))[0] == abi.MOE_ERR_INVALID_ARG
    assert _ws_size(lib, _prob(capacity_factor=1.25, min_capacity=-3))[0] == \
        abi.MOE_ERR_INVALID_ARG
    assert _ws_size(lib, _prob(capacity_factor=1.25, min_capacity=4))[0] == abi.MOE_OK
    # kernel-plan fields: unknown values; the matrix-core GEMM forced on an fp32 layer; the
    # one-work-group dispatch forced past its expert limit
    for field in ("gemm_kernel", "dispatch_kernel"):
        for bad in (-1, 9):
            pb = _prob()
            setattr(pb, field, bad)
            assert _ws_size(lib, pb)[0] == abi.MOE_ERR_INVALID_ARG
    assert _ws_size(lib, _prob(gemm_kernel="mfma"))[0] == abi.MOE_ERR_UNSUPPORTED
    assert _ws_size(lib, _prob(E=1000, K=4, dispatch_kernel="one_workgroup"))[0] == \
        abi.MOE_ERR_UNSUPPORTED
    assert _ws_size(lib, _prob(E=768, K=4, dispatch_kernel="one_workgroup"))[0] == abi.MOE_OK
    assert lib.moe_workspace_size(None, None) == abi.MOE_ERR_INVALID_ARG
    assert b"NULL" in lib.moe_last_error()
    # the workspace grows with T; the atomic combine needs no [T*K, D] row buffer
    assert _ws_size(lib, _prob(T=128))[1] > _ws_size(lib, _prob(T=64))[1]
    pa = _prob()
    pa.flags = abi.MOE_FLAG_ATOMIC_COMBINE
    assert _ws_size(lib, pa)[1] < _ws_size(lib, _prob())[1]


def test_peak_probes_validate_before_launch(lib):
    assert lib.moe_peak_hbm_read(None, 65536, ALIGNED, None) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_peak_hbm_read(ALIGNED, 65536 + 16, ALIGNED, None) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_peak_hbm_read(ALIGNED + 4, 65536, ALIGNED, None) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_peak_hbm_read(ALIGNED, 0, ALIGNED, None) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_peak_mfma_bf16(6, 10, ALIGNED, None) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_peak_mfma_bf16(0, 10, ALIGNED, None) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_peak_mfma_bf16(8, 10, None, None) == abi.MOE_ERR_INVALID_ARG


def test_status_strings(lib):
    for code, name in [(0, b"MOE_OK"), (-1, b"MOE_ERR_INVALID_ARG"), (-2, b"MOE_ERR_UNSUPPORTED"),
                       (-3, b"MOE_ERR_WORKSPACE"), (-4, b"MOE_ERR_HIP")]:
        assert lib.moe_status_string(code) == name


# Fake device addresses: never dereferenced, because validation rejects the call first.
ALIGNED = 0x7F0000000000
MISALIGNED = ALIGNED + 4


def _weights(**kw):
    w = abi.moe_weights()
    for n in ("w_router", "w_gate_up", "w_down"):
        setattr(w, n, ALIGNED)
    for k, v in kw.items():
        setattr(w, k, v)
    return w


def test_invalid_calls_fail_before_launch(lib):
    p = _prob()
    st, need = _ws_size(lib, p)
    w = _weights()
    r = abi.moe_routing()
    out = ALIGNED
    # NULL x / out
    assert lib.moe_forward(ctypes.byref(p), None, ctypes.byref(w), None, out, ALIGNED, need,
                           None) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_forward(ctypes.byref(p), ALIGNED + 4096, ctypes.byref(w), None, None, ALIGNED,
                           need, None) == abi.MOE_ERR_INVALID_ARG
    # misaligned weight
    wm = _weights(w_down=MISALIGNED)
    assert lib.moe_forward(ctypes.byref(p), ALIGNED + 4096, ctypes.byref(wm), None, out, ALIGNED,
                           need, None) == abi.MOE_ERR_INVALID_ARG
    assert b"w_down" in lib.moe_last_error()
    # workspace too small / missing
    assert lib.moe_forward(ctypes.byref(p), ALIGNED + 4096, ctypes.byref(w), None, out, ALIGNED,
                           need - 1, None) == abi.MOE_ERR_WORKSPACE
    assert lib.moe_forward(ctypes.byref(p), ALIGNED + 4096, ctypes.byref(w), None, out, None,
                           need, None) == abi.MOE_ERR_WORKSPACE
    # out aliasing x
    assert lib.moe_forward(ctypes.byref(p), out, ctypes.byref(w), None, out, ALIGNED, need,
                           None) == abi.MOE_ERR_INVALID_ARG
    # shared expert declared but its weights missing
    ps = _prob(F_shared=64)
    ps.shared_gated = 1
    _, need_s = _ws_size(lib, ps)
    assert lib.moe_forward(ctypes.byref(ps), ALIGNED + 4096, ctypes.byref(w), None, out, ALIGNED,
                           need_s, None) == abi.MOE_ERR_INVALID_ARG
    # route: required outputs missing; K > E
    assert lib.moe_route(ctypes.byref(p), ALIGNED, ctypes.byref(w), ctypes.byref(r), ALIGNED,
                         need, None) == abi.MOE_ERR_INVALID_ARG
    pk = _prob(K=9)
    r2 = abi.moe_routing(topk_idx=ALIGNED, topk_w=ALIGNED)
    assert lib.moe_route_logits(ctypes.byref(pk), ALIGNED, None, ctypes.byref(r2),
                                None) == abi.MOE_ERR_INVALID_ARG
    # unaligned select_bias; bias update without counts / with an unaligned bias
    r3 = abi.moe_routing(topk_idx=ALIGNED, topk_w=ALIGNED)
    assert lib.moe_route_logits(ctypes.byref(p), ALIGNED, ALIGNED + 4, ctypes.byref(r3),
                                None) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_update_select_bias(ctypes.byref(p), None, ALIGNED, 0.01,
                                      None) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_update_select_bias(ctypes.byref(p), ALIGNED, ALIGNED + 4, 0.01,
                                      None) == abi.MOE_ERR_INVALID_ARG
    # router statistics: missing inputs / output, workspace too small
    assert lib.moe_router_stats(ctypes.byref(p), None, ALIGNED, ALIGNED, ALIGNED, need,
                                None) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_router_stats(ctypes.byref(p), ALIGNED, ALIGNED, None, ALIGNED, need,
                                None) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_router_stats(ctypes.byref(p), ALIGNED, ALIGNED, ALIGNED, ALIGNED, need - 1,
                                None) == abi.MOE_ERR_WORKSPACE
    # dispatch / experts / combine: missing routing tensors
    assert lib.moe_dispatch(ctypes.byref(p), None, ctypes.byref(r), None, ALIGNED, need,
                            None) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_experts(ctypes.byref(p), ALIGNED, None, ctypes.byref(w), ctypes.byref(r),
                           ALIGNED, None, ALIGNED, need, None) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(ctypes.byref(p), ALIGNED, ctypes.byref(r), None, ALIGNED,
                           None) == abi.MOE_ERR_INVALID_ARG


def test_noalloc_rejects_before_touching_the_device(lib):
    """moe_forward_noalloc validates the problem and its workspace need against the fixed
    scratch size before it looks up any device."""
    import torch
    w = _weights()
    out = ALIGNED
    big = abi.make_problem(T=4096, D=2048, E=256, K=8, F=512, dtype=torch.bfloat16)
    st, need = _ws_size(lib, big)
    assert st == abi.MOE_OK and need > abi.MOE_NOALLOC_SCRATCH_BYTES
    assert lib.moe_forward_noalloc(ctypes.byref(big), ALIGNED + 4096, ctypes.byref(w), None, out,
                                   None) == abi.MOE_ERR_WORKSPACE
    assert b"scratch" in lib.moe_last_error()
    small = abi.make_problem(T=64, D=2048, E=256, K=8, F=512, dtype=torch.bfloat16)
    assert _ws_size(lib, small)[1] <= abi.MOE_NOALLOC_SCRATCH_BYTES
    assert lib.moe_forward_noalloc(ctypes.byref(_prob(K=9)), ALIGNED, ctypes.byref(w), None, out,
                                   None) == abi.MOE_ERR_INVALID_ARG
    assert lib.moe_forward_noalloc(ctypes.byref(_prob(T=0)), None, None, None, None,
                                   None) == abi.MOE_OK


def test_empty_batch_returns_ok_without_touching_pointers(lib):
    p = _prob(T=0)
    w = abi.moe_weights()
    assert lib.moe_forward(ctypes.byref(p), None, ctypes.byref(w), None, None, None, 0,
                           None) == abi.MOE_OK
    assert lib.moe_route(ctypes.byref(p), None, None, None, None, 0, None) == abi.MOE_OK
    assert lib.moe_combine(ctypes.byref(p), None, None, None, None, None) == abi.MOE_OK


def test_binding_refuses_host_tensors():
    import torch
    p = _prob()
    with pytest.raises(ValueError):
        abi._ptr(torch.zeros(4), "x")
    with pytest.raises(RuntimeError):
        abi.load_library(os.path.join(tempfile.gettempdir(), "does-not-exist", "libmoe.so"))
