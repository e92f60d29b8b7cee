"""moe_forward_noalloc (the entry point for callers that cannot allocate) against moe_forward
with a caller workspace: two calls in a row on one GPU, the second with a smaller batch, each
bit-identical to the workspace path (same kernels, deterministic combine) in its output and
every routing table, and so within the layer's tolerance of the oracle as moe_forward is."""

import numpy as np
import pytest
import torch

from mixture_experts_layer_renorm_amd import abi
from mixture_experts_layer_renorm_amd.synth import CONFIGS, make_layer
from oracle import moe_oracle as O
from tests.moe_testlib import TOL_BF16, f64, oracle_args, problem_for, rel_max_err, weights_for

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(cfg, layer, T):
    p = problem_for(cfg, T=T, out_dtype=torch.float32)
    assert abi.moe_workspace_size(p) <= abi.MOE_NOALLOC_SCRATCH_BYTES
    x = layer["x"][:T].contiguous()
    w = weights_for(layer)
    r_ws, r_na = abi.alloc_routing(p, DEV), abi.alloc_routing(p, DEV)
    out_ws = torch.empty((T, cfg.D), dtype=torch.float32, device=DEV)
    out_na = torch.full((T, cfg.D), float("nan"), dtype=torch.float32, device=DEV)
    abi.moe_forward(p, x, w, r_ws, out_ws, abi.alloc_workspace(p, DEV))
    abi.moe_forward_noalloc(p, x, w, r_na, out_na)
    torch.cuda.synchronize()
    return p, x, r_ws, r_na, out_ws, out_na


@pytest.mark.parametrize("name", ["a3b_decode", "ds_sigmoid"])
def test_noalloc_matches_workspace_path_twice(name):
    cfg = CONFIGS[name]
    if name == "ds_sigmoid":
        cfg = cfg.with_(E=32)  # keeps the shared expert and the sigmoid router, fits the scratch
    layer = make_layer(cfg, device=DEV, T=64)
    for T in (64, 23):  # the second call is smaller and finds the first call's contents
        p, x, r_ws, r_na, out_ws, out_na = _both(cfg, layer, T)
        assert torch.equal(out_na, out_ws), f"{name} T={T}: outputs differ"
        for k in ("logits", "topk_idx", "topk_w", "expert_counts", "expert_offsets", "perm",
                  "inv_perm"):
            n = int(r_ws["expert_offsets"][-1]) if k == "perm" else None
            a, b = r_ws[k], r_na[k]
            if n is not None:
                a, b = a[:n], b[:n]
            assert torch.equal(a, b), f"{name} T={T}: {k} differs"
        args, kw = oracle_args(cfg, {**layer, "x": x})
        ref = O.moe_forward(*args, logits=f64(r_na["logits"]), **kw)
        np.testing.assert_array_equal(r_na["topk_idx"].cpu().numpy(), ref["topk_idx"])
        assert rel_max_err(out_na, ref["out"]) <= TOL_BF16


def test_noalloc_rejects_a_batch_beyond_its_scratch():
    cfg = CONFIGS["a3b_prefill"]
    p = problem_for(cfg, T=cfg.T)
    assert abi.moe_workspace_size(p) > abi.MOE_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((1, cfg.D), dtype=cfg.torch_dtype, device=DEV)  # never read
    out = torch.zeros((1, cfg.D), dtype=cfg.torch_dtype, device=DEV)
    w = {"w_router": x, "w_gate_up": x, "w_down": x}
    with pytest.raises(abi.MoEError) as ei:
        abi.moe_forward_noalloc(p, x, w, None, out)
    assert ei.value.status == abi.MOE_ERR_WORKSPACE
