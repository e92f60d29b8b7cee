"""GPU parity of stage 2 (dispatch): counts, offsets, perm and inv_perm must be bit-exact."""

import numpy as np
import pytest
import torch

from mixture_experts_layer_renorm_amd import abi
from oracle import moe_oracle as O
from tests.moe_testlib import i64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run_dispatch(idx: torch.Tensor, E: int, x=None, D=64, capacity_factor=0.0, min_capacity=0,
                  path="auto"):
    T, K = idx.shape
    p = abi.make_problem(T=T, D=D, E=E, K=K, F=64, capacity_factor=capacity_factor,
                         min_capacity=min_capacity, dispatch_kernel=path)
    r = abi.alloc_routing(p, DEV, logits=False)
    r["topk_idx"] = idx.to(DEV, torch.int32).contiguous()
    x_perm = None
    if x is not None:
        x_perm = torch.full((T * K, D), float("nan"), dtype=x.dtype, device=DEV)
    abi.moe_dispatch(p, x, r, x_perm, abi.alloc_workspace(p, DEV))
    torch.cuda.synchronize()
    return r, x_perm


def _check(idx: torch.Tensor, E: int, path="auto"):
    r, _ = _run_dispatch(idx, E, path=path)
    want = O.dispatch(i64(idx), E)
    n = int(want["offsets"][E])
    np.testing.assert_array_equal(i64(r["expert_counts"]), want["counts"])
    np.testing.assert_array_equal(i64(r["expert_offsets"]), want["offsets"])
    np.testing.assert_array_equal(i64(r["perm"])[:n], want["perm"])
    np.testing.assert_array_equal(i64(r["inv_perm"]), want["inv_perm"])


def _topk_like(T, E, K, gen, hot=None, hot_frac=0.0):
    """Distinct experts per token (a top-K table), optionally concentrated on `hot`."""
    scores = torch.rand((T, E), generator=gen)
    if hot is not None:
        bump = torch.zeros(E)
        bump[hot] = hot_frac
        scores = scores + bump
    return torch.topk(scores, K, dim=1).indices.to(torch.int32)


@pytest.mark.parametrize("T,E,K", [(64, 8, 2), (64, 256, 8), (4096, 256, 8), (8192, 512, 10),
                                   (16384, 256, 6), (1, 1, 1), (3, 5, 5), (1023, 7, 3),
                                   (1025, 1000, 9), (20000, 64, 64)])
def test_dispatch_uniform(T, E, K):
    g = torch.Generator().manual_seed(T + E + K)
    _check(_topk_like(T, E, K, g), E)


def test_dispatch_skewed_and_concentrated():
    g = torch.Generator().manual_seed(5)
    hot = [i * 32 for i in range(8)]
    _check(_topk_like(4096, 256, 8, g, hot, 0.9), 256)   # most assignments on 8 experts
    _check(_topk_like(4096, 256, 8, g, hot, 10.0), 256)  # every token picks the same 8 (U=8)


def test_dispatch_sentinels_skipped():
    g = torch.Generator().manual_seed(6)
    idx = _topk_like(3000, 128, 4, g)
    mask = torch.rand(idx.shape, generator=g) < 0.1
    idx[mask] = -1
    mask2 = torch.rand(idx.shape, generator=g) < 0.05
    idx[mask2] = 128  # the id equal to E is a sentinel too
    _check(idx, 128)


def test_dispatch_row_gather():
    g = torch.Generator().manual_seed(7)
    T, E, K, D = 333, 16, 3, 128
    idx = _topk_like(T, E, K, g)
    x = torch.randn((T, D), generator=g).to(torch.bfloat16).to(DEV)
    r, x_perm = _run_dispatch(idx, E, x=x, D=D)
    perm = i64(r["perm"])
    assert torch.equal(x_perm, x[torch.as_tensor(perm // K, device=DEV)])


def test_dispatch_deterministic():
    g = torch.Generator().manual_seed(8)
    idx = _topk_like(8192, 512, 10, g)
    a, _ = _run_dispatch(idx, 512)
    b, _ = _run_dispatch(idx, 512)
    for k in ("expert_counts", "expert_offsets", "perm", "inv_perm"):
        assert torch.equal(a[k], b[k])


# Both dispatch implementations (one work-group for small batches; count/scan/scatter kernels
# otherwise) forced on the same inputs, inside and outside their default ranges.  The
# multi-kernel path cuts the assignments into segments of 128, 256 or 512 ids by batch size:
# T*K = 32768 (128), 48000 and 65536 (256, the second at the bound of 256 segments), 65544 and
# 1.28 M (512), each with a short last segment where T*K allows one.
@pytest.mark.parametrize("path", ["one_workgroup", "multi"])
@pytest.mark.parametrize("T,E,K", [(1, 1, 1), (64, 256, 8), (1023, 7, 3), (4096, 256, 8),
                                   (2000, 768, 9), (6000, 256, 8), (8192, 320, 8),
                                   (8193, 256, 8), (20000, 64, 64)])
def test_dispatch_both_paths(path, T, E, K):
    g = torch.Generator().manual_seed(100 + T + E + K)
    idx = _topk_like(T, E, K, g)
    if T > 1:
        idx[torch.rand(idx.shape, generator=g) < 0.05] = -1  # sentinels
    _check(idx, E, path)


# Expert capacity: each expert keeps its first C assignments; the rest are dropped.
@pytest.mark.parametrize("path", ["one_workgroup", "multi"])
@pytest.mark.parametrize("T,E,K,cf,minc", [(64, 8, 2, 1.0, 0), (1023, 7, 3, 0.5, 0),
                                           (4096, 256, 8, 1.25, 4), (3000, 128, 4, 1.0, 40),
                                           (20000, 64, 8, 1.1, 0), (50, 16, 4, 0.01, 0)])
def test_dispatch_capacity(path, T, E, K, cf, minc):
    g = torch.Generator().manual_seed(200 + T + E)
    hot = [i * max(1, E // 8) for i in range(min(8, E))]
    idx = _topk_like(T, E, K, g, hot, 0.3)  # skewed, so hot experts overflow
    idx[torch.rand(idx.shape, generator=g) < 0.03] = -1
    r, _ = _run_dispatch(idx, E, capacity_factor=cf, min_capacity=minc, path=path)
    C = O.expert_capacity(T * K, E, float(np.float32(cf)), minc)
    want = O.dispatch(i64(idx), E, C)
    assert want["dropped"] > 0
    n = int(want["offsets"][E])
    np.testing.assert_array_equal(i64(r["expert_counts"]), want["counts"])
    np.testing.assert_array_equal(i64(r["expert_offsets"]), want["offsets"])
    np.testing.assert_array_equal(i64(r["perm"])[:n], want["perm"])
    np.testing.assert_array_equal(i64(r["inv_perm"]), want["inv_perm"])
