"""GPU parity of moe_permute: counts, offsets, sorted_ids and inv bit-exact
against the oracle; the gathered rows a bitwise copy of x."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
import mixture_experts_router_amd as moe
from mixture_experts_router_amd import device as dev
from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _permute(gpu, ids_np, E, H=0, x_np=None):
    T, k = ids_np.shape
    s = moe.shape(T, max(H, 64), E, k, 64)
    ids = torch.from_numpy(ids_np.astype(np.int32)).cuda()
    A = T * k
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sorted_ids = torch.empty(A, dtype=torch.int32, device="cuda")
    inv = torch.empty(A, dtype=torch.int32, device="cuda")
    ws = torch.empty(moe.permute_workspace_bytes(s), dtype=torch.uint8, device="cuda")
    x = xp = None
    if x_np is not None:
        x = dev.to_device(x_np)
        xp = torch.empty((A, H), dtype=torch.bfloat16, device="cuda")
    gpu.permute(s, ids, x, counts, offsets, sorted_ids, inv, xp, ws)
    torch.cuda.synchronize()
    res = [t.cpu().numpy() for t in (counts, offsets, sorted_ids, inv)]
    if xp is not None:
        res.append(dev.bf16_bits(xp))
    return res


def _check(gpu, ids, E, label, H=0):
    T, k = ids.shape
    say(f"permute {label}: T={T} k={k} E={E} A={T * k}")
    x = mi.random_bf16((T, H), seed=T) if H else None
    got = _permute(gpu, ids, E, H, x)
    c, o = oracle.counts_offsets(ids, E)
    si, inv = oracle.permutation(ids)
    assert (got[0] == c).all(), f"{label}: counts"
    assert (got[1] == o).all(), f"{label}: offsets"
    assert (got[2] == si).all(), f"{label}: sorted_ids"
    assert (got[3] == inv).all(), f"{label}: inv"
    if H:
        assert (got[4] == x[si // k]).all(), f"{label}: gathered rows"
        back = got[4][inv].reshape(T, k, H)
        assert (back == x[:, None, :]).all()


# (8192, 128, 8): 64 chunks of 1024 assignments, the most the scan runs
# inside the scatter blocks; (8193, 128, 8): 65 chunks, a scan launch of its own
@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (8, 128, 8), (16, 8, 2), (128, 128, 8),
                                   (129, 128, 8), (300, 16, 4), (2048, 128, 8), (777, 1000, 3),
                                   (8192, 128, 8), (8193, 128, 8), (5000, 1024, 32)])
def test_uniform_routing(gpu, T, E, k):
    _check(gpu, mi.random_ids(T, E, k, seed=T + E), E, "uniform")


def test_zipf_skew_full_size(gpu):
    p = np.exp(mi.zipf_log_prior(128, 1.2).astype(np.float64))
    ids = mi.random_ids(8192, 128, 8, seed=3, p=p / p.sum())
    _check(gpu, ids, 128, "zipf")


def test_hot_expert_and_empty_experts(gpu):
    T, k, E = 3000, 2, 64
    ids = np.zeros((T, k), dtype=np.int32)
    ids[:, 1] = 63                           # experts 1..62 empty
    _check(gpu, ids, E, "two hot experts")
    ids = np.stack([np.full(700, 5), np.arange(700) % 3], axis=1).astype(np.int32)
    _check(gpu, ids, 6, "one expert owns every token")


def test_gathered_rows(gpu):
    _check(gpu, mi.random_ids(50, 16, 4, seed=1), 16, "small + rows", H=128)
    _check(gpu, mi.random_ids(700, 128, 8, seed=2), 128, "multi-block + rows", H=2816)
