"""moe_permute_noalloc (the allocation-free permute, on the library's static
scratch) against moe_permute with a caller's workspace, through the C ABI:
two calls in a row on one device, the second with a smaller input, every
output bit for bit.  The routing of each call is the oracle's selection on
seeded random probabilities (top-K, and Expert Race with up to E slots per
token)."""
import numpy as np
import pytest
import torch

import oracle
from parity import to_np

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _routing(N, E, K, race, seed):
    rng = np.random.default_rng(seed)
    P = oracle.softmax(rng.standard_normal((N, E)))
    if race:
        return oracle.race_select(P, K)[0]
    return oracle.topk_select(P, K)[0]


def _outputs(N, E, Kmax, D, copy):
    i32, i64 = torch.int32, torch.int64
    return dict(counts=torch.full((E,), -7, dtype=i32, device=DEV),
                offs=torch.full((E + 1,), -7, dtype=i64, device=DEV),
                rt=torch.full((max(N * Kmax, 1),), -7, dtype=i32, device=DEV),
                sr=torch.full((N, Kmax), -7, dtype=i32, device=DEV),
                xp=(torch.full((N * Kmax, D), 7.0, dtype=torch.bfloat16,
                               device=DEV) if copy else None))


def _compare(N, D, E, K, race, copy, seed):
    from sparse_moe_diffusion_amd import ops
    idx = _routing(N, E, K, race, seed)
    Kmax = idx.shape[1]
    A = K * N
    print(f"[noalloc] N={N} D={D} E={E} K={K} Kmax={Kmax} copy={copy}",
          flush=True)
    x = torch.from_numpy(np.random.default_rng(seed + 1).standard_normal(
        (N, D)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    tidx = torch.from_numpy(idx.astype(np.int32)).to(DEV)
    ref = _outputs(N, E, Kmax, D, copy)
    got = _outputs(N, E, Kmax, D, copy)
    ws = torch.empty(max(ops.permute_workspace_size(N, E, Kmax), 1),
                     dtype=torch.uint8, device=DEV)
    ops.moe_permute(x, tidx, E, K, ref["counts"], ref["offs"], ref["rt"],
                    ref["sr"], ref["xp"], ws)
    ops.moe_permute_noalloc(x, tidx, E, K, got["counts"], got["offs"],
                            got["rt"], got["sr"], got["xp"])
    torch.cuda.synchronize()
    for k in ("counts", "offs", "sr"):
        assert torch.equal(got[k], ref[k]), k
    assert torch.equal(got["rt"][:A], ref["rt"][:A])
    if copy:
        assert torch.equal(got["xp"][:A].view(torch.int16),
                           ref["xp"][:A].view(torch.int16))
    # and the oracle's permutation of the same routing
    counts, offsets, row_token, slot_row = oracle.permute(idx, E)
    assert np.array_equal(to_np(got["counts"]), counts)
    assert np.array_equal(to_np(got["offs"]), offsets)
    assert np.array_equal(to_np(got["rt"])[:A], row_token)
    assert np.array_equal(to_np(got["sr"]), slot_row)


def test_permute_noalloc_two_calls():
    # a large top-K routing with the row copy, then a smaller race routing
    # (E = 16 slots per token) without it: the second call reuses the
    # scratch the first left behind
    _compare(40000, 256, 8, 2, False, True, 1)
    _compare(3001, 128, 16, 2, True, False, 2)


def test_permute_noalloc_near_limit():
    # the largest top-K shape of the configured layers' kind near the
    # scratch's limit (workspace just under 1 MiB at E = 64), then a tiny one
    _compare(340000, 64, 64, 2, False, False, 3)
    _compare(5, 64, 64, 2, False, True, 4)
