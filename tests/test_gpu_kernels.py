"""Per-call parity of the C ABI entry points against the CPU oracle, on
edge shapes: empty and single-token inputs, ragged tails, empty expert
groups, K = E, E = 1 and E = 64, ties, biases, both dtypes."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import (TOL, assert_close, chunks, near_topk, pmap,
                    reconcile_race, reconcile_topk, to_np)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _bits_tensor(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.to(DEV)


def _ops():
    from sparse_moe_diffusion_amd import _lib, ops
    return _lib, ops


def _run_gate(x32, wg, bias, K, route, dtype):
    _lib, ops = _ops()
    N, D = x32.shape
    E = wg.shape[0]
    Kmax = E if route == "race" else K
    x = _bits_tensor(x32, dtype)
    wgt = torch.from_numpy(wg).to(DEV)
    bt = None if bias is None else torch.from_numpy(bias).to(DEV)
    probs = torch.empty(N, E, dtype=torch.float32, device=DEV)
    idx = torch.empty(N, Kmax, dtype=torch.int32, device=DEV)
    w = torch.empty(N, Kmax, dtype=torch.float32, device=DEV)
    rc = _lib.MOE_ROUTE_EXPERT_RACE if route == "race" else _lib.MOE_ROUTE_TOPK
    ws = torch.empty(max(ops.gate_workspace_size(N, E, K, rc), 1),
                     dtype=torch.uint8, device=DEV)
    ops.moe_gate_topk(x, wgt, bt, K, rc, probs, idx, w, ws)
    torch.cuda.synchronize()
    return to_np(probs), to_np(idx), to_np(w)


GATE_CASES = [  # N, D, E, K, bias, dtype
    (1, 8, 1, 1, False, "bf16"), (63, 128, 8, 2, False, "bf16"),
    (64, 128, 8, 2, True, "bf16"), (65, 1152, 8, 2, False, "bf16"),
    (1000, 384, 16, 2, True, "bf16"), (300, 2048, 16, 2, False, "bf16"),
    (257, 72, 3, 3, True, "f32"), (200, 136, 33, 5, True, "bf16"),
    (130, 64, 64, 7, False, "f32"), (500, 384, 8, 1, False, "f32"),
    # bf16, E <= 16 with unused expert columns and a partial last 32-wide
    # feature slice; N leaves part of the last workgroup empty
    (777, 72, 12, 3, True, "bf16"), (129, 200, 5, 2, False, "bf16"),
    # split gate weights past the LDS budget, streamed in phases: two phases
    # of 96 + 4 slices (E <= 8), three of 48 slices (E <= 16)
    (200, 3200, 8, 2, True, "bf16"), (130, 4608, 12, 3, False, "bf16"),
]


@pytest.mark.parametrize("N,D,E,K,bias,dtype", GATE_CASES)
def test_gate_topk(N, D, E, K, bias, dtype):
    rng = np.random.default_rng(N * 31 + D + E)
    x = synth.bf16_to_f32(synth.bf16_bits(rng.standard_normal((N, D)).astype(np.float32)))
    if dtype == "f32":
        x = rng.standard_normal((N, D)).astype(np.float32)
    wg = (rng.standard_normal((E, D)) * 0.05).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32) if bias else None
    probs, idx, w = _run_gate(x, wg, b, K, "topk", dtype)
    P = oracle.softmax(oracle.gate_logits(x, wg, b))
    assert np.abs(probs - P).max() <= 1e-6
    idx_o, _ = oracle.topk_select(P, K)
    rec, bad, near = reconcile_topk(P, idx_o, idx)
    assert not bad
    assert np.array_equal(idx, rec)
    assert np.abs(w - oracle.slot_weights(P, idx)).max() <= 1e-6


def test_gate_zero_weights_ties():
    """Zero gate: probabilities exactly 1/E, ties resolved to low indices."""
    N, D, E, K = 100, 64, 8, 3
    x = np.random.default_rng(0).standard_normal((N, D)).astype(np.float32)
    probs, idx, w = _run_gate(x, np.zeros((E, D), np.float32), None, K, "topk",
                              "f32")
    assert np.all(probs == np.float32(1.0 / E))
    assert np.all(idx == np.arange(K)) and np.all(w == np.float32(1.0 / E))


def test_gate_empty():
    probs, idx, w = _run_gate(np.zeros((0, 64), np.float32),
                              np.ones((8, 64), np.float32), None, 2, "topk",
                              "bf16")
    assert probs.shape == (0, 8)


@pytest.mark.parametrize("N,D,E,K", [(10, 64, 4, 2), (333, 128, 16, 2),
                                     (64, 72, 5, 3), (1, 64, 8, 8),
                                     (2048, 256, 16, 2), (97, 64, 64, 5)])
def test_race_select(N, D, E, K):
    rng = np.random.default_rng(N + E)
    x = rng.standard_normal((N, D)).astype(np.float32)
    wg = (rng.standard_normal((E, D)) * 0.1).astype(np.float32)
    probs, idx, w = _run_gate(x, wg, None, K, "race", "f32")
    P = oracle.softmax(oracle.gate_logits(x, wg))
    idx_o, tau, near = oracle.race_select(P, K)
    rec, bad = reconcile_race(P, K, idx_o, idx, tau)
    assert not bad
    assert np.array_equal(idx, rec)
    assert int((idx >= 0).sum()) == K * N
    assert np.all(w[idx < 0] == 0)


@pytest.mark.parametrize("N,D,E,K", [(333, 128, 16, 2), (1000, 200, 8, 2)])
def test_race_select_bf16(N, D, E, K):
    """Race on bf16 tokens (probabilities from the bf16 gate path)."""
    rng = np.random.default_rng(N + 7 * E)
    x = synth.bf16_to_f32(synth.bf16_bits(rng.standard_normal((N, D)).astype(np.float32)))
    wg = (rng.standard_normal((E, D)) * 0.1).astype(np.float32)
    probs, idx, w = _run_gate(x, wg, None, K, "race", "bf16")
    P = oracle.softmax(oracle.gate_logits(x, wg))
    assert np.abs(probs - P).max() <= 1e-6
    idx_o, tau, near = oracle.race_select(P, K)
    rec, bad = reconcile_race(P, K, idx_o, idx, tau)
    assert not bad
    assert np.array_equal(idx, rec)
    assert int((idx >= 0).sum()) == K * N


def test_race_all_ties():
    """Zero gate: every score is exactly 1/E; the first K*N flat entries
    win, so the first K*N/E tokens take every expert."""
    N, D, E, K = 40, 64, 4, 2
    x = np.random.default_rng(1).standard_normal((N, D)).astype(np.float32)
    probs, idx, w = _run_gate(x, np.zeros((E, D), np.float32), None, K, "race",
                              "f32")
    full = K * N // E
    assert np.all(idx[:full] == np.arange(E))
    assert np.all(idx[full:] == -1)


def test_race_identical_tokens_equals_topk():
    N, D, E, K = 256, 64, 16, 2
    rng = np.random.default_rng(2)
    x = np.tile(rng.standard_normal((1, D)).astype(np.float32), (N, 1))
    wg = (rng.standard_normal((E, D)) * 0.3).astype(np.float32)
    _, idx_r, _ = _run_gate(x, wg, None, K, "race", "f32")
    _, idx_k, _ = _run_gate(x, wg, None, K, "topk", "f32")
    assert np.array_equal(idx_r[:, :K], np.sort(idx_k, axis=1))
    assert np.all(idx_r[:, K:] == -1)


def _run_permute(x32, idx, E, K, dtype, with_copy=True):
    _lib, ops = _ops()
    N, D = x32.shape
    Kmax = idx.shape[1]
    A = K * N
    x = _bits_tensor(x32, dtype)
    it = torch.from_numpy(idx.astype(np.int32)).to(DEV)
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    offs = torch.empty(E + 1, dtype=torch.int64, device=DEV)
    rt = torch.full((max(A, 1),), -7, dtype=torch.int32, device=DEV)
    sr = torch.empty(N, Kmax, dtype=torch.int32, device=DEV)
    xp = torch.empty(A, D, dtype=x.dtype, device=DEV) if with_copy else None
    ws = torch.empty(ops.permute_workspace_size(N, E, Kmax), dtype=torch.uint8,
                     device=DEV)
    ops.moe_permute(x, it, E, K, counts, offs, rt, sr, xp, ws)
    torch.cuda.synchronize()
    return (to_np(counts), to_np(offs), to_np(rt)[:A], to_np(sr),
            None if xp is None else to_np(xp))


@pytest.mark.parametrize("N,D,E,Kmax,K,dtype", [
    (1, 64, 8, 2, 2, "bf16"), (255, 128, 8, 2, 2, "bf16"),
    (257, 1152, 8, 2, 2, "bf16"), (1000, 64, 16, 16, 2, "bf16"),
    (513, 72, 5, 3, 3, "f32"), (300, 64, 64, 64, 4, "bf16"),
    (4096, 256, 8, 1, 1, "bf16"), (700, 128, 1, 1, 1, "f32")])
def test_permute(N, D, E, Kmax, K, dtype):
    rng = np.random.default_rng(N + 7 * E)
    if Kmax == K:  # top-K form: K distinct experts per token, some skewed
        p = rng.dirichlet(np.ones(E) * 0.3)
        idx = np.stack([rng.choice(E, size=K, replace=False, p=p) for _ in range(N)])
    else:  # race form: exactly K*N kept slots, 0..E per token
        keep = np.zeros(N * E, bool)
        keep[rng.choice(N * E, size=K * N, replace=False)] = True
        keep = keep.reshape(N, E)
        idx = np.full((N, E), -1)
        for t in range(N):
            sel = np.nonzero(keep[t])[0]
            idx[t, :sel.size] = sel
    x = rng.standard_normal((N, D)).astype(np.float32)
    if dtype == "bf16":
        x = synth.bf16_to_f32(synth.bf16_bits(x))
    counts, offs, rt, sr, xp = _run_permute(x, idx, E, K, dtype)
    c_o, o_o, rt_o, sr_o = oracle.permute(idx.astype(np.int32), E)
    assert np.array_equal(counts, c_o)
    assert np.array_equal(offs, o_o)
    assert np.array_equal(rt, rt_o)
    assert np.array_equal(sr, sr_o)
    assert np.array_equal(xp, x[rt_o])  # bitwise row copies
    # index-only mode writes the same indices
    c2, o2, rt2, sr2, _ = _run_permute(x, idx, E, K, dtype, with_copy=False)
    assert np.array_equal(rt2, rt_o) and np.array_equal(sr2, sr_o)


@pytest.mark.parametrize("E,Kmax,K", [(8, 2, 2), (16, 16, 2)])
def test_permute_out_of_range_slots_are_empty(E, Kmax, K):
    """Slot contents outside [-1, E) are treated as empty (the header's
    contract): the result is the oracle's on those slots set to -1, and the
    routed rows past the valid selections are not written."""
    rng = np.random.default_rng(E + Kmax)
    N, D = 700, 64
    if Kmax == K:
        idx = np.stack([rng.choice(E, size=K, replace=False) for _ in range(N)])
    else:
        idx = np.full((N, E), -1)
        for t in range(N):
            sel = np.sort(rng.choice(E, size=K, replace=False))
            idx[t, :K] = sel
    bad = rng.random(idx.shape) < 0.15
    junk = rng.choice([E, E + 3, 1 << 20, -2, -9], size=idx.shape)
    idx_in = np.where(bad & (idx >= 0), junk, idx)
    clean = np.where((idx_in >= 0) & (idx_in < E), idx_in, -1)
    x = synth.bf16_to_f32(synth.bf16_bits(rng.standard_normal((N, D)).astype(np.float32)))
    counts, offs, rt, sr, xp = _run_permute(x, idx_in, E, K, "bf16")
    c_o, o_o, rt_o, sr_o = oracle.permute(clean.astype(np.int32), E)
    n = int(o_o[-1])
    assert n < K * N
    assert np.array_equal(counts, c_o) and np.array_equal(offs, o_o)
    assert np.array_equal(sr, sr_o)
    assert np.array_equal(rt[:n], rt_o) and np.all(rt[n:] == -7)
    assert np.array_equal(xp[:n], x[rt_o])


def _run_ffn(xs, offsets, w1, w2, b1, b2, dtype, row_index=None, y_f32=False):
    _, ops = _ops()
    G, H, D = w1.shape
    total = int(offsets[-1])
    x = _bits_tensor(xs, dtype)
    ri = None if row_index is None else torch.from_numpy(
        row_index.astype(np.int32)).to(DEV)
    ot = torch.from_numpy(offsets.astype(np.int64)).to(DEV)
    w1t, w2t = _bits_tensor(w1, dtype), _bits_tensor(w2, dtype)
    b1t = None if b1 is None else torch.from_numpy(b1).to(DEV)
    b2t = None if b2 is None else torch.from_numpy(b2).to(DEV)
    h = torch.empty(total, H, dtype=x.dtype, device=DEV)
    ydt = torch.float32 if (y_f32 or dtype == "f32") else torch.bfloat16
    y = torch.full((total, D), float("nan"), dtype=ydt, device=DEV)
    ops.moe_grouped_ffn(x, ri, total, ot, w1t, b1t, w2t, b2t, h, y)
    torch.cuda.synchronize()
    return to_np(y)


@pytest.mark.parametrize("sizes,D,H,dtype,gather,bias", [
    ([100, 0, 129, 1, 256, 0, 0, 300], 128, 256, "bf16", False, False),
    ([100, 0, 129, 1, 256, 0, 0, 300], 128, 256, "bf16", True, True),
    ([0, 0, 0], 64, 128, "bf16", False, False),
    ([513], 136, 264, "bf16", False, True),
    ([77, 3, 200], 1152, 4608, "bf16", True, False),
    ([31, 64, 0, 97], 72, 136, "f32", True, True),
    ([128, 128], 256, 512, "f32", False, False),
    # many ragged groups, some empty: the device-side tile scheduler walks 64
    # and 128 (the maximum) groups
    ([(i * 37) % 23 * 3 for i in range(64)], 128, 256, "bf16", True, False),
    ([(i * 11) % 7 for i in range(128)], 64, 128, "bf16", False, True),
    # more tiles than workgroups: every persistent workgroup takes several
    ([5000, 0, 5240], 64, 2048, "bf16", True, False),
])
def test_grouped_ffn(sizes, D, H, dtype, gather, bias):
    rng = np.random.default_rng(sum(sizes) + D)
    G = len(sizes)
    offsets = np.concatenate([[0], np.cumsum(sizes)])
    total = int(offsets[-1])
    rnd = lambda *s: (rng.standard_normal(s) * 0.05).astype(np.float32)
    q = (lambda a: synth.bf16_to_f32(synth.bf16_bits(a))) if dtype == "bf16" else (lambda a: a)
    nsrc = total + 13
    xsrc = q(rng.standard_normal((nsrc, D)).astype(np.float32))
    w1, w2 = q(rnd(G, H, D)), q(rnd(G, D, H))
    b1 = rnd(G, H) if bias else None
    b2 = rnd(G, D) if bias else None
    ri = rng.permutation(nsrc)[:total] if gather else None
    y = _run_ffn(xsrc if gather else xsrc[:total], offsets, w1, w2, b1, b2, dtype,
                 row_index=ri)
    if total == 0:
        return
    rows = xsrc[ri] if gather else xsrc[:total]
    ref = np.zeros((total, D))
    for g in range(G):
        a, b = offsets[g], offsets[g + 1]
        if b > a:
            ref[a:b] = oracle.expert_mlp(rows[a:b], w1[g], w2[g],
                                         None if b1 is None else b1[g],
                                         None if b2 is None else b2[g])
    assert_close(y, ref, dtype, "grouped ffn")


def _grouped_reference(xrows, offsets, w1, w2, b1=None, b2=None):
    """oracle.expert_mlp on every row of every group, the oracle's calls on
    chunks of 1024 rows run side by side."""
    jobs = []
    for g in range(len(offsets) - 1):
        a, b = int(offsets[g]), int(offsets[g + 1])
        jobs += [(g, c) for c in chunks(np.arange(a, b))]
    ref = np.zeros((xrows.shape[0], w2.shape[1]))
    bias = lambda b, g: None if b is None else b[g]
    for (g, c), v in zip(jobs, pmap(
            lambda j: oracle.expert_mlp(xrows[j[1]], w1[j[0]], w2[j[0]],
                                        bias(b1, j[0]), bias(b2, j[0])),
            jobs)):
        ref[c] = v
    return ref


@pytest.mark.parametrize("sizes,D,H,y_f32,bias", [
    # 288 / 216 large tiles in stages 1 / 2: both stages take the large tiles
    ([3000, 2500, 0, 2700], 1152, 2048, False, False),
    ([3000, 2500, 0, 2700], 1152, 2048, True, False),
    # stage 1 large (288 tiles), stage 2 small (72 large tiles, under 3/4 of
    # the CUs)
    ([9000], 256, 2048, False, False),
    # the XL layer's expert shapes (D = 1152, H = 4608) with ragged groups:
    # stage 1 has 1440 large tiles of 18 k stages (several per persistent
    # workgroup), stage 2 480 tiles of 72 k stages (about two per workgroup);
    # once more with biases on both matrices (the large tiles add them to the
    # accumulators before staging the tile)
    ([7000, 6000, 0, 7100], 1152, 4608, False, False),
    ([7000, 6000, 0, 7100], 1152, 4608, False, True),
    # stage 2's large tiles (three token-row k stages in flight) with a
    # reduction length that ends in a partial k stage (H % 64 = 8), and with
    # one partial stage (H = 40) or two (H = 104) in all
    ([3000, 2500, 0, 2700], 1152, 2056, False, True),
    ([12000, 9000], 1152, 40, False, False),
    ([12000, 9000], 1152, 104, True, False),
    # groups of 9, 33, 13, 1 and 17 row tiles: stage 1's bands of about 8
    # row tiles come out as [9], [9, 8, 8, 8], [7, 6], [1] and [9, 8]
    ([2100, 8300, 3200, 200, 4300], 1152, 2048, False, True),
])
def test_grouped_ffn_tile_forms(sizes, D, H, y_f32, bias):
    """Shapes on either side of the large/small tile switch, every row
    compared with the oracle."""
    rng = np.random.default_rng(sum(sizes) + D + H)
    G = len(sizes)
    offsets = np.concatenate([[0], np.cumsum(sizes)])
    total = int(offsets[-1])
    q = lambda a: synth.bf16_to_f32(synth.bf16_bits(a.astype(np.float32)))
    nsrc = total + 5
    xsrc = q(rng.standard_normal((nsrc, D)))
    w1 = q(rng.standard_normal((G, H, D)) * 0.03)
    w2 = q(rng.standard_normal((G, D, H)) * 0.03)
    b1 = (rng.standard_normal((G, H)) * 0.1).astype(np.float32) if bias else None
    b2 = (rng.standard_normal((G, D)) * 0.1).astype(np.float32) if bias else None
    ri = rng.permutation(nsrc)[:total]
    y = _run_ffn(xsrc, offsets, w1, w2, b1, b2, "bf16", row_index=ri,
                 y_f32=y_f32)
    assert not np.isnan(y).any()
    ref = _grouped_reference(xsrc[ri], offsets, w1, w2, b1, b2)
    for g in range(G):
        a, b = int(offsets[g]), int(offsets[g + 1])
        if b > a:
            assert_close(y[a:b], ref[a:b], "bf16", f"group {g}")


def _split_case(sizes, D, H, y_f32, bias, rng):
    """One moe_grouped_ffn_split call (gathered rows) and its oracle."""
    _, ops = _ops()
    G = len(sizes)
    offsets = np.concatenate([[0], np.cumsum(sizes)])
    total = int(offsets[-1])
    q = lambda a: synth.bf16_to_f32(synth.bf16_bits(a.astype(np.float32)))
    nsrc = total + 3
    xsrc = q(rng.standard_normal((nsrc, D)))
    w1 = q(rng.standard_normal((G, H, D)) * 0.03)
    w2 = q(rng.standard_normal((G, D, H)) * 0.03)
    b1 = (rng.standard_normal((G, H)) * 0.1).astype(np.float32) if bias else None
    b2 = (rng.standard_normal((G, D)) * 0.1).astype(np.float32) if bias else None
    ri = rng.permutation(nsrc)[:total]
    return dict(xsrc=xsrc, offsets=offsets, w1=w1, w2=w2, b1=b1, b2=b2, ri=ri,
                y_f32=y_f32)


def _run_split(c, ws):
    _, ops = _ops()
    G, H, D = c["w1"].shape
    total = int(c["offsets"][-1])
    x = _bits_tensor(c["xsrc"], "bf16")
    ri = torch.from_numpy(c["ri"].astype(np.int32)).to(DEV)
    ot = torch.from_numpy(c["offsets"].astype(np.int64)).to(DEV)
    w1t, w2t = _bits_tensor(c["w1"], "bf16"), _bits_tensor(c["w2"], "bf16")
    b1t = None if c["b1"] is None else torch.from_numpy(c["b1"]).to(DEV)
    b2t = None if c["b2"] is None else torch.from_numpy(c["b2"]).to(DEV)
    h = torch.empty(total, H, dtype=torch.bfloat16, device=DEV)
    ydt = torch.float32 if c["y_f32"] else torch.bfloat16
    y = torch.full((total, D), float("nan"), dtype=ydt, device=DEV)
    ops.moe_grouped_ffn(x, ri, total, ot, w1t, b1t, w2t, b2t, h, y,
                        split_ws=ws)
    return y


@pytest.mark.parametrize("sizes,D,H,y_f32,bias", [
    # 44 row-tiles x 6 feature tiles = 264 stage-2 tiles on 256 workgroups:
    # the last 8 split into 32 pieces of one k stage each (H = 2048)
    ([256 * 15 + 10, 256 * 14 + 100, 256 * 13], 1152, 2048, False, True),
    # 43 row-tiles: 2 tiles left over, 72 pieces of one stage (H = 4608)
    ([256 * 43 - 5], 1152, 4608, True, False),
    # 1560 tiles (about the XL layer's routed stage 2): 24 tiles in 10
    # pieces of 7 or 8 stages
    ([8292, 8092, 8292, 8092, 8192, 8192, 8292, 8092], 1152, 4608, False, False),
    # a whole number of rounds (768 tiles): no split
    ([256 * 32, 256 * 48, 256 * 48], 1152, 2048, False, False),
    # a reduction that ends in a partial k stage (H % 64 = 8, 33 stages):
    # the last piece of each split tile carries the k tail
    ([256 * 15 + 10, 256 * 14 + 100, 256 * 13], 1152, 2056, True, True),
])
def test_grouped_ffn_split(sizes, D, H, y_f32, bias):
    """moe_grouped_ffn_split, every row against the oracle, where stage 2's
    last round of tiles is split along k (or not, for a whole number of
    rounds); and against moe_grouped_ffn to fp32-summation accuracy."""
    _, ops = _ops()
    rng = np.random.default_rng(sum(sizes) + H)
    c = _split_case(sizes, D, H, y_f32, bias, rng)
    ws = torch.empty(ops.ffn_split_workspace_size(), dtype=torch.uint8,
                     device=DEV)
    ws.fill_(0xFF)   # needs no initialisation
    y = to_np(_run_split(c, ws))
    torch.cuda.synchronize()
    assert not np.isnan(y).any()
    ref = _grouped_reference(c["xsrc"][c["ri"]], c["offsets"], c["w1"],
                             c["w2"], c["b1"], c["b2"])
    offs = c["offsets"]
    for g in range(len(sizes)):
        a, b = int(offs[g]), int(offs[g + 1])
        if b > a:
            assert_close(y[a:b], ref[a:b], "bf16", f"group {g}")
    y0 = to_np(_run_split(c, None))
    if y_f32:
        assert np.allclose(y, y0, rtol=1e-4, atol=1e-4 * np.abs(y0).max())
    else:
        # bf16 outputs: the two roundings of sums that differ in the last
        # fp32 bits agree to one bf16 step
        assert np.abs(y - y0).max() <= 2 ** -7 * np.abs(y0).max()


def test_grouped_ffn_split_workspace_reuse():
    """Two split calls in a row on one workspace, the second with another
    split (the header is rewritten every call), then one with no split."""
    _, ops = _ops()
    rng = np.random.default_rng(7)
    ws = torch.empty(ops.ffn_split_workspace_size(), dtype=torch.uint8,
                     device=DEV)
    for sizes, H in (([256 * 15 + 10, 256 * 14 + 100, 256 * 13], 2048),
                     ([256 * 43 - 5], 1024),
                     ([256 * 32, 256 * 48, 256 * 48], 1024)):
        c = _split_case(sizes, 1152, H, False, True, rng)
        y = to_np(_run_split(c, ws))
        ref = _grouped_reference(c["xsrc"][c["ri"]], c["offsets"], c["w1"],
                                 c["w2"], c["b1"], c["b2"])
        assert_close(y, ref, "bf16", f"sizes {sizes}")


@pytest.mark.parametrize("rows,D,H", [(3000, 256, 1024), (12800, 256, 1024)],
                         ids=["small_tiles", "large_tiles"])
def test_gelu_saturation(rows, D, H):
    """Stage 1 with pre-activations far into both tails (W1 ~ N(0, 1), so
    u ~ N(0, 16) and |u| reaches 50): every h against the oracle's
    gelu_tanh of the exact u, element by element.  Positive tails give u
    itself, negative tails go to zero through the underflow of the
    exp2/rcp form: allowed an absolute error below 1e-6 (the exact values
    there are below 1e-6 too)."""
    _lib, ops = _ops()
    rng = np.random.default_rng(rows + D + H)
    q = lambda a: synth.bf16_to_f32(synth.bf16_bits(a.astype(np.float32)))
    x = q(rng.standard_normal((rows, D)))
    w1 = q(rng.standard_normal((1, H, D)))
    w2 = q(rng.standard_normal((1, D, H)) * 0.02)
    offs = torch.from_numpy(np.array([0, rows], np.int64)).to(DEV)
    h = torch.empty(rows, H, dtype=torch.bfloat16, device=DEV)
    u = torch.empty(rows, H, dtype=torch.bfloat16, device=DEV)
    ops.moe_grouped_ffn(_bits_tensor(x, "bf16"), None, rows, offs,
                        _bits_tensor(w1, "bf16"), None,
                        _bits_tensor(w2, "bf16"), None, h, None,
                        _lib.MOE_FFN_UP, u)
    torch.cuda.synchronize()
    hg, ug = to_np(h), to_np(u)
    uref = np.concatenate(pmap(lambda c: x[c].astype(np.float64) @
                               w1[0].T.astype(np.float64), chunks(np.arange(rows))))
    assert np.abs(uref).max() > 40 and (uref > 10).any() and (uref < -10).any()
    href = oracle.gelu_tanh(uref)
    assert np.isfinite(hg).all()
    assert_close(ug, uref, "bf16", "u")
    assert_close(hg, href, "bf16", "h")
    # elementwise: the bf16 rounding of h, plus the fp32 accumulation error
    # of u (at most 2^-20 of the sum of |x_d w_d|) times |gelu'| <= 1.13,
    # plus the underflow of the negative tail
    absum = np.concatenate(pmap(lambda c: np.abs(x[c]).astype(np.float64) @
                                np.abs(w1[0]).T.astype(np.float64),
                                chunks(np.arange(rows))))
    err = np.abs(hg - href)
    bound = 2.0 ** -7 * np.abs(href) + 1.13 * 2.0 ** -20 * absum + 1e-6
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert (err <= bound).all(), (uref[worst], hg[worst], href[worst])
    far = np.abs(uref) > 10
    assert np.all(np.abs(hg[far & (uref < 0)]) <= 1e-6)
    pos = far & (uref > 0)
    assert np.all(np.abs(hg[pos] - uref[pos]) <=
                  2.0 ** -7 * uref[pos] + 2.0 ** -20 * absum[pos])


@pytest.mark.parametrize("sizes,D,H,gather,bias,y_f32", [
    ([100, 0, 129, 1, 256, 0, 0, 300], 128, 256, False, False, False),
    ([100, 0, 129, 1, 256, 0, 0, 300], 256, 512, True, True, False),
    ([513], 384, 64, False, True, True),
    ([77, 3, 200], 384, 1536, True, False, False),
    ([(i * 37) % 23 * 3 for i in range(64)], 128, 192, True, False, True),
    ([0, 0, 0], 128, 256, False, False, False),
    # the S layer's routed experts: 16 groups of about 1024 rows
    ([1024 + (i * 97) % 200 - 100 for i in range(16)], 384, 1536, True, False,
     False),
])
def test_grouped_mlp_fused(sizes, D, H, gather, bias, y_f32):
    """The one-kernel MLP against the two-stage grouped FFN on the same
    inputs (same bits) and against the oracle (rows sampled when large)."""
    _, ops = _ops()
    rng = np.random.default_rng(sum(sizes) + D + H)
    G = len(sizes)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    total = int(offsets[-1])
    q = lambda a: synth.bf16_to_f32(synth.bf16_bits(a.astype(np.float32)))
    nsrc = total + 9
    xsrc = q(rng.standard_normal((nsrc, D)))
    w1 = q(rng.standard_normal((G, H, D)) * 0.05)
    w2 = q(rng.standard_normal((G, D, H)) * 0.05)
    b1 = (rng.standard_normal((G, H)) * 0.1).astype(np.float32) if bias else None
    b2 = (rng.standard_normal((G, D)) * 0.1).astype(np.float32) if bias else None
    ri = rng.permutation(nsrc)[:total] if gather else None
    xs = xsrc if gather else xsrc[:total]
    y_two = _run_ffn(xs, offsets, w1, w2, b1, b2, "bf16", row_index=ri,
                     y_f32=y_f32)
    x = _bits_tensor(xs, "bf16")
    rit = None if ri is None else torch.from_numpy(ri.astype(np.int32)).to(DEV)
    ydt = torch.float32 if y_f32 else torch.bfloat16
    y = torch.full((total, D), float("nan"), dtype=ydt, device=DEV)
    b1t = None if b1 is None else torch.from_numpy(b1).to(DEV)
    b2t = None if b2 is None else torch.from_numpy(b2).to(DEV)
    ops.moe_grouped_mlp_fused(x, rit, total, torch.from_numpy(offsets).to(DEV),
                              _bits_tensor(w1, "bf16"), b1t,
                              _bits_tensor(w2, "bf16"), b2t, y)
    torch.cuda.synchronize()
    yf = to_np(y)
    if total == 0:
        return
    assert np.array_equal(yf, y_two), np.abs(yf - y_two).max()
    rows_all = xsrc[ri] if gather else xsrc[:total]
    pick = (np.arange(total) if total <= 3000 else
            np.unique(np.concatenate([rng.choice(total, 64, replace=False),
                                      offsets[1:-1] - 1, offsets[1:-1]])))
    pick = pick[pick < total]
    grp = np.searchsorted(offsets, pick, side="right") - 1
    ref = np.zeros((pick.size, D))
    for g in np.unique(grp):
        m = grp == g
        ref[m] = oracle.expert_mlp(rows_all[pick[m]], w1[g], w2[g],
                                   None if b1 is None else b1[g],
                                   None if b2 is None else b2[g])
    assert_close(yf[pick], ref, "bf16", "fused mlp")


def test_grouped_ffn_bf16_rows_fp32_out():
    rng = np.random.default_rng(3)
    q = lambda a: synth.bf16_to_f32(synth.bf16_bits(a.astype(np.float32)))
    offsets = np.array([0, 70, 70, 200])
    x = q(rng.standard_normal((200, 128)))
    w1 = q(rng.standard_normal((3, 256, 128)) * 0.05)
    w2 = q(rng.standard_normal((3, 128, 256)) * 0.05)
    y = _run_ffn(x, offsets, w1, w2, None, None, "bf16", y_f32=True)
    ref = np.concatenate([oracle.expert_mlp(x[a:b], w1[g], w2[g])
                          for g, (a, b) in enumerate(zip(offsets[:-1], offsets[1:]))
                          if b > a])
    assert_close(y, ref, "bf16", "grouped ffn fp32 out")


@pytest.mark.parametrize("N,D,Kmax,dtype,shared", [
    (1, 64, 2, "bf16", True), (1000, 1152, 2, "bf16", True),
    (300, 72, 5, "f32", False), (129, 256, 16, "bf16", True)])
def test_combine(N, D, Kmax, dtype, shared):
    _, ops = _ops()
    rng = np.random.default_rng(N + D)
    A = N * Kmax
    q = (lambda a: synth.bf16_to_f32(synth.bf16_bits(a))) if dtype == "bf16" else (lambda a: a)
    yr = q(rng.standard_normal((A, D)).astype(np.float32))
    sr = rng.permutation(A).reshape(N, Kmax).astype(np.int32)
    sr[rng.random((N, Kmax)) < 0.2] = -1
    w = rng.random((N, Kmax)).astype(np.float32)
    ysh = q(rng.standard_normal((N, D)).astype(np.float32)) if shared else None
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    y = torch.empty(N, D, dtype=dt, device=DEV)
    ops.moe_combine(_bits_tensor(yr, dtype), torch.from_numpy(sr).to(DEV),
                    torch.from_numpy(w).to(DEV),
                    None if ysh is None else _bits_tensor(ysh, dtype), y)
    torch.cuda.synchronize()
    ref = np.zeros((N, D))
    for k in range(Kmax):
        m = sr[:, k] >= 0
        ref[m] += w[m, k, None].astype(np.float64) * yr[sr[m, k]]
    if shared:
        ref += ysh
    assert_close(to_np(y), ref, dtype, "combine")


@pytest.mark.parametrize("B,T,E,K,race,mode", [
    (1, 1, 1, 1, False, "sequence"), (4, 256, 8, 2, False, "sequence"),
    (3, 100, 16, 2, True, "sequence"), (5, 64, 5, 3, False, "global"),
    (2, 1024, 64, 4, True, "global"), (32, 1024, 8, 2, False, "sequence")])
def test_balance(B, T, E, K, race, mode):
    _lib, ops = _ops()
    rng = np.random.default_rng(B * T + E)
    N = B * T
    P = oracle.softmax(rng.standard_normal((N, E)))
    P32 = P.astype(np.float32)
    if race:
        idx, _, _ = oracle.race_select(P32.astype(np.float64), K)
    else:
        idx, _ = oracle.topk_select(P32.astype(np.float64), K)
    counts = torch.empty(B, E, dtype=torch.int32, device=DEV)
    ps = torch.empty(B, E, dtype=torch.float32, device=DEV)
    loss = torch.empty(1, dtype=torch.float32, device=DEV)
    ops.moe_balance_stats(torch.from_numpy(P32).to(DEV),
                          torch.from_numpy(idx.astype(np.int32)).to(DEV), B, T,
                          K, 0.01,
                          _lib.MOE_BAL_GLOBAL if mode == "global" else _lib.MOE_BAL_PER_SEQUENCE,
                          counts, ps, loss)
    torch.cuda.synchronize()
    c_o, p_o, l_o = oracle.balance_stats(P32.astype(np.float64), idx, B, T, K,
                                         0.01, mode)
    assert np.array_equal(to_np(counts), c_o)
    assert np.allclose(to_np(ps), p_o, rtol=1e-5, atol=1e-5)
    assert abs(float(to_np(loss)[0]) - l_o) <= 1e-5 * abs(l_o)


@pytest.mark.parametrize("B,T,D,E,K,dtype,mode,bias", [
    (1, 16, 64, 1, 1, "bf16", "sequence", False),     # one group, E = 1
    (4, 256, 1152, 8, 2, "bf16", "sequence", True),
    (3, 112, 384, 16, 2, "bf16", "global", False),    # E = 16 columns
    (5, 64, 200, 5, 3, "bf16", "sequence", True),     # unused expert columns
    (3, 100, 256, 8, 2, "bf16", "sequence", False),   # T % 16 != 0: separate
    (2, 64, 128, 8, 2, "f32", "global", False),       # fp32 x: separate
    (2, 32, 2048, 16, 2, "bf16", "sequence", False),  # weights split in two phases
    (16, 1024, 2048, 16, 2, "bf16", "global", True),  # the race layer's shape
    (32, 1024, 1152, 8, 2, "bf16", "sequence", False),  # the XL layer
    (0, 16, 128, 8, 2, "bf16", "sequence", False),    # no tokens
    (0, 16, 128, 8, 2, "bf16", "global", False),
])
def test_gate_balance_matches_separate(B, T, D, E, K, dtype, mode, bias):
    """moe_gate_topk_balance against moe_gate_topk + moe_balance_stats on the
    same inputs: routing and counts bit for bit, the probability sums and
    the loss to fp32 summation-order accuracy; and against the oracle's
    balance statistic on the routing the GPU chose."""
    _lib, ops = _ops()
    rng = np.random.default_rng(B * T + D + E)
    N = B * T
    x32 = rng.standard_normal((N, D)).astype(np.float32)
    x = _bits_tensor(x32, dtype)
    wg = torch.from_numpy((rng.standard_normal((E, D)) * 0.05).astype(np.float32)).to(DEV)
    bt = (torch.from_numpy(rng.standard_normal(E).astype(np.float32)).to(DEV)
          if bias else None)
    mc = _lib.MOE_BAL_GLOBAL if mode == "global" else _lib.MOE_BAL_PER_SEQUENCE

    def bufs():
        f32, i32 = torch.float32, torch.int32
        return (torch.full((N, E), -1.0, dtype=f32, device=DEV),
                torch.full((N, K), -7, dtype=i32, device=DEV),
                torch.full((N, K), -1.0, dtype=f32, device=DEV),
                torch.full((B, E), -7, dtype=i32, device=DEV),
                torch.full((B, E), -1.0, dtype=f32, device=DEV),
                torch.full((1,), -1.0, dtype=f32, device=DEV))

    sep = bufs()
    ops.moe_gate_topk(x, wg, bt, K, _lib.MOE_ROUTE_TOPK, sep[0], sep[1], sep[2],
                      None)
    ops.moe_balance_stats(sep[0], sep[1], B, T, K, 0.01, mc, sep[3], sep[4],
                          sep[5])
    fus = bufs()
    ws = torch.empty(max(ops.gate_balance_workspace_size(B, T, E), 1),
                     dtype=torch.uint8, device=DEV)
    ws.fill_(0xFF)
    for _ in range(2):   # the workspace needs no initialisation
        ops.moe_gate_topk_balance(x, wg, bt, B, T, K, 0.01, mc, *fus, ws)
    torch.cuda.synchronize()
    s, f = [to_np(t) for t in sep], [to_np(t) for t in fus]
    for i, name in enumerate(("probs", "idx", "w", "counts")):
        assert np.array_equal(s[i], f[i]), name
    assert np.allclose(f[4], s[4], rtol=2e-6, atol=1e-6)
    if B == 0:
        assert float(f[5][0]) == 0.0 and float(s[5][0]) == 0.0
        return
    c_o, p_o, l_o = oracle.balance_stats(f[0].astype(np.float64),
                                         f[1].astype(np.int64), B, T, K, 0.01,
                                         mode)
    assert np.array_equal(f[3], c_o)
    assert np.allclose(f[4], p_o, rtol=1e-5, atol=1e-5)
    assert abs(float(f[5][0]) - l_o) <= 1e-5 * abs(l_o)
    assert abs(float(f[5][0]) - float(s[5][0])) <= 1e-5 * abs(l_o)


@pytest.mark.parametrize("B,T,D,E,K,dtype,mode,bias", [
    (1, 16, 64, 1, 1, "bf16", "sequence", False),     # one group, E = 1
    (4, 256, 1152, 8, 2, "bf16", "sequence", True),
    (3, 272, 384, 16, 2, "bf16", "global", False),    # last 256-token block partial
    (5, 48, 200, 12, 3, "bf16", "sequence", True),    # E = 12, K = 3
    (1, 4096, 384, 16, 1, "bf16", "sequence", False),  # one image, K = 1
    (3, 100, 256, 8, 2, "bf16", "sequence", False),   # T % 16 != 0: separate
    (2, 64, 128, 8, 2, "f32", "global", False),       # fp32 x: separate
    (16, 1024, 2048, 16, 2, "bf16", "global", True),  # the race layer's shape
    (32, 1024, 1152, 8, 2, "bf16", "sequence", False),  # the XL layer
    (0, 16, 128, 8, 2, "bf16", "sequence", False),    # no tokens
])
def test_gate_route_matches_separate(B, T, D, E, K, dtype, mode, bias):
    """moe_gate_route against moe_gate_topk_balance followed by moe_permute
    (index form) on the same inputs: every output bit for bit, twice in a row
    on a workspace full of garbage; and the permutation against the oracle's
    on the routing the GPU chose."""
    _lib, ops = _ops()
    rng = np.random.default_rng(B * T + D + E + K)
    N = B * T
    x32 = rng.standard_normal((N, D)).astype(np.float32)
    x = _bits_tensor(x32, dtype)
    wg = torch.from_numpy((rng.standard_normal((E, D)) * 0.05).astype(np.float32)).to(DEV)
    bt = (torch.from_numpy(rng.standard_normal(E).astype(np.float32)).to(DEV)
          if bias else None)
    mc = _lib.MOE_BAL_GLOBAL if mode == "global" else _lib.MOE_BAL_PER_SEQUENCE
    f32, i32, i64 = torch.float32, torch.int32, torch.int64

    def bufs():
        return (torch.full((N, E), -1.0, dtype=f32, device=DEV),
                torch.full((N, K), -7, dtype=i32, device=DEV),
                torch.full((N, K), -1.0, dtype=f32, device=DEV),
                torch.full((B, E), -7, dtype=i32, device=DEV),
                torch.full((B, E), -1.0, dtype=f32, device=DEV),
                torch.full((1,), -1.0, dtype=f32, device=DEV),
                torch.full((E,), -7, dtype=i32, device=DEV),
                torch.full((E + 1,), -7, dtype=i64, device=DEV),
                torch.full((max(K * N, 1),), -7, dtype=i32, device=DEV),
                torch.full((N, K), -7, dtype=i32, device=DEV))

    sep = bufs()
    gws = torch.empty(max(ops.gate_balance_workspace_size(B, T, E), 1),
                      dtype=torch.uint8, device=DEV)
    ops.moe_gate_topk_balance(x, wg, bt, B, T, K, 0.01, mc, *sep[:6], gws)
    pws = torch.empty(max(ops.permute_workspace_size(N, E, K), 1),
                      dtype=torch.uint8, device=DEV)
    ops.moe_permute(x, sep[1], E, K, sep[6], sep[7], sep[8], sep[9], None, pws)
    fus = bufs()
    ws = torch.empty(max(ops.gate_route_workspace_size(B, T, E), 1),
                     dtype=torch.uint8, device=DEV)
    ws.fill_(0xFF)
    for _ in range(2):   # the workspace needs no initialisation
        ops.moe_gate_route(x, wg, bt, B, T, K, 0.01, mc, *fus, ws)
    torch.cuda.synchronize()
    s, f = [to_np(t) for t in sep], [to_np(t) for t in fus]
    names = ("probs", "idx", "w", "counts", "prob_sums", "loss",
             "expert_counts", "expert_offsets", "row_token", "slot_row")
    for i, name in enumerate(names):
        assert np.array_equal(s[i], f[i]), name
    if B == 0:
        assert float(f[5][0]) == 0.0 and f[7].tolist() == [0] * (E + 1)
        return
    c_o, o_o, rt_o, sr_o = oracle.permute(f[1].astype(np.int32), E)
    assert np.array_equal(f[6], c_o) and np.array_equal(f[7], o_o)
    assert np.array_equal(f[8][:K * N], rt_o) and np.array_equal(f[9], sr_o)


# ------------------------------------------------------- routing analytics --

def _run_hist(idx, B, T, E, tags, n_tags, calls=1):
    _lib, ops = _ops()
    pos = torch.zeros(T, E, dtype=torch.int64, device=DEV)
    tag = None if tags is None else torch.zeros(n_tags, E, dtype=torch.int64,
                                                device=DEV)
    ti = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).to(DEV)
    tg = None if tags is None else torch.from_numpy(
        np.asarray(tags, dtype=np.int32)).to(DEV)
    for _ in range(calls):
        ops.moe_routing_histogram(ti, B, T, E, pos, tg, tag)
    torch.cuda.synchronize()
    return to_np(pos), None if tag is None else to_np(tag)


@pytest.mark.parametrize("B,T,E,Kmax,kind,tagged", [
    (1, 1, 1, 1, "topk", True), (3, 70, 8, 2, "topk", True),
    (9, 129, 16, 2, "race", True), (32, 1024, 8, 2, "topk", True),
    (5, 64, 64, 4, "random", True), (17, 33, 5, 3, "random", False),
    (16, 1024, 16, 16, "race", True)])
def test_routing_histogram(B, T, E, Kmax, kind, tagged):
    """Bit-exact counts; random rows include -1 and indices >= E, and some
    tags lie outside [0, n_tags)."""
    rng = np.random.default_rng(B * 1000 + T + E)
    N = B * T
    if kind == "random":
        idx = rng.integers(-1, E + 3, size=(N, Kmax))
    else:
        P = oracle.softmax(rng.standard_normal((N, E)) * 2.0)
        if kind == "race":
            idx, _, _ = oracle.race_select(P, Kmax if Kmax < E else 2)
        else:
            idx, _ = oracle.topk_select(P, Kmax)
    n_tags = 7
    tags = rng.integers(-1, n_tags + 1, size=B) if tagged else None
    pos, tag = _run_hist(idx, B, T, E, tags, n_tags)
    pos_o, tag_o = oracle.routing_histogram(idx, B, T, E, tags=tags,
                                            n_tags=n_tags)
    assert np.array_equal(pos, pos_o)
    if tagged:
        assert np.array_equal(tag, tag_o)


def test_routing_histogram_accumulates():
    """Two calls add: totals are twice one batch's counts."""
    rng = np.random.default_rng(5)
    B, T, E = 6, 200, 8
    P = oracle.softmax(rng.standard_normal((B * T, E)))
    idx, _ = oracle.topk_select(P, 2)
    tags = np.arange(B) % 3
    pos, tag = _run_hist(idx, B, T, E, tags, 3, calls=2)
    pos_o, tag_o = oracle.routing_histogram(idx, B, T, E, tags=tags, n_tags=3)
    assert np.array_equal(pos, 2 * pos_o) and np.array_equal(tag, 2 * tag_o)


def test_routing_histogram_empty_batch():
    pos, tag = _run_hist(np.zeros((0, 2), np.int32), 0, 16, 8, None, 0)
    assert not pos.any()


# ------------------------------------------- shared stage 2 + combine, fused --

@pytest.mark.parametrize("N,D,H,Kmax,empty,bias", [
    (1, 64, 128, 1, 0.0, False), (300, 128, 256, 2, 0.1, True),
    (1000, 384, 512, 4, 0.3, False), (2049, 1152, 384, 2, 0.0, True),
    (777, 200, 136, 3, 0.5, True),
    # the large-tile form: 474 tiles of 256 x 192 (about two per persistent
    # workgroup) over 72 k stages, XL's shared hidden width per expert
    (20000, 1152, 4608, 2, 0.05, False),
    # Expert Race's slot layout: 16 slots per token, most of them empty
    # (the 16-column form of the kernel), small and large tiles
    (700, 256, 512, 16, 0.85, True), (5000, 2048, 1024, 16, 0.88, False),
    # large tiles whose reduction ends in a partial k stage (H % 64 = 8),
    # with 2 and 16 slots (the 16-slot form loads its slot table late)
    (20000, 1152, 4616, 2, 0.05, True), (5000, 2048, 1032, 16, 0.88, True)])
def test_ffn_down_combine_matches_separate(N, D, H, Kmax, empty, bias):
    """The fused kernel gives the bits of stage 2 (one group of all tokens)
    followed by the combine kernel, and both agree with the oracle on every
    row."""
    _lib, ops = _ops()
    rng = np.random.default_rng(N + D + H + Kmax)
    q = lambda a: synth.bf16_to_f32(synth.bf16_bits(a.astype(np.float32)))
    h = q(rng.standard_normal((N, H)))
    w2 = q(rng.standard_normal((1, D, H)) * 0.05)
    b2 = (rng.standard_normal((1, D)) * 0.1).astype(np.float32) if bias else None
    A = N * Kmax
    yr = q(rng.standard_normal((A, D)))
    sr = rng.permutation(A).reshape(N, Kmax).astype(np.int32)
    sr[rng.random((N, Kmax)) < empty] = -1
    w = rng.random((N, Kmax)).astype(np.float32)
    bf = lambda a: _bits_tensor(a, "bf16")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    th, tw2, tyr = bf(h), bf(w2), bf(yr)
    tb2 = None if b2 is None else dev(b2)
    tsr, tw = dev(sr), dev(w)
    # separate: stage 2 of one group of all N tokens, then the combine
    y_sh = torch.empty(N, D, dtype=torch.bfloat16, device=DEV)
    offs = dev(np.array([0, N], np.int64))
    ops.moe_grouped_ffn(None, None, N, offs, None, None, tw2, tb2, th, y_sh,
                        _lib.MOE_FFN_DOWN)
    y_sep = torch.empty(N, D, dtype=torch.bfloat16, device=DEV)
    ops.moe_combine(tyr, tsr, tw, y_sh, y_sep)
    y_fused = torch.empty(N, D, dtype=torch.bfloat16, device=DEV)
    ops.moe_ffn_down_combine(th, tw2, tb2, tyr, tsr, tw, y_fused)
    torch.cuda.synchronize()
    assert torch.equal(y_fused.view(torch.int16), y_sep.view(torch.int16))
    w2t = w2[0].T.astype(np.float64)
    ref = np.concatenate(pmap(lambda c: h[c].astype(np.float64) @ w2t,
                              chunks(np.arange(N))))
    if b2 is not None:
        ref += b2[0]
    for k in range(Kmax):
        m = sr[:, k] >= 0
        ref[m] += w[m, k, None].astype(np.float64) * yr[sr[m, k]]
    assert_close(to_np(y_fused), ref, "bf16", "fused stage 2 + combine")


def test_ffn_down_combine_empty():
    _lib, ops = _ops()
    z = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    w2 = torch.zeros(1, 64, 64, dtype=torch.bfloat16, device=DEV)
    sr = torch.empty(0, 2, dtype=torch.int32, device=DEV)
    w = torch.empty(0, 2, dtype=torch.float32, device=DEV)
    ops.moe_ffn_down_combine(z, w2, None, z, sr, w, z)
    torch.cuda.synchronize()
