"""Checks that pin the CPU oracle to facts outside itself.

Each check raises AssertionError when the oracle disagrees with a closed
form, an invariant, a library routine, a brute force on tiny inputs or a
hand-worked fixture under tests/golden/.  The checks look the oracle's
functions up at call time, so the mutation tests can plant a mistake in one
oracle function and confirm that some check fails.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F
from scipy.special import softmax as scipy_softmax

import synth
from oracle import moe_oracle as om

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _tiny_inputs(seed=0, B=2, T=8, D=16, H=24, E=4, K=2, n_s=1, bias=False,
                 route="topk", scale=0.3):
    cfg = synth.LayerConfig("pin", B=B, T=T, D=D, H=H, E=E, K=K, n_s=n_s,
                            dtype="f32", route=route, logit_bias=bias, seed=seed)
    r = _rng(seed)
    x = r.standard_normal((cfg.N, D))
    wg = r.standard_normal((E, D)) * scale
    b = r.standard_normal(E) if bias else None
    w1 = r.standard_normal((E, H, D)) * scale
    w2 = r.standard_normal((E, D, H)) * scale
    w1s = r.standard_normal((n_s, H, D)) * scale
    w2s = r.standard_normal((n_s, D, H)) * scale
    return synth.LayerInputs(cfg, x, wg, b, w1, w2, w1s, w2s)


# ------------------------------------------------------------------ gate --

def check_gate_logits():
    r = _rng(1)
    N, D, E = 7, 11, 5
    x = r.standard_normal((N, D))
    # one-hot gate rows pick distinct input features: logit_i = x[:, c_i]
    cols = np.array([3, 0, 9, 4, 7])
    wg = np.zeros((E, D))
    wg[np.arange(E), cols] = 1.0
    assert np.array_equal(om.gate_logits(x, wg), x[:, cols])
    # a zero gate leaves the bias
    bias = r.standard_normal(E)
    assert np.array_equal(om.gate_logits(x, np.zeros((E, D)), bias),
                          np.broadcast_to(bias, (N, E)))
    # scaled one-hot plus bias
    l = om.gate_logits(x, 2.0 * wg, bias)
    assert np.allclose(l, 2.0 * x[:, cols] + bias, rtol=0, atol=1e-14)


def check_softmax():
    r = _rng(2)
    l = r.standard_normal((50, 8)) * 3
    P = om.softmax(l)
    assert np.allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.allclose(P, scipy_softmax(l, axis=1), rtol=1e-13, atol=0)
    assert np.allclose(om.softmax(l + 123.0), P, rtol=1e-12, atol=0)
    # equal logits: exactly 1/E for E a power of two; E = 1 gives 1
    for E in (1, 2, 8, 16):
        assert np.all(om.softmax(np.full((3, E), 0.7)) == 1.0 / E)
    # large logits do not overflow
    big = om.softmax(np.array([[1000.0, 999.0, -1000.0]]))
    assert np.isfinite(big).all() and abs(big[0, 0] / big[0, 1] - math.e) < 1e-12


# --------------------------------------------------------------- routing --

def _scores_with_ties(N, E, seed):
    r = _rng(seed)
    # quantised probabilities: many exact ties
    q = r.integers(1, 6, size=(N, E)).astype(np.float64)
    return q / q.sum(axis=1, keepdims=True)


def check_topk():
    for seed, (N, E, K) in enumerate([(40, 8, 2), (30, 4, 1), (25, 5, 5),
                                      (20, 16, 3)]):
        P = _scores_with_ties(N, E, seed + 10)
        s = P.astype(np.float32)
        idx, margin = om.topk_select(P, K)
        assert idx.shape == (N, K)
        for t in range(N):
            # brute force: the K-permutation that is largest under the total
            # order (score desc, index asc) is the sorted prefix
            best = sorted(range(E), key=lambda i: (-float(s[t, i]), i))[:K]
            assert list(idx[t]) == best, (t, idx[t], best)
            sel = set(best)
            for i in sel:
                for j in set(range(E)) - sel:
                    assert s[t, i] > s[t, j] or (s[t, i] == s[t, j] and i < j)
            if K < E:
                kth = s[t, best[-1]]
                nxt = max(float(s[t, j]) for j in range(E) if j not in sel)
                assert margin[t] == float(kth) - nxt
    # zero gate: every token picks experts 0..K-1 with zero margin
    P = om.softmax(np.zeros((6, 8)))
    idx, margin = om.topk_select(P, 2)
    assert (idx == np.array([0, 1])).all() and (margin == 0).all()


def check_race():
    for seed, (N, E, K) in enumerate([(12, 4, 2), (9, 8, 1), (10, 3, 3)]):
        P = _scores_with_ties(N, E, seed + 20)
        s = P.astype(np.float32)
        idx, tau, near = om.race_select(P, K)
        assert idx.shape == (N, E)
        # brute force: python sort of all (score, flat index) keys
        keys = sorted(range(N * E), key=lambda f: (-float(s.flat[f]), f))
        chosen = set(keys[:K * N])
        got = set()
        for t in range(N):
            row = list(idx[t])
            sel = [i for i in row if i >= 0]
            assert row == sel + [-1] * (E - len(sel))      # padding at end
            assert sel == sorted(sel)                      # ascending index
            got.update(t * E + i for i in sel)
        assert got == chosen
        assert len(got) == K * N
        assert tau == float(s.flat[keys[K * N - 1]])
    # identical tokens (distinct scores within a token): race == top-K
    r = _rng(5)
    row = r.permutation(np.arange(1, 9, dtype=np.float64))
    P = np.tile(row / row.sum(), (10, 1))
    idx_r, _, _ = om.race_select(P, 3)
    idx_k, _ = om.topk_select(P, 3)
    assert (np.sort(idx_k, axis=1) == idx_r[:, :3]).all()
    assert (idx_r[:, 3:] == -1).all()


def check_permute():
    r = _rng(3)
    N, E, Kmax = 37, 6, 3
    idx = np.full((N, Kmax), -1, dtype=np.int32)
    for t in range(N):
        m = r.integers(0, Kmax + 1)
        idx[t, :m] = r.choice(E, size=m, replace=False)
    counts, offsets, row_token, slot_row = om.permute(idx, E)
    # brute force enumeration: expert-major, then token, then slot
    rows = [(t, k) for e in range(E) for t in range(N) for k in range(Kmax)
            if idx[t, k] == e]
    assert list(row_token) == [t for t, _ in rows]
    for rr, (t, k) in enumerate(rows):
        assert slot_row[t, k] == rr
    assert (slot_row[idx < 0] == -1).all()
    assert list(counts) == [int((idx == e).sum()) for e in range(E)]
    assert offsets[0] == 0 and list(np.diff(offsets)) == list(counts)
    assert sorted(slot_row[idx >= 0].tolist()) == list(range(len(rows)))


# --------------------------------------------------------------- experts --

def check_gelu():
    u = np.linspace(-12, 12, 4801)
    g = om.gelu_tanh(u)
    ref = F.gelu(torch.from_numpy(u), approximate="tanh").numpy()
    assert np.allclose(g, ref, rtol=1e-14, atol=1e-15)
    assert om.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert np.allclose(g - om.gelu_tanh(-u), u, rtol=0, atol=1e-13)
    assert om.gelu_tanh(np.array([8.0]))[0] == 8.0
    # the tanh form stays within 6e-4 of the exact erf GELU, and differs
    exact = 0.5 * u * (1.0 + np.vectorize(math.erf)(u / math.sqrt(2.0)))
    gap = np.abs(g - exact).max()
    assert 1e-5 < gap < 6e-4, gap


def check_expert_mlp():
    r = _rng(4)
    x = r.standard_normal((9, 12))
    w1 = r.standard_normal((20, 12)) * 0.4
    w2 = r.standard_normal((12, 20)) * 0.4
    b1 = r.standard_normal(20)
    b2 = r.standard_normal(12)
    tx = torch.from_numpy
    ref = F.linear(F.gelu(F.linear(tx(x), tx(w1), tx(b1)), approximate="tanh"),
                   tx(w2), tx(b2)).numpy()
    assert np.allclose(om.expert_mlp(x, w1, w2, b1, b2), ref, rtol=1e-12,
                       atol=1e-13)


def _dense_mask_reference(inp, idx):
    """MoE(x) = sum_{i=1..E} g(x)_i e_i(x), evaluated densely with torch on
    every expert and every token; g is the softmax masked to the selection."""
    tx = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    x = tx(inp.x)
    l = x @ tx(inp.w_gate).T
    if inp.bias is not None:
        l = l + tx(inp.bias)
    P = torch.softmax(l, dim=1)
    E = inp.cfg.E
    mask = torch.zeros_like(P)
    for t in range(idx.shape[0]):
        for i in idx[t]:
            if i >= 0:
                mask[t, int(i)] = 1.0
    g = P * mask
    y = torch.zeros_like(x)
    for i in range(E):
        e_i = F.linear(F.gelu(F.linear(x, tx(inp.w1[i])), approximate="tanh"),
                       tx(inp.w2[i]))
        y = y + g[:, i:i + 1] * e_i
    for s in range(inp.cfg.n_s):
        y = y + F.linear(F.gelu(F.linear(x, tx(inp.w1s[s])), approximate="tanh"),
                         tx(inp.w2s[s]))
    return y.numpy(), P.numpy()


def check_dense_mask():
    cases = [dict(E=4, K=2, n_s=1), dict(E=6, K=6, n_s=0),
             dict(E=5, K=1, n_s=2, bias=True), dict(E=1, K=1, n_s=0),
             dict(E=8, K=3, n_s=2, route="race")]
    for seed, kw in enumerate(cases):
        inp = _tiny_inputs(seed=100 + seed, **kw)
        out = om.forward(inp)
        ref, Pref = _dense_mask_reference(inp, out["idx"])
        assert np.allclose(out["P"], Pref, rtol=1e-13, atol=1e-15)
        assert np.allclose(out["y"], ref, rtol=1e-11, atol=1e-12), kw


def check_dense_mlp_special_case():
    """E = 1, K = 1, n_s = 0: P = 1 so the layer is the plain MLP."""
    inp = _tiny_inputs(seed=7, E=1, K=1, n_s=0, bias=True)
    out = om.forward(inp)
    assert np.all(out["P"] == 1.0)
    tx = torch.from_numpy
    ref = F.linear(F.gelu(F.linear(tx(inp.x), tx(inp.w1[0])), approximate="tanh"),
                   tx(inp.w2[0])).numpy()
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-13)


def check_full_mixture():
    """K = E keeps every expert: the layer is the full softmax mixture."""
    inp = _tiny_inputs(seed=8, E=5, K=5, n_s=0)
    out = om.forward(inp)
    tx = torch.from_numpy
    x = tx(inp.x)
    P = torch.softmax(x @ tx(inp.w_gate).T, dim=1)
    y = sum(P[:, i:i + 1] * F.linear(F.gelu(F.linear(x, tx(inp.w1[i])),
                                            approximate="tanh"), tx(inp.w2[i]))
            for i in range(5))
    assert np.allclose(out["y"], y.numpy(), rtol=1e-11, atol=1e-12)


def one_hot_channel_inputs(cfg, seed=0):
    """Inputs whose outputs are known exactly (needs D >= E + n_s + 1).

    x[t][D-1] = 1; expert i has W1[0][D-1] = 8 and W2[i][0] = 1/8; shared
    expert s has W1[0][D-1] = 8 and W2[E+s][0] = 1/8.  Then u_0 = 8,
    gelu(8) = 8 exactly in fp32 and fp64, every other hidden unit is 0, so
    y[t][i] = P(t,i) when i is selected (else 0) and y[t][E+s] = 1.
    All values are exact in bf16.
    """
    E, D, H, n_s = cfg.E, cfg.D, cfg.H, cfg.n_s
    assert D >= E + n_s + 1
    inp = synth.make_inputs(cfg, seed=seed)
    x = inp.x.copy()
    x[:, D - 1] = 1.0
    w1 = np.zeros_like(inp.w1)
    w2 = np.zeros_like(inp.w2)
    w1[:, 0, D - 1] = 8.0
    for i in range(E):
        w2[i, i, 0] = 0.125
    w1s = np.zeros_like(inp.w1s)
    w2s = np.zeros_like(inp.w2s)
    w1s[:, 0, D - 1] = 8.0
    for s in range(n_s):
        w2s[s, E + s, 0] = 0.125
    return synth.LayerInputs(cfg, x, inp.w_gate, inp.bias, w1, w2, w1s, w2s)


def check_one_hot_channels():
    for route in ("topk", "race"):
        cfg = synth.small_config(B=2, T=16, D=32, H=16, E=8, K=2, n_s=2,
                                 dtype="f32", route=route, seed=9)
        inp = one_hot_channel_inputs(cfg)
        out = om.forward(inp)
        y, P, idx = out["y"], out["P"], out["idx"]
        E = cfg.E
        for t in range(cfg.N):
            sel = set(int(i) for i in idx[t] if i >= 0)
            for i in range(E):
                want = P[t, i] if i in sel else 0.0
                assert y[t, i] == want, (route, t, i)
            assert (y[t, E:E + cfg.n_s] == 1.0).all()
            assert (y[t, E + cfg.n_s:] == 0.0).all()
        if route == "topk":
            assert all(len(set(idx[t])) == cfg.K for t in range(cfg.N))


# --------------------------------------------------------------- balance --

def check_balance_uniform_probs():
    """Uniform P (zero gate): L = alpha for any routing."""
    for K, E in [(2, 8), (1, 4), (3, 3)]:
        B, T = 3, 16
        P = om.softmax(np.zeros((B * T, E)))
        idx, _ = om.topk_select(P, K)
        c, ps, L = om.balance_stats(P, idx, B, T, K, 0.01)
        assert abs(L - 0.01) <= 1e-17, L
        r = _rng(6)
        ridx = np.stack([r.choice(E, size=K, replace=False) for _ in range(B * T)])
        assert abs(om.balance_stats(P, ridx, B, T, K, 0.01)[2] - 0.01) <= 1e-17
        assert abs(om.balance_stats(P, ridx, B, T, K, 0.01, "global")[2]
                   - 0.01) <= 1e-17


def uniform_counts_inputs(B=2, T=32, E=8, K=2, D=16, dtype="f32"):
    """Gate whose top-K counts are exactly K*T/E per expert and image."""
    assert T % E == 0
    cfg = synth.small_config(B=B, T=T, D=D, H=16, E=E, K=K, n_s=0, dtype=dtype,
                             seed=11)
    inp = synth.make_inputs(cfg)
    wg = np.zeros((E, D), dtype=np.float32)
    wg[np.arange(E), np.arange(E)] = 1.0
    x = np.zeros((B * T, D), dtype=np.float32)
    t = np.arange(B * T)
    x[t, t % E] = 4.0
    x[t, (t + 1) % E] = 3.5
    return synth.LayerInputs(cfg, x, wg, None, inp.w1, inp.w2, inp.w1s, inp.w2s)


def check_balance_uniform_counts():
    """Equal counts K*T/E for every expert: L = alpha for any P."""
    inp = uniform_counts_inputs()
    cfg = inp.cfg
    out = om.forward(inp)
    assert (out["bal_counts"] == cfg.K * cfg.T // cfg.E).all()
    assert abs(out["loss"] - cfg.alpha) < 1e-15


def check_balance_invariants():
    inp = _tiny_inputs(seed=12, B=3, T=10, E=5, K=2, bias=True)
    out = om.forward(inp)
    c = out["bal_counts"]
    # sum_i f_i = n per image with f_i = n/(K T) c_i
    f = inp.cfg.E / (inp.cfg.K * inp.cfg.T) * c
    assert np.allclose(f.sum(axis=1), inp.cfg.E, rtol=0, atol=1e-13)
    assert (c.sum(axis=1) == inp.cfg.K * inp.cfg.T).all()
    assert np.allclose(out["bal_psum"].sum(axis=1), inp.cfg.T, atol=1e-12)


def check_balance_golden():
    with open(os.path.join(GOLDEN, "balance_tiny.json")) as fh:
        g = json.load(fh)
    P = np.array(g["P"], dtype=np.float64)
    idx, _ = om.topk_select(P, g["K"])
    assert idx.tolist() == g["idx"]
    c, ps, L = om.balance_stats(P, idx, g["B"], g["T"], g["K"], g["alpha"])
    assert c.tolist() == g["counts"]
    assert abs(L - g["loss"]) < 1e-15, (L, g["loss"])


# ----------------------------------------------------- routing analytics --

def check_routing_histogram_golden():
    with open(os.path.join(GOLDEN, "routing_histogram_tiny.json")) as fh:
        g = json.load(fh)
    pos, tag = om.routing_histogram(np.array(g["idx"]), g["B"], g["T"], g["E"],
                                    tags=g["tags"], n_tags=g["n_tags"])
    assert pos.tolist() == g["pos"]
    assert tag.tolist() == g["tag"]


def check_routing_histogram_brute():
    r = _rng(21)
    B, T, E, Kmax = 3, 5, 6, 3
    idx = r.integers(-1, E + 2, size=(B * T, Kmax))   # includes -1 and >= E
    tags = np.array([2, -1, 0])
    n_tags = 3
    pos_bf = [[0] * E for _ in range(T)]
    tag_bf = [[0] * E for _ in range(n_tags)]
    for b in range(B):
        for p in range(T):
            for k in range(Kmax):
                e = int(idx[b * T + p][k])
                if 0 <= e < E:
                    pos_bf[p][e] += 1
                    if 0 <= tags[b] < n_tags:
                        tag_bf[tags[b]][e] += 1
    pos, tag = om.routing_histogram(idx, B, T, E, tags=tags, n_tags=n_tags)
    assert pos.tolist() == pos_bf and tag.tolist() == tag_bf


def check_routing_histogram_invariants():
    # top-K routing of random probabilities: every position sees B*K
    # selections; per-image tags reproduce the balance statistic's counts; a
    # single tag holds the column sums of the position histogram
    inp = _tiny_inputs(seed=23, B=4, T=9, E=6, K=2)
    cfg = inp.cfg
    P = om.softmax(om.gate_logits(inp.x, inp.w_gate))
    idx, _ = om.topk_select(P, cfg.K)
    pos, tag = om.routing_histogram(idx, cfg.B, cfg.T, cfg.E,
                                    tags=np.arange(cfg.B), n_tags=cfg.B)
    assert (pos.sum(axis=1) == cfg.B * cfg.K).all()
    counts, _, _ = om.balance_stats(P, idx, cfg.B, cfg.T, cfg.K, 0.01)
    assert np.array_equal(tag, counts)
    _, tag1 = om.routing_histogram(idx, cfg.B, cfg.T, cfg.E,
                                   tags=np.zeros(cfg.B, np.int64), n_tags=1)
    assert np.array_equal(tag1[0], pos.sum(axis=0))
    # race: K*N selections in all, empty slots count nowhere
    ridx, _, _ = om.race_select(P, cfg.K)
    rpos, _ = om.routing_histogram(ridx, cfg.B, cfg.T, cfg.E)
    assert rpos.sum() == cfg.K * cfg.N
    # a zero gate: every token keeps experts 0..K-1
    P0 = om.softmax(om.gate_logits(inp.x, np.zeros_like(inp.w_gate)))
    zidx, _ = om.topk_select(P0, cfg.K)
    zpos, _ = om.routing_histogram(zidx, cfg.B, cfg.T, cfg.E)
    expect = np.zeros((cfg.T, cfg.E), np.int64)
    expect[:, :cfg.K] = cfg.B
    assert np.array_equal(zpos, expect)


# --------------------------------------------------------------- backward --

def check_gelu_grad():
    u = np.linspace(-6.0, 6.0, 241)
    h = 1e-5
    fd = (om.gelu_tanh(u + h) - om.gelu_tanh(u - h)) / (2 * h)
    assert np.abs(om.gelu_tanh_grad(u) - fd).max() < 1e-9
    # gelu(u) - gelu(-u) = u exactly, so gelu'(u) + gelu'(-u) = 1
    assert np.abs(om.gelu_tanh_grad(u) + om.gelu_tanh_grad(-u) - 1.0).max() < 1e-14
    # torch's tanh GELU, differentiated by autograd
    t = torch.tensor(u, dtype=torch.float64, requires_grad=True)
    g, = torch.autograd.grad(F.gelu(t, approximate="tanh").sum(), t)
    assert np.abs(om.gelu_tanh_grad(u) - g.numpy()).max() < 1e-14


def _loss_fixed_routing(inp, idx, dy, dloss, mode):
    """<dy, y> + dloss * L_balance at the inputs, routing held at idx; built
    from the forward functions only."""
    cfg = inp.cfg
    P = om.softmax(om.gate_logits(inp.x, inp.w_gate, inp.bias))
    w = om.slot_weights(P, idx)
    y = om.layer_output(inp, idx, w)
    _, _, L = om.balance_stats(P, idx, cfg.B, cfg.T, cfg.K, cfg.alpha, mode)
    return float((dy * y).sum()) + dloss * L


def _replace(inp, name, arr):
    f = dict(x=inp.x, w_gate=inp.w_gate, bias=inp.bias, w1=inp.w1, w2=inp.w2,
             w1s=inp.w1s, w2s=inp.w2s)
    f[name] = arr
    return synth.LayerInputs(inp.cfg, f["x"], f["w_gate"], f["bias"], f["w1"],
                             f["w2"], f["w1s"], f["w2s"])


def check_backward_finite_differences():
    for mode, route in (("sequence", "topk"), ("global", "race")):
        inp = _tiny_inputs(seed=31, B=2, T=4, D=6, H=8, E=3, K=2, n_s=1,
                           bias=True, route=route)
        cfg = inp.cfg
        r = om.route(inp)
        dy = _rng(32).standard_normal((cfg.N, cfg.D))
        dloss = 3.0
        g = om.layer_backward(inp, r["idx"], r["w"], r["P"], dy, dloss, mode)
        keys = dict(x="dx", w_gate="dw_gate", bias="dbias", w1="dw1",
                    w2="dw2", w1s="dw1s", w2s="dw2s")
        pick = _rng(33)
        h = 1e-6
        for name, gk in keys.items():
            base = np.array(getattr(inp, name), dtype=np.float64)
            for _ in range(6):
                j = tuple(int(pick.integers(0, n)) for n in base.shape)
                plus, minus = base.copy(), base.copy()
                plus[j] += h
                minus[j] -= h
                fd = (_loss_fixed_routing(_replace(inp, name, plus), r["idx"],
                                          dy, dloss, mode)
                      - _loss_fixed_routing(_replace(inp, name, minus),
                                            r["idx"], dy, dloss, mode)) / (2 * h)
                an = g[gk][j]
                assert abs(an - fd) <= 1e-6 * max(1.0, abs(fd)), (mode, name, j, an, fd)


def check_backward_autograd():
    """torch autograd (fp64, CPU) of the same loss with the routing fixed."""
    inp = _tiny_inputs(seed=34, B=3, T=5, D=7, H=9, E=4, K=2, n_s=2, bias=True)
    cfg = inp.cfg
    r = om.route(inp)
    idx = r["idx"]
    dy = _rng(35).standard_normal((cfg.N, cfg.D))
    dloss = 0.7
    T_ = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    x, wg, b = T_(inp.x), T_(inp.w_gate), T_(inp.bias)
    w1, w2, w1s, w2s = T_(inp.w1), T_(inp.w2), T_(inp.w1s), T_(inp.w2s)
    P = torch.softmax(x @ wg.T + b, dim=1)
    mlp = lambda z, a1, a2: F.gelu(z @ a1.T, approximate="tanh") @ a2.T
    y = torch.zeros(cfg.N, cfg.D, dtype=torch.float64)
    for t in range(cfg.N):
        for k in range(cfg.K):
            e = int(idx[t, k])
            y[t] = y[t] + P[t, e] * mlp(x[t:t + 1], w1[e], w2[e])[0]
    for s_ in range(cfg.n_s):
        y = y + mlp(x, w1s[s_], w2s[s_])
    I = torch.tensor(om.selection_indicator(idx, cfg.E), dtype=torch.float64)
    c = I.reshape(cfg.B, cfg.T, cfg.E).sum(1)
    pbar = P.reshape(cfg.B, cfg.T, cfg.E).sum(1) / cfg.T
    L = cfg.alpha * ((cfg.E / (cfg.K * cfg.T)) * c * pbar).sum(1).mean()
    loss = (torch.tensor(dy) * y).sum() + dloss * L
    grads = torch.autograd.grad(loss, [x, wg, b, w1, w2, w1s, w2s])
    g = om.layer_backward(inp, idx, r["w"], r["P"], dy, dloss, "sequence")
    for name, ref in zip(["dx", "dw_gate", "dbias", "dw1", "dw2", "dw1s", "dw2s"],
                         grads):
        assert np.abs(g[name] - ref.numpy()).max() < 1e-10, name


def check_backward_dense_mlp():
    """E = 1, K = 1, no shared expert: P = 1, the gate gets no gradient and
    dx, dW1, dW2 are those of the plain MLP (torch autograd)."""
    inp = _tiny_inputs(seed=36, B=2, T=6, D=5, H=7, E=1, K=1, n_s=0)
    cfg = inp.cfg
    r = om.route(inp)
    dy = _rng(37).standard_normal((cfg.N, cfg.D))
    g = om.layer_backward(inp, r["idx"], r["w"], r["P"], dy, 0.0)
    x = torch.tensor(inp.x, requires_grad=True)
    w1 = torch.tensor(inp.w1[0], requires_grad=True)
    w2 = torch.tensor(inp.w2[0], requires_grad=True)
    y = F.linear(F.gelu(F.linear(x, w1), approximate="tanh"), w2)
    gx, g1, g2 = torch.autograd.grad((torch.tensor(dy) * y).sum(), [x, w1, w2])
    assert np.abs(g["dx"] - gx.numpy()).max() < 1e-12
    assert np.abs(g["dw1"][0] - g1.numpy()).max() < 1e-12
    assert np.abs(g["dw2"][0] - g2.numpy()).max() < 1e-12
    assert np.abs(g["dw_gate"]).max() == 0.0 and np.abs(g["dbias"]).max() == 0.0


ALL_CHECKS = [check_gate_logits, check_softmax, check_topk, check_race,
              check_permute, check_gelu, check_expert_mlp, check_dense_mask,
              check_dense_mlp_special_case, check_full_mixture,
              check_one_hot_channels, check_balance_uniform_probs,
              check_balance_uniform_counts, check_balance_invariants,
              check_balance_golden, check_routing_histogram_golden,
              check_routing_histogram_brute, check_routing_histogram_invariants,
              check_gelu_grad, check_backward_finite_differences,
              check_backward_autograd, check_backward_dense_mlp]
