"""GPU-vs-oracle comparison helpers shared by the GPU tests and smoke().

Routing is compared exactly except on near-tie tokens (two fp32 scores that
decide the selection or the slot order closer than 1e-6); those tokens take
the GPU's choice when it is a valid resolution of the tie, and everything
downstream (permutation, counts, outputs, balance) is then checked against
the oracle evaluated on that reconciled routing.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch
from threadpoolctl import threadpool_limits

import oracle
import synth

NEAR = oracle.NEAR_TIE

# Output tolerances: fp32 layers 1e-4 relative; bf16 layers 2e-2 of the
# largest reference magnitude and 5e-3 on average.  Loss 1e-5 relative.
TOL = {"f32": dict(max_rel=1e-4, mean_rel=1e-4),
       "bf16": dict(max_rel=2e-2, mean_rel=5e-3)}
LOSS_RTOL = 1e-5
PROB_ATOL = 1e-6


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def rel_errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(got - ref)
    mx = max(float(np.abs(ref).max(initial=0.0)), 1e-30)
    sm = max(float(np.abs(ref).sum()), 1e-30)
    return float(d.max(initial=0.0)) / mx, float(d.sum()) / sm


def assert_close(got, ref, dtype: str, what: str):
    mx, mean = rel_errors(got, ref)
    tol = TOL[dtype]
    assert mx <= tol["max_rel"] and mean <= tol["mean_rel"], (
        f"{what}: max-rel {mx:.3g} (<= {tol['max_rel']}), "
        f"mean-rel {mean:.3g} (<= {tol['mean_rel']})")
    return mx, mean


def near_topk(P, K):
    """Tokens whose top-K set or slot order hinges on a gap below 1e-6
    between adjacent fp32 scores among the first K+1."""
    s = oracle.decision_scores(P).astype(np.float64)
    srt = -np.sort(-s, axis=1)
    upto = min(K + 1, s.shape[1])
    if upto < 2:
        return np.zeros(s.shape[0], bool)
    gaps = srt[:, :upto - 1] - srt[:, 1:upto]
    return (gaps < NEAR).any(axis=1)


def reconcile_topk(P, idx_o, idx_g):
    s = oracle.decision_scores(P).astype(np.float64)
    N, K = idx_o.shape
    near = near_topk(P, K)
    rec = idx_o.copy()
    mism = np.nonzero((idx_o != idx_g).any(axis=1))[0]
    bad = []
    for t in mism:
        g = idx_g[t]
        ok = near[t] and len(set(g.tolist())) == K and g.min() >= 0 and g.max() < s.shape[1]
        if ok:
            kth = s[t, idx_o[t, K - 1]]
            sel = set(g.tolist())
            ok = all(s[t, i] >= kth - NEAR for i in sel) and all(
                s[t, j] <= kth + NEAR for j in range(s.shape[1]) if j not in sel)
            # slot order: descending within the tie band
            ok = ok and all(s[t, g[k]] >= s[t, g[k + 1]] - NEAR for k in range(K - 1))
        if ok:
            rec[t] = g
        else:
            bad.append(int(t))
    return rec, bad, near


def reconcile_race(P, K, idx_o, idx_g, tau):
    s = oracle.decision_scores(P).astype(np.float64)
    N, E = s.shape
    rec = idx_o.copy()
    mism = np.nonzero((idx_o != idx_g).any(axis=1))[0]
    bad = []
    for t in mism:
        so = set(i for i in idx_o[t].tolist() if i >= 0)
        g = [i for i in idx_g[t].tolist() if i >= 0]
        sg = set(g)
        padded = list(idx_g[t][len(g):]) == [-1] * (E - len(g))
        ok = (padded and g == sorted(g) and len(sg) == len(g) and
              all(0 <= i < E for i in g) and
              all(abs(s[t, i] - tau) < NEAR for i in so ^ sg))
        if ok:
            rec[t] = idx_g[t]
        else:
            bad.append(int(t))
    total = int((rec >= 0).sum())
    if total != K * N:
        bad.append(-1)
    return rec, bad


class GpuLayer:
    """Upload one layer's inputs, run the library, fetch the results."""

    def __init__(self, inp, gather=False, y_rows_f32=False, device="cuda",
                 save_u=False):
        from sparse_moe_diffusion_amd import layer
        self.layer = layer
        self.inp = inp
        self.cfg = inp.cfg
        dt = torch.bfloat16 if self.cfg.dtype == "bf16" else torch.float32
        self.x = layer._to_device(inp.x, dt, device)
        self.w = layer.LayerWeights.from_inputs(inp, device)
        self.buf = layer.LayerBuffers(self.cfg, device, gather=gather,
                                      y_rows_f32=y_rows_f32, save_u=save_u)

    def run(self, balance_mode="sequence"):
        self.layer.forward(self.cfg, self.x, self.w, self.buf, balance_mode)
        torch.cuda.synchronize()
        return self

    def result(self):
        b = self.buf
        out = dict(probs=to_np(b.probs), idx=to_np(b.topk_idx),
                   w=to_np(b.topk_w), expert_counts=to_np(b.expert_counts),
                   offsets=to_np(b.expert_offsets),
                   row_token=to_np(b.row_token)[:self.cfg.A],
                   slot_row=to_np(b.slot_row), y=to_np(b.y),
                   bal_counts=to_np(b.bal_counts), bal_psum=to_np(b.bal_psum),
                   loss=float(to_np(b.loss)[0]))
        return out


def check_layer(inp, g, sample_tokens=None, balance_mode="sequence",
                check_probs=True):
    """Compare GPU results ``g`` (GpuLayer.result()) with the oracle.

    Routing, permutation and balance counts are checked on every token;
    outputs on ``sample_tokens`` (default: all).  Returns a report dict.
    """
    cfg = inp.cfg
    r = oracle.route(inp)
    P = r["P"]
    rep = {}
    if check_probs:
        dp = float(np.abs(g["probs"] - P).max(initial=0.0))
        assert dp <= PROB_ATOL, f"probs differ by {dp:.3g}"
        rep["probs_maxabs"] = dp
    if cfg.route == "race":
        rec, bad = reconcile_race(P, cfg.K, r["idx"], g["idx"], r["tau"])
        rep["near_tokens"] = int(r["near"].sum())
    else:
        rec, bad, near = reconcile_topk(P, r["idx"], g["idx"])
        rep["near_tokens"] = int(near.sum())
    assert not bad, f"routing differs on non-tie tokens {bad[:10]}"
    rep["reconciled_tokens"] = int((rec != r["idx"]).any(axis=1).sum())
    # slot weights are the GPU's fp32 probabilities of the chosen experts
    wo = oracle.slot_weights(P, rec)
    assert np.abs(g["w"] - wo).max(initial=0.0) <= PROB_ATOL
    # permutation: bit-exact
    counts, offsets, row_token, slot_row = oracle.permute(rec, cfg.E)
    assert np.array_equal(g["expert_counts"], counts)
    assert np.array_equal(g["offsets"], offsets)
    assert np.array_equal(g["row_token"], row_token)
    assert np.array_equal(g["slot_row"], slot_row)
    # outputs
    tokens = np.arange(cfg.N) if sample_tokens is None else np.asarray(sample_tokens)
    yo = oracle_layer_output(inp, rec, wo, tokens)
    rep["y_max_rel"], rep["y_mean_rel"] = assert_close(g["y"][tokens], yo,
                                                       cfg.dtype, "y")
    # balance statistic
    bc, bp, loss = oracle.balance_stats(P, rec, cfg.B, cfg.T, cfg.K, cfg.alpha,
                                        balance_mode)
    assert np.array_equal(g["bal_counts"], bc)
    assert np.allclose(g["bal_psum"], bp, rtol=1e-5, atol=1e-5)
    rep["loss"], rep["loss_ref"] = g["loss"], loss
    assert abs(g["loss"] - loss) <= LOSS_RTOL * abs(loss), (g["loss"], loss)
    return rep


def workers() -> int:
    """Host threads for the oracle's chunked runs: the CPUs this process may
    use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def pmap(fn, items):
    """[fn(i) for i in items] on a thread pool, BLAS held to one thread per
    call.  numpy's elementwise passes and matrix products release the GIL,
    so oracle calls on disjoint row chunks run side by side; each result is
    the oracle's own call on its chunk."""
    items = list(items)
    with threadpool_limits(1), ThreadPoolExecutor(workers()) as ex:
        return list(ex.map(fn, items))


def chunks(rows, size=1024):
    rows = np.asarray(rows)
    return [rows[i:i + size] for i in range(0, rows.size, size)]


def oracle_layer_output(inp, idx, w, tokens=None):
    """oracle.layer_output on every token (or on ``tokens``), evaluated as
    the oracle's calls on chunks of 1024 tokens in parallel."""
    tokens = np.arange(inp.cfg.N) if tokens is None else np.asarray(tokens)
    parts = pmap(lambda t: oracle.layer_output(inp, idx, w, t), chunks(tokens))
    return np.concatenate(parts) if parts else np.zeros((0, inp.cfg.D))


def sample_tokens(cfg, n=48, seed=0):
    """A spread of token rows: first, last and random ones."""
    rng = np.random.default_rng(seed)
    t = rng.choice(cfg.N, size=min(n, cfg.N), replace=False)
    return np.unique(np.concatenate([t, [0, cfg.N - 1]]))
