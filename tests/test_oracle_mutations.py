"""Plant plausible mistakes in the CPU oracle and confirm the pins catch each.

Every mutation replaces one oracle function with a wrong variant (a dropped
term, a wrong sign, index or axis, a transposed operand, a wrong
normalisation) for the duration of one test; at least one pin must fail.
"""
import numpy as np
import pytest

import oracle_pins as pins
from oracle import moe_oracle as om

_orig = {n: getattr(om, n) for n in dir(om) if callable(getattr(om, n))}


def _gelu_no_cubic(u):
    u = np.asarray(u, dtype=np.float64)
    return 0.5 * u * (1.0 + np.tanh(om.GELU_C * u))


def _gelu_wrong_const(u):
    u = np.asarray(u, dtype=np.float64)
    return 0.5 * u * (1.0 + np.tanh(np.sqrt(np.pi / 2) * (u + om.GELU_A * u ** 3)))


def _gelu_erf(u):
    import math
    u = np.asarray(u, dtype=np.float64)
    return 0.5 * u * (1.0 + np.vectorize(math.erf)(u / math.sqrt(2.0)))


def _softmax_wrong_axis(l):
    l = np.asarray(l, dtype=np.float64)
    e = np.exp(l - l.max(axis=0, keepdims=True))
    return e / e.sum(axis=0, keepdims=True)


def _softmax_no_shift(l):
    l = np.asarray(l, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(l)
        return e / e.sum(axis=1, keepdims=True)


def _gate_transposed(x, w_gate, bias=None):
    l = np.asarray(x, np.float64) @ np.asarray(w_gate, np.float64).T[::-1]
    return l if bias is None else l + bias


def _gate_drop_bias(x, w_gate, bias=None):
    return _orig["gate_logits"](x, w_gate, None)


def _topk_ascending(P, K):
    s = om.decision_scores(P)
    order = np.argsort(s, axis=1, kind="stable")
    return order[:, :K].astype(np.int32), np.full(s.shape[0], np.inf)


def _topk_high_index_ties(P, K):
    s = om.decision_scores(P)
    E = s.shape[1]
    order = (E - 1 - np.argsort(-s[:, ::-1], axis=1, kind="stable"))
    idx, margin = _orig["topk_select"](P, K)
    return order[:, :K].astype(np.int32), margin


def _race_per_token(P, K):
    idx, _ = _orig["topk_select"](P, K)
    N, E = P.shape
    out = np.full((N, E), -1, dtype=np.int32)
    out[:, :K] = np.sort(idx, axis=1)
    return out, 0.0, np.zeros(N, bool)


def _race_descending(P, K):
    idx, tau, near = _orig["race_select"](P, K)
    E = idx.shape[1]
    srt = np.sort(np.where(idx < 0, -1, idx), axis=1)[:, ::-1]
    return srt.astype(np.int32), tau, near


def _weights_renormalised(P, idx):
    w = _orig["slot_weights"](P, idx)
    return w / w.sum(axis=1, keepdims=True)


def _weights_one(P, idx):
    return np.where(idx >= 0, 1.0, 0.0)


def _mlp_transposed_w2(x_rows, w1, w2, b1=None, b2=None):
    return _orig["expert_mlp"](x_rows, w1, np.swapaxes(w2, -1, -2).copy()
                               if w2.shape[0] == w2.shape[1] else w2[:, ::-1],
                               b1, b2)


def _shared_half(x, w1s, w2s, tokens=None):
    return 0.5 * _orig["shared_output"](x, w1s, w2s, tokens)


def _balance_no_n(P, idx, B, T, K, alpha, mode="sequence"):
    c, ps, L = _orig["balance_stats"](P, idx, B, T, K, alpha, mode)
    return c, ps, L / P.shape[1]


def _balance_no_K(P, idx, B, T, K, alpha, mode="sequence"):
    c, ps, L = _orig["balance_stats"](P, idx, B, T, K, alpha, mode)
    return c, ps, L * K


def _balance_selected_probs(P, idx, B, T, K, alpha, mode="sequence"):
    I = om.selection_indicator(idx, P.shape[1])
    return _orig["balance_stats"](np.asarray(P) * I, idx, B, T, K, alpha, mode)


def _permute_unstable(idx, E):
    counts, offsets, row_token, slot_row = _orig["permute"](idx, E)
    # reverse the row order inside each expert group
    rt = row_token.copy()
    sr = slot_row.copy()
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        rt[a:b] = row_token[a:b][::-1]
        m = (sr >= a) & (sr < b)
        sr[m] = a + b - 1 - sr[m]
    return counts, offsets, rt, sr


def _hist_wraps_empty(idx, B, T, E, tags=None, n_tags=0):
    # an empty slot (-1) counted as the last expert (Python's negative index)
    idx = np.asarray(idx)
    return _orig["routing_histogram"](np.where(idx < 0, E - 1, idx), B, T, E,
                                      tags, n_tags)


def _hist_position_by_image(idx, B, T, E, tags=None, n_tags=0):
    # rows taken image-major as position-major: position = t // B
    idx = np.asarray(idx)
    N = idx.shape[0]
    perm = (np.arange(N) % B) * T + np.arange(N) // B
    return _orig["routing_histogram"](idx[perm], B, T, E, tags, n_tags)


def _hist_tag_by_position(idx, B, T, E, tags=None, n_tags=0):
    # the tag looked up by token position instead of by image
    pos, tag = _orig["routing_histogram"](idx, B, T, E, None, 0)
    if tags is None:
        return pos, None
    out = np.zeros((n_tags, E), np.int64)
    idx = np.asarray(idx)
    for t in range(idx.shape[0]):
        g = tags[(t % T) % len(tags)]
        for e in idx[t]:
            if 0 <= e < E and 0 <= g < n_tags:
                out[g, e] += 1
    return pos, out


def _gelu_grad_no_cubic(u):
    u = np.asarray(u, dtype=np.float64)
    th = np.tanh(om.GELU_C * (u + om.GELU_A * u ** 3))
    return 0.5 * (1.0 + th) + 0.5 * u * (1.0 - th * th) * om.GELU_C


def _softmax_backward_no_centering(P, dP):
    return np.asarray(P, np.float64) * np.asarray(dP, np.float64)


def _balance_grad_no_batch_mean(idx, E, B, T, K, alpha, mode="sequence"):
    return _orig["balance_grad"](idx, E, B, T, K, alpha, mode) * B


def _mlp_backward_w2_transposed(x_rows, w1, w2, dv, b1=None):
    dx, g1, g2, db1, db2 = _orig["expert_mlp_backward"](x_rows, w1, w2, dv, b1)
    return dx, g1, g2[::-1], db1, db2


def _mlp_backward_no_gelu_grad(x_rows, w1, w2, dv, b1=None):
    x = np.asarray(x_rows, np.float64)
    u = x @ np.asarray(w1, np.float64).T
    a = om.gelu_tanh(u)
    du = np.asarray(dv, np.float64) @ np.asarray(w2, np.float64)
    return du @ np.asarray(w1, np.float64), du.T @ x, np.asarray(dv).T @ a, du.sum(0), np.asarray(dv).sum(0)


MUTATIONS = {
    "gelu_no_cubic": ("gelu_tanh", _gelu_no_cubic),
    "gelu_wrong_constant": ("gelu_tanh", _gelu_wrong_const),
    "gelu_erf_variant": ("gelu_tanh", _gelu_erf),
    "softmax_wrong_axis": ("softmax", _softmax_wrong_axis),
    "softmax_no_max_shift": ("softmax", _softmax_no_shift),
    "gate_wrong_expert_rows": ("gate_logits", _gate_transposed),
    "gate_drops_bias": ("gate_logits", _gate_drop_bias),
    "topk_keeps_lowest": ("topk_select", _topk_ascending),
    "topk_ties_to_high_index": ("topk_select", _topk_high_index_ties),
    "race_per_token": ("race_select", _race_per_token),
    "race_descending_slots": ("race_select", _race_descending),
    "weights_renormalised": ("slot_weights", _weights_renormalised),
    "weights_ignored": ("slot_weights", _weights_one),
    "mlp_transposed_w2": ("expert_mlp", _mlp_transposed_w2),
    "shared_weight_half": ("shared_output", _shared_half),
    "balance_drops_n": ("balance_stats", _balance_no_n),
    "balance_drops_K": ("balance_stats", _balance_no_K),
    "balance_selected_probs": ("balance_stats", _balance_selected_probs),
    "permute_unstable": ("permute", _permute_unstable),
    "histogram_counts_empty_slots": ("routing_histogram", _hist_wraps_empty),
    "histogram_position_by_image": ("routing_histogram", _hist_position_by_image),
    "histogram_tag_by_position": ("routing_histogram", _hist_tag_by_position),
    "gelu_grad_drops_cubic_term": ("gelu_tanh_grad", _gelu_grad_no_cubic),
    "softmax_backward_not_centred": ("softmax_backward", _softmax_backward_no_centering),
    "balance_grad_not_averaged": ("balance_grad", _balance_grad_no_batch_mean),
    "mlp_backward_w2_transposed": ("expert_mlp_backward", _mlp_backward_w2_transposed),
    "mlp_backward_no_gelu_grad": ("expert_mlp_backward", _mlp_backward_no_gelu_grad),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(om, attr, bad)
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check()
        except Exception:  # noqa: BLE001 -- any failure counts as caught
            failed.append(check.__name__)
    assert failed, f"mutation {name} passed every pin"
