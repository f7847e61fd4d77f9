"""CPU oracle for the DiT-MoE sparse MoE feed-forward layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does.  It
shares no code with the HIP library and imports nothing from it.

Everything is computed in float64 from the exact stored input values (bf16
or fp32 values upcast exactly).  The one place where floating point decides
an integer -- which experts a token uses -- is decided on the probabilities
rounded to fp32, the precision the layer's gate is specified in.

Sources (cited by page title and section):
  [hub]   "DiT-MoE" project hub page, section 1 "MoE Gate routing": the gate
          weight is [n_routed_experts][gating_dim], scores are a softmax over
          the routed experts, the top-k experts are kept, an auxiliary
          balance loss is added.
  [paper] "Scaling Diffusion Transformers to 16 Billion Parameters" (reading
          note), Methods: "MoE recap" eq. MoE(x) = sum_i g(x)_i e_i(x);
          "MoE-DiT" eq. MLP(x) = W2 gelu(W1 x), shared expert routing,
          expert-level balance loss eq. L_balance; compute analysis (n, K,
          n_s per layer).
  [dit]   "Scalable Diffusion Models with Transformers (DiT)", model
          architecture, DiT block details: the GELU is the tanh
          approximation.
  [race]  "Expert Race: A Flexible Routing Strategy for Scaling Diffusion
          Transformer with Mixture of Experts", abstract: tokens and experts
          compete together and the top candidates are selected.

Readings where the pages are silent (each also listed in the design notes):
  * routed outputs are weighted by the full-softmax probability, with no
    renormalisation over the kept K;
  * shared experts are weighted 1;
  * ties go to the lower expert index (race: the lower flat index t*E+i);
  * race scores are the per-token softmax probabilities, the global top
    K*N of all N*E scores is kept, and a token lists its experts in
    ascending index order, padded with -1;
  * a token's slots are in descending-probability order for top-K;
  * the balance statistic is taken per image (T tokens) and averaged over
    the B images; a global variant pools all B*T tokens;
  * no capacity limit: every selection is computed;
  * backward (training, as the pages train with the balance loss added): the
    gradient of <dy, y> + dloss * L_balance with the routing held fixed --
    the selection itself has no gradient, the slot weights g(x)_i = P[t][i]
    do, and the balance statistic's counts carry none.
"""
from __future__ import annotations

import math

import numpy as np

# tanh-GELU constants: Hendrycks & Gimpel, "Gaussian Error Linear Units"
# (2016), the tanh approximation named by [dit].
GELU_C = math.sqrt(2.0 / math.pi)
GELU_A = 0.044715

NEAR_TIE = 1e-6


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------- gate ----

def gate_logits(x, w_gate, bias=None):
    """[hub] gate scores: l[t][i] = sum_d x[t][d] * W_g[i][d] (+ bias[i]).

    ``w_gate`` is [E][D] (n_routed_experts x gating_dim).  ``bias`` is an
    optional per-expert logit offset added before the softmax.
    """
    l = _f64(x) @ _f64(w_gate).T
    if bias is not None:
        l = l + _f64(bias)[None, :]
    return l


def softmax(logits):
    """[hub] scoring function 'softmax' over the E routed experts, per token:
    P[t][i] = exp(l_i - m) / sum_j exp(l_j - m) with m = max_j l_j."""
    l = _f64(logits)
    m = l.max(axis=1, keepdims=True)
    e = np.exp(l - m)
    return e / e.sum(axis=1, keepdims=True)


def decision_scores(P):
    """The fp32 probabilities the routing decisions are taken on."""
    return np.asarray(P, dtype=np.float64).astype(np.float32)


# ------------------------------------------------------------- routing ----

def topk_select(P, K):
    """[hub] keep the top-k experts of each token; [paper] MoE recap: a sparse
    g with k non-zero weights.

    Order the E experts by (fp32 probability descending, index ascending)
    and keep the first K.  Returns ``idx`` [N][K] int32 in that order and
    ``margin`` [N]: the gap between the K-th and (K+1)-th score (inf when
    K = E), used to flag near-ties.
    """
    s = decision_scores(P)
    N, E = s.shape
    if not 1 <= K <= E:
        raise ValueError("need 1 <= K <= E")
    order = np.argsort(-s, axis=1, kind="stable")
    idx = order[:, :K].astype(np.int32)
    if K < E:
        rows = np.arange(N)
        margin = (s[rows, order[:, K - 1]].astype(np.float64)
                  - s[rows, order[:, K]].astype(np.float64))
    else:
        margin = np.full(N, np.inf)
    return idx, margin


def race_select(P, K):
    """[race] tokens and experts compete in one pool: of all N*E scores keep
    the K*N largest, ordered by (fp32 probability descending, flat index
    t*E+i ascending).

    Returns ``idx`` [N][E] int32 -- each token's selected experts in
    ascending index order, padded with -1 --, the threshold ``tau`` (score
    of the last entry kept) and ``near`` [N] bool: tokens holding an entry
    within 1e-6 of ``tau``.
    """
    s = decision_scores(P)
    N, E = s.shape
    A = K * N
    flat = s.ravel()
    order = np.argsort(-flat, kind="stable")
    keep = np.zeros(N * E, dtype=bool)
    keep[order[:A]] = True
    keep = keep.reshape(N, E)
    cols = np.where(keep, np.arange(E)[None, :], E)
    cols.sort(axis=1)
    idx = np.where(cols == E, -1, cols).astype(np.int32)
    tau = float(flat[order[A - 1]]) if A > 0 else np.inf
    near = (np.abs(s.astype(np.float64) - tau) < NEAR_TIE).any(axis=1)
    return idx, tau, near


def slot_weights(P, idx):
    """Routed weight of each slot: the token's probability of that expert
    (0 for an empty slot)."""
    P = _f64(P)
    safe = np.where(idx >= 0, idx, 0)
    w = np.take_along_axis(P, safe, axis=1)
    return np.where(idx >= 0, w, 0.0)


def selection_indicator(idx, E):
    """I(t, i): 1 when token t selected expert i ([paper] balance loss)."""
    N = idx.shape[0]
    I = np.zeros((N, E), dtype=np.int64)
    t, k = np.nonzero(idx >= 0)
    np.add.at(I, (t, idx[t, k]), 1)
    return I


# ------------------------------------------------------------- permute ----

def permute(idx, E):
    """Group the selected (token, slot) pairs by expert.

    Rows of expert e are its selections in ascending (token, slot) order;
    ``offsets`` is the exclusive scan of the per-expert counts.  Returns
    counts [E], offsets [E+1], row_token [A] and slot_row [N][Kmax] (-1 for
    an empty slot).
    """
    N, Kmax = idx.shape
    flat = idx.ravel()
    pos = np.nonzero(flat >= 0)[0]
    experts = flat[pos]
    order = pos[np.argsort(experts, kind="stable")]
    counts = np.bincount(experts, minlength=E).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    row_token = (order // Kmax).astype(np.int32)
    slot_row = np.full(N * Kmax, -1, dtype=np.int64)
    slot_row[order] = np.arange(order.size)
    return counts, offsets, row_token, slot_row.reshape(N, Kmax).astype(np.int32)


# ------------------------------------------------------------- experts ----

def gelu_tanh(u):
    """[dit] tanh-approximated GELU:
    0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3)))."""
    u = _f64(u)
    return 0.5 * u * (1.0 + np.tanh(GELU_C * (u + GELU_A * u ** 3)))


def expert_mlp(x_rows, w1, w2, b1=None, b2=None):
    """[paper] MoE-DiT, eq. MLP: e(x) = W2 gelu(W1 x) for each row x.

    ``w1`` is [H][D] and ``w2`` is [D][H] (output features by input
    features).  Optional biases are added after each product.
    """
    u = _f64(x_rows) @ _f64(w1).T
    if b1 is not None:
        u = u + _f64(b1)
    a = gelu_tanh(u)
    v = a @ _f64(w2).T
    if b2 is not None:
        v = v + _f64(b2)
    return v


def routed_output(x, idx, w, w1, w2, tokens=None):
    """[paper] MoE recap: sum over the selected experts i of g(x)_i e_i(x),
    with g(x)_i the slot weight.  Only the selected experts are evaluated.

    ``tokens`` restricts the output to those token rows (default: all).
    """
    x = _f64(x)
    if tokens is None:
        tokens = np.arange(x.shape[0])
    tokens = np.asarray(tokens)
    sub_idx = idx[tokens]
    sub_w = _f64(w)[tokens]
    y = np.zeros((tokens.size, x.shape[1]))
    for e in range(w1.shape[0]):
        r, k = np.nonzero(sub_idx == e)
        if r.size == 0:
            continue
        v = expert_mlp(x[tokens[r]], w1[e], w2[e])
        np.add.at(y, r, sub_w[r, k][:, None] * v)
    return y


def shared_output(x, w1s, w2s, tokens=None):
    """[paper] shared expert routing: every token goes to each of the n_s
    shared experts, whatever the router picks; their outputs are summed with
    weight 1."""
    x = _f64(x)
    if tokens is not None:
        x = x[np.asarray(tokens)]
    y = np.zeros_like(x)
    for s in range(w1s.shape[0]):
        y += expert_mlp(x, w1s[s], w2s[s])
    return y


def gelu_tanh_grad(u):
    """Derivative of gelu_tanh: with z = sqrt(2/pi) (u + 0.044715 u^3),
    d/du [0.5 u (1 + tanh z)] = 0.5 (1 + tanh z)
                                + 0.5 u (1 - tanh^2 z) sqrt(2/pi) (1 + 3 0.044715 u^2)."""
    u = _f64(u)
    th = np.tanh(GELU_C * (u + GELU_A * u ** 3))
    return 0.5 * (1.0 + th) + 0.5 * u * (1.0 - th * th) * GELU_C * (
        1.0 + 3.0 * GELU_A * u * u)


def expert_mlp_backward(x_rows, w1, w2, dv, b1=None):
    """Gradients of v = W2 gelu(W1 x (+ b1)) (+ b2), row by row, given dv =
    dLoss/dv: returns (dx_rows, dW1 [H][D], dW2 [D][H], db1 [H], db2 [D])."""
    x = _f64(x_rows)
    u = x @ _f64(w1).T
    if b1 is not None:
        u = u + _f64(b1)
    a = gelu_tanh(u)
    dv = _f64(dv)
    du = (dv @ _f64(w2)) * gelu_tanh_grad(u)
    return du @ _f64(w1), du.T @ x, dv.T @ a, du.sum(axis=0), dv.sum(axis=0)


def softmax_backward(P, dP):
    """dLoss/dlogits of P = softmax(logits) per row: P (dP - sum_j P_j dP_j)."""
    P = _f64(P)
    dP = _f64(dP)
    return P * (dP - (P * dP).sum(axis=1, keepdims=True))


def balance_grad(idx, E, B, T, K, alpha, mode="sequence"):
    """dL/dP[t][i] of the balance statistic with the counts held fixed (the
    selection indicator has no gradient):
      sequence: alpha / B * (n/(K T)) c[b][i] / T   for token t of image b
      global:   alpha * (n/(K B T)) sum_b c[b][i] / (B T)"""
    I = selection_indicator(idx, E)
    counts = I.reshape(B, T, E).sum(axis=1).astype(np.float64)
    if mode == "sequence":
        g = alpha / B * (E / (K * T)) * counts / T          # [B][E]
        return np.repeat(g, T, axis=0)
    if mode == "global":
        Tg = B * T
        g = alpha * (E / (K * Tg)) * counts.sum(axis=0) / Tg
        return np.broadcast_to(g, (Tg, E)).copy()
    raise ValueError(mode)


def layer_backward(inputs, idx, w, P, dy, dloss=0.0, balance_mode="sequence"):
    """Gradients of  Loss = <dy, y> + dloss * L_balance  with the routing idx
    held fixed (selection has no gradient; the slot weights w = P[idx] do):

      routed slot (t,k) with expert e: dv = w[t][k] dy[t],
        dw[t][k] = <dy[t], e(x_t)>, expert backward for dx, dW1[e], dW2[e]
      shared expert s: dv = dy
      dP[t][i] = sum_k [idx[t][k] == i] dw[t][k] + dloss * dL/dP[t][i]
      dlogits = softmax_backward(P, dP);  dW_g = dlogits^T x;
      dbias = sum_t dlogits;  dx = routed + shared + dlogits W_g.
    Returns a dict of fp64 arrays."""
    cfg = inputs.cfg
    x = _f64(inputs.x)
    dy = _f64(dy)
    N, D = x.shape
    E = cfg.E
    Kmax = idx.shape[1]
    dx = np.zeros((N, D))
    dw = np.zeros((N, Kmax))
    dw1 = np.zeros(_f64(inputs.w1).shape)
    dw2 = np.zeros(_f64(inputs.w2).shape)
    for e in range(E):
        r, k = np.nonzero(idx == e)
        if r.size == 0:
            continue
        v = expert_mlp(x[r], inputs.w1[e], inputs.w2[e])
        dw[r, k] = (dy[r] * v).sum(axis=1)
        dv = _f64(w)[r, k][:, None] * dy[r]
        dxr, g1, g2, _, _ = expert_mlp_backward(x[r], inputs.w1[e],
                                                inputs.w2[e], dv)
        np.add.at(dx, r, dxr)
        dw1[e] += g1
        dw2[e] += g2
    out = dict(dw=dw, dw1=dw1, dw2=dw2)
    if cfg.n_s > 0:
        dw1s = np.zeros(_f64(inputs.w1s).shape)
        dw2s = np.zeros(_f64(inputs.w2s).shape)
        for s_ in range(cfg.n_s):
            dxs, g1, g2, _, _ = expert_mlp_backward(x, inputs.w1s[s_],
                                                    inputs.w2s[s_], dy)
            dx += dxs
            dw1s[s_] = g1
            dw2s[s_] = g2
        out.update(dw1s=dw1s, dw2s=dw2s)
    dP = np.zeros((N, E))
    valid = idx >= 0
    np.add.at(dP, (np.nonzero(valid)[0], idx[valid]), dw[valid])
    if dloss:
        dP += dloss * balance_grad(idx, E, cfg.B, cfg.T, cfg.K, cfg.alpha,
                                   balance_mode)
    dl = softmax_backward(P, dP)
    dx += dl @ _f64(inputs.w_gate)
    out.update(dP=dP, dlogits=dl, dw_gate=dl.T @ x, dbias=dl.sum(axis=0),
               dx=dx)
    return out


# ------------------------------------------------------------- balance ----

def balance_stats(P, idx, B, T, K, alpha, mode="sequence"):
    """[paper] expert-level balance loss:
        L = alpha * sum_i (n/(K T) sum_t I(t,i)) * (1/T sum_t P(t,i))
    with n the number of routed experts, T the patch-sequence length,
    I(t,i) the selection indicator and P(t,i) the token's full softmax
    probability of expert i.

    mode "sequence": the sums run over each image's T tokens and the loss is
    the mean over the B images.  mode "global": one pool of B*T tokens.
    Returns counts [B][E] (int64), prob_sums [B][E] and the loss.
    """
    P = _f64(P)
    N, E = P.shape
    if N != B * T:
        raise ValueError("P must hold B*T rows")
    I = selection_indicator(idx, E)
    counts = I.reshape(B, T, E).sum(axis=1)
    psum = P.reshape(B, T, E).sum(axis=1)
    if mode == "sequence":
        f = (E / (K * T)) * counts
        pbar = psum / T
        loss = alpha * float(np.mean((f * pbar).sum(axis=1)))
    elif mode == "global":
        Tg = B * T
        f = (E / (K * Tg)) * counts.sum(axis=0)
        pbar = psum.sum(axis=0) / Tg
        loss = alpha * float((f * pbar).sum())
    else:
        raise ValueError(mode)
    return counts, psum, loss


# ---------------------------------------------------- routing analytics ----

def routing_histogram(idx, B, T, E, tags=None, n_tags=0):
    """[paper] Expert Specialization Analysis: how often each expert is
    selected, seen by spatial position and by image class or denoising time
    step; [hub] section 4 (expert activation frequency per class, heatmaps by
    class, patch and step).

    idx [B*T][Kmax]: the routing of B images of T tokens.
      pos[p][i] = number of (image b, slot k) with idx[b*T + p][k] == i
      tag[g][i] = number of (token t, slot k) of the images b with
                  tags[b] == g and idx[t][k] == i
    Entries outside [0, E) (the -1 of an empty race slot) count nowhere; an
    image whose tag lies outside [0, n_tags) counts only by position.
    Returns (pos [T][E] int64, tag [n_tags][E] int64 or None).
    """
    idx = np.asarray(idx)
    N, Kmax = idx.shape
    if N != B * T:
        raise ValueError("idx must hold B*T rows")
    valid = (idx >= 0) & (idx < E)
    position = np.broadcast_to((np.arange(N) % T)[:, None], idx.shape)
    pos = np.zeros((T, E), np.int64)
    np.add.at(pos, (position[valid], idx[valid]), 1)
    if tags is None:
        return pos, None
    tag_of_token = np.repeat(np.asarray(tags, np.int64), T)
    g = np.broadcast_to(tag_of_token[:, None], idx.shape)
    ok = valid & (g >= 0) & (g < n_tags)
    tag = np.zeros((n_tags, E), np.int64)
    np.add.at(tag, (g[ok], idx[ok]), 1)
    return pos, tag


# --------------------------------------------------------- whole layer ----

def route(inputs):
    """Gate, softmax and selection for every token of ``inputs``.

    Returns a dict with P [N][E] (fp64), idx, slot weights w, and the
    near-tie flags of each token (``near`` [N] bool).
    """
    cfg = inputs.cfg
    P = softmax(gate_logits(inputs.x, inputs.w_gate, inputs.bias))
    if cfg.route == "race":
        idx, tau, near = race_select(P, cfg.K)
        extra = {"tau": tau}
    else:
        idx, margin = topk_select(P, cfg.K)
        near = margin < NEAR_TIE
        extra = {"margin": margin}
    return dict(P=P, idx=idx, w=slot_weights(P, idx), near=near, **extra)


def layer_output(inputs, idx, w, tokens=None):
    """y = routed sum + shared sum, for the given routing (fp64)."""
    y = routed_output(inputs.x, idx, w, inputs.w1, inputs.w2, tokens)
    if inputs.cfg.n_s > 0:
        y = y + shared_output(inputs.x, inputs.w1s, inputs.w2s, tokens)
    return y


def forward(inputs, balance_mode="sequence"):
    """The whole layer on every token: routing, permutation, outputs and
    balance statistic."""
    cfg = inputs.cfg
    r = route(inputs)
    counts, offsets, row_token, slot_row = permute(r["idx"], cfg.E)
    y = layer_output(inputs, r["idx"], r["w"])
    bc, bp, loss = balance_stats(r["P"], r["idx"], cfg.B, cfg.T, cfg.K,
                                 cfg.alpha, balance_mode)
    r.update(expert_counts=counts, offsets=offsets, row_token=row_token,
             slot_row=slot_row, y=y, bal_counts=bc, bal_psum=bp, loss=loss)
    return r
