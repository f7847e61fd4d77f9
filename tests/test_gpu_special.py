"""Exact constructions through the real bf16 GEMM path, determinism, the
stage-split FFN, and degenerate layers (empty, single token)."""
import numpy as np
import pytest
import torch

import synth
from oracle_pins import one_hot_channel_inputs, uniform_counts_inputs
from parity import GpuLayer, check_layer, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("route", ["topk", "race"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_one_hot_channels_exact(route, dtype):
    """y[t][i] = P(t,i) for each selected routed expert i (0 otherwise) and
    y[t][E+s] = 1 for each shared expert, bit for bit: exactly K routed plus
    n_s shared contributions, weighted by the gate probability."""
    cfg = synth.small_config(B=2, T=96, D=64, H=128, E=8, K=2, n_s=2,
                             dtype=dtype, route=route, seed=31)
    inp = one_hot_channel_inputs(cfg)
    g = GpuLayer(inp).run().result()
    y, P, idx = g["y"], g["probs"], g["idx"]
    E = cfg.E
    want = np.zeros_like(y)
    for t in range(cfg.N):
        for i in idx[t]:
            if i >= 0:
                want[t, i] = P[t, i]
    want[:, E:E + cfg.n_s] = 1.0
    if dtype == "bf16":
        want = synth.bf16_to_f32(synth.bf16_bits(want.astype(np.float32)))
    assert np.array_equal(y, want)
    if route == "topk":
        assert np.all((y[:, :E] != 0).sum(axis=1) == cfg.K)
    else:
        assert int((y[:, :E] != 0).sum()) == cfg.K * cfg.N
    check_layer(inp, g)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_uniform_counts_loss_is_alpha(dtype):
    inp = uniform_counts_inputs(dtype=dtype)
    g = GpuLayer(inp).run().result()
    cfg = inp.cfg
    assert np.all(g["bal_counts"] == cfg.K * cfg.T // cfg.E)
    assert abs(g["loss"] - cfg.alpha) <= 1e-5 * cfg.alpha


def test_zero_gate_loss_is_alpha():
    cfg = synth.small_config(B=3, T=64, E=8, K=2, seed=32)
    inp = synth.make_inputs(cfg)
    inp.w_gate[:] = 0.0
    g = GpuLayer(inp).run().result()
    assert np.all(g["idx"] == np.arange(cfg.K))
    assert abs(g["loss"] - cfg.alpha) <= 1e-6 * cfg.alpha
    check_layer(inp, g)


def test_deterministic_bits():
    cfg = synth.small_config(B=4, T=100, D=256, H=512, E=8, K=2, n_s=2,
                             logit_bias=True, seed=33)
    inp = synth.make_inputs(cfg)
    gl = GpuLayer(inp)
    a = gl.run().result()
    b = gl.run().result()
    for k in ("probs", "idx", "w", "slot_row", "row_token", "y", "bal_psum"):
        assert np.array_equal(a[k], b[k]), k
    assert a["loss"] == b["loss"]


def test_race_deterministic_bits():
    cfg = synth.small_config(B=2, T=128, E=16, K=2, route="race", seed=34)
    gl = GpuLayer(synth.make_inputs(cfg))
    a = gl.run().result()
    b = gl.run().result()
    assert np.array_equal(a["idx"], b["idx"]) and np.array_equal(a["y"], b["y"])


def test_stage_split_matches_both():
    """Running the two FFN stages as two calls gives the same bits."""
    from sparse_moe_diffusion_amd import layer
    cfg = synth.small_config(B=2, T=90, D=128, H=256, seed=35)
    gl = GpuLayer(synth.make_inputs(cfg)).run()
    y_both = to_np(gl.buf.y).copy()
    gl.buf.y.zero_()
    gl.buf.y_rows.zero_()
    gl.buf.h.zero_()
    for name, step in layer.STEPS:
        step(cfg, gl.x, gl.w, gl.buf)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(gl.buf.y), y_both)


def test_empty_layer():
    """N = 0: every call succeeds and writes zero counts and a zero loss."""
    cfg = synth.small_config(B=0, T=16, seed=36)
    gl = GpuLayer(synth.make_inputs(cfg)).run()
    g = gl.result()
    assert g["expert_counts"].sum() == 0 and np.all(g["offsets"] == 0)
    assert g["loss"] == 0.0


@pytest.mark.parametrize("route,save_u", [("topk", False), ("race", False),
                                          ("topk", True)])
def test_layer_in_hip_graph(route, save_u):
    """The whole forward (and, for bf16 top-K, the backward) captured in one
    HIP graph and replayed three times, with eager work and synchronisation
    between the replays: every replay gives the eager pass's bits (no call
    allocates, synchronises or clears memory with hipMemsetAsync)."""
    from sparse_moe_diffusion_amd import layer
    cfg = synth.small_config(B=2, T=96, D=128, H=256, E=8, K=2, n_s=2,
                             route=route, seed=61)
    inp = synth.make_inputs(cfg)
    gl = GpuLayer(inp, gather=True, save_u=save_u)
    backward = route == "topk"
    dy = torch.randn(cfg.N, cfg.D, device="cuda",
                     generator=torch.Generator(device="cuda").manual_seed(3)
                     ).to(torch.bfloat16)
    grads = layer.BackwardBuffers(cfg) if backward else None

    def step():
        layer.forward(cfg, gl.x, gl.w, gl.buf)
        if backward:
            layer.backward(cfg, gl.x, gl.w, gl.buf, grads, dy, 1.0)

    names = ["probs", "topk_idx", "topk_w", "slot_row", "y", "bal_psum", "loss"]
    gnames = ["dx", "dw1", "dw2", "dw_gate"] if backward else []

    def snapshot():
        torch.cuda.synchronize()
        out = [getattr(gl.buf, n).clone() for n in names]
        out += [getattr(grads, n).clone() for n in gnames]
        return out

    step()
    ref = snapshot()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in [getattr(gl.buf, n) for n in names]:
            t.zero_()                      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        got = snapshot()
        for n, a, b in zip(names + gnames, ref, got):
            assert torch.equal(a, b), (rep, n)
