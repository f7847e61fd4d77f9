"""Whole-layer parity: the HIP path through the C ABI against the CPU oracle.

Every layer, the full-size workloads included, is compared on every token:
routing, permutation, outputs and the balance statistic.
"""
import numpy as np
import pytest

import synth
from parity import GpuLayer, check_layer

pytestmark = pytest.mark.gpu

sc = synth.small_config
SMALL = [
    sc("tiny_bf16"),
    sc("tiny_f32", dtype="f32"),
    # D and H not multiples of the 64-wide k-tile or 128-wide output tile
    sc("ragged", B=3, T=77, D=136, H=264, E=5, K=2, n_s=1, seed=3),
    sc("e16_bias", B=2, T=96, D=192, H=384, E=16, K=2, n_s=2, logit_bias=True,
       seed=4),
    sc("k1_ns0", E=4, K=1, n_s=0, seed=5),
    sc("e1", E=1, K=1, n_s=0, seed=6),
    sc("k_eq_e", E=4, K=4, n_s=1, seed=8),
    sc("e64", B=2, T=64, D=64, H=128, E=64, K=3, n_s=1, seed=9),
    sc("e3_bias", B=2, T=50, D=64, H=128, E=3, K=2, n_s=2, logit_bias=True,
       seed=10),
    sc("race", B=2, T=64, D=128, H=256, E=16, K=2, n_s=2, route="race", seed=11),
    sc("race_f32", B=2, T=48, D=64, H=128, E=8, K=2, n_s=1, route="race",
       dtype="f32", seed=12),
    sc("race_e5", B=3, T=33, D=72, H=136, E=5, K=3, n_s=0, route="race", seed=13),
    sc("one_token", B=1, T=1, seed=14),
    sc("many_groups_tail", B=4, T=129, D=256, H=512, E=8, K=2, n_s=2,
       logit_bias=True, seed=15),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
@pytest.mark.parametrize("gather", [False, True], ids=["x_perm", "gather"])
def test_small_layer(cfg, gather):
    inp = synth.make_inputs(cfg)
    g = GpuLayer(inp, gather=gather).run().result()
    rep = check_layer(inp, g)
    print(cfg.name, rep, flush=True)


def test_small_layer_fp32_expert_outputs():
    cfg = sc("y_f32", B=2, T=70, seed=21)
    inp = synth.make_inputs(cfg)
    g = GpuLayer(inp, y_rows_f32=True).run().result()
    check_layer(inp, g)


@pytest.mark.parametrize("mode", ["sequence", "global"])
def test_balance_modes(mode):
    cfg = sc("bal", B=5, T=48, E=8, K=2, logit_bias=True, seed=22)
    inp = synth.make_inputs(cfg)
    g = GpuLayer(inp).run(balance_mode=mode).result()
    check_layer(inp, g, balance_mode=mode)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_full_size_workload(name):
    """The benchmark's workloads at their full sizes, in the launch
    configuration it times (gathered rows, fused gate+balance and
    stage-2+combine where the layer fuses them): y on all N tokens."""
    cfg = synth.CONFIGS[name]
    print(f"[full-size] {name} N={cfg.N} D={cfg.D} H={cfg.H} E={cfg.E}",
          flush=True)
    inp = synth.make_inputs(cfg)
    gl = GpuLayer(inp, gather=True).run()
    g = gl.result()
    del gl
    rep = check_layer(inp, g)
    counts = g["expert_counts"]
    print(name, rep, "expert rows", counts.tolist(), flush=True)
    assert counts.sum() == cfg.A
