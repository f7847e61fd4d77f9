"""The C ABI on the host (no GPU): every symbol of include/moe.h is
exported, workspace queries answer, and invalid arguments are rejected with
the documented status before anything is launched."""
import ctypes
import os
import re

import pytest

from sparse_moe_diffusion_amd import _lib
from libmoe_build import ensure_built

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = ensure_built()
    names = _declared_functions()
    assert len(names) >= 9, names
    for n in names:
        assert hasattr(lib, n), n
    # the binding covers every declared entry point, same names
    assert set(names) == set(_lib.SIGNATURES), set(names) ^ set(_lib.SIGNATURES)


def test_status_strings():
    ensure_built()
    for code, name in [(0, "MOE_OK"), (1, "MOE_ERR_INVALID_ARGUMENT"),
                       (2, "MOE_ERR_UNSUPPORTED"),
                       (3, "MOE_ERR_WORKSPACE_TOO_SMALL"), (4, "MOE_ERR_HIP")]:
        assert _lib.status_string(code) == name


def test_workspace_queries():
    lib = ensure_built()
    assert lib.moe_gate_workspace_size(1000, 8, 2, _lib.MOE_ROUTE_TOPK) == 0
    assert lib.moe_gate_workspace_size(1000, 16, 2, _lib.MOE_ROUTE_EXPERT_RACE) > 0
    a = lib.moe_permute_workspace_size(32768, 8, 2)
    b = lib.moe_permute_workspace_size(65536, 8, 2)
    assert 0 < a < b


FAKE = 0x1000  # never dereferenced: validation fails before any launch


def _gate(**kw):
    a = dict(x=FAKE, dt=_lib.MOE_BF16, wg=FAKE, bias=None, N=64, D=128, E=8,
             K=2, route=_lib.MOE_ROUTE_TOPK, probs=FAKE, idx=FAKE, w=FAKE,
             ws=None, wsb=0, stream=None)
    a.update(kw)
    return _lib.call_status("moe_gate_topk", *a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(wg=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(probs=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(K=0), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(K=9), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(N=-1), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(route=7), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(E=65, K=2), _lib.MOE_ERR_UNSUPPORTED),
    (dict(D=100), _lib.MOE_ERR_UNSUPPORTED),
    (dict(dt=5), _lib.MOE_ERR_UNSUPPORTED),
    (dict(N=1 << 30, K=2), _lib.MOE_ERR_UNSUPPORTED),
    (dict(route=_lib.MOE_ROUTE_EXPERT_RACE), _lib.MOE_ERR_WORKSPACE_TOO_SMALL),
])
def test_gate_rejects(kw, status):
    ensure_built()
    assert _gate(**kw) == status
    assert _lib.last_error()


def _permute(**kw):
    a = dict(x=FAKE, dt=_lib.MOE_BF16, idx=FAKE, N=64, D=128, E=8, Kmax=2, K=2,
             counts=FAKE, offsets=FAKE, row_token=FAKE, slot_row=FAKE,
             x_perm=FAKE, ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    return _lib.call_status("moe_permute", *a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(idx=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(x=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(Kmax=3), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(K=0), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(E=70, K=2), _lib.MOE_ERR_UNSUPPORTED),
    (dict(D=12), _lib.MOE_ERR_UNSUPPORTED),
    (dict(wsb=0), _lib.MOE_ERR_WORKSPACE_TOO_SMALL),
])
def test_permute_rejects(kw, status):
    ensure_built()
    assert _permute(**kw) == status


def _permute_noalloc(**kw):
    a = dict(x=FAKE, dt=_lib.MOE_BF16, idx=FAKE, N=64, D=128, E=8, Kmax=2, K=2,
             counts=FAKE, offs=FAKE, rt=FAKE, sr=FAKE, xp=None, stream=None)
    a.update(kw)
    return _lib.call_status("moe_permute_noalloc", *a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(counts=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(idx=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(K=0), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(Kmax=3), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(N=-1), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(xp=FAKE, x=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(E=65), _lib.MOE_ERR_UNSUPPORTED),
    (dict(D=100), _lib.MOE_ERR_UNSUPPORTED),
    # the static scratch holds moe_permute's workspace up to 1 MiB
    (dict(N=1 << 24, E=64, Kmax=2), _lib.MOE_ERR_UNSUPPORTED),
    (dict(N=3 << 20, E=8, Kmax=2), _lib.MOE_ERR_UNSUPPORTED),
])
def test_permute_noalloc_rejects(kw, status):
    ensure_built()
    assert _permute_noalloc(**kw) == status
    assert "moe_permute_noalloc" in _lib.last_error()


def test_permute_noalloc_limit_matches_workspace_size():
    """The static scratch's size is the header's constant, and the sizes the
    call accepts are those whose moe_permute workspace fits it."""
    lib = ensure_built()
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    m = re.search(r"#define MOE_PERMUTE_NOALLOC_SCRATCH_BYTES \(1u << (\d+)\)",
                  text)
    limit = 1 << int(m.group(1))
    assert lib.moe_permute_workspace_size(2_700_000, 8, 2) <= limit
    assert lib.moe_permute_workspace_size(3 << 20, 8, 2) > limit


def _ffn(**kw):
    a = dict(x=FAKE, idx=None, src=0, dt=_lib.MOE_BF16, total=100, offs=FAKE,
             G=8,
             D=128, H=512, w1=FAKE, b1=None, w2=FAKE, b2=None, h=FAKE, u=None,
             y=FAKE, ydt=_lib.MOE_BF16, stages=_lib.MOE_FFN_BOTH, stream=None)
    a.update(kw)
    return _lib.call_status("moe_grouped_ffn", *a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(offs=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(h=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(G=0), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(total=-5), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(stages=0), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(stages=4), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(w1=None, stages=_lib.MOE_FFN_UP), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(y=None, stages=_lib.MOE_FFN_DOWN), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(G=129), _lib.MOE_ERR_UNSUPPORTED),
    (dict(H=100), _lib.MOE_ERR_UNSUPPORTED),
    (dict(dt=_lib.MOE_F32, ydt=_lib.MOE_BF16), _lib.MOE_ERR_UNSUPPORTED),
    (dict(dt=_lib.MOE_F32, ydt=_lib.MOE_F32, u=FAKE), _lib.MOE_ERR_UNSUPPORTED),
    (dict(total=1 << 31), _lib.MOE_ERR_UNSUPPORTED),
    # gathered rows: the source matrix's row count bounds the index
    (dict(idx=FAKE, src=0), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(idx=FAKE, src=-3), _lib.MOE_ERR_INVALID_ARGUMENT),
    # (src + 1) * D * 2 + 256 must stay within 2^32 (D = 128: src <= 2^24 - 2)
    (dict(idx=FAKE, src=(1 << 24) - 1), _lib.MOE_ERR_UNSUPPORTED),
    (dict(idx=FAKE, src=1 << 40), _lib.MOE_ERR_UNSUPPORTED),
    (dict(idx=FAKE, src=(1 << 23), dt=_lib.MOE_F32, ydt=_lib.MOE_F32),
     _lib.MOE_ERR_UNSUPPORTED),
])
def test_ffn_rejects(kw, status):
    ensure_built()
    assert _ffn(**kw) == status


def test_combine_and_balance_reject():
    ensure_built()
    args = dict(yr=FAKE, ydt=_lib.MOE_BF16, sr=FAKE, w=FAKE, N=10, D=64, Kmax=2,
                ysh=None, shdt=_lib.MOE_BF16, y=FAKE, odt=_lib.MOE_BF16,
                stream=None)
    for kw, st in [(dict(sr=None), _lib.MOE_ERR_INVALID_ARGUMENT),
                   (dict(Kmax=0), _lib.MOE_ERR_INVALID_ARGUMENT),
                   (dict(D=60), _lib.MOE_ERR_UNSUPPORTED),
                   (dict(odt=9), _lib.MOE_ERR_UNSUPPORTED)]:
        a = dict(args); a.update(kw)
        assert _lib.call_status("moe_combine", *a.values()) == st
    bargs = dict(p=FAKE, idx=FAKE, B=4, T=16, E=8, Kmax=2, K=2,
                 alpha=ctypes.c_float(0.01), mode=_lib.MOE_BAL_PER_SEQUENCE,
                 counts=FAKE, ps=FAKE, loss=FAKE, stream=None)
    for kw, st in [(dict(loss=None), _lib.MOE_ERR_INVALID_ARGUMENT),
                   (dict(T=0), _lib.MOE_ERR_INVALID_ARGUMENT),
                   (dict(K=9), _lib.MOE_ERR_INVALID_ARGUMENT),
                   (dict(mode=3), _lib.MOE_ERR_INVALID_ARGUMENT),
                   (dict(E=80, K=2), _lib.MOE_ERR_UNSUPPORTED)]:
        a = dict(bargs); a.update(kw)
        assert _lib.call_status("moe_balance_stats", *a.values()) == st


def _mlp_fused(**kw):
    a = dict(x=FAKE, ri=None, src=0, dt=_lib.MOE_BF16, total=256, off=FAKE,
             G=2, D=384, H=1536, w1=FAKE, b1=None, w2=FAKE, b2=None, y=FAKE,
             ydt=_lib.MOE_BF16, stream=None)
    a.update(kw)
    return _lib.call_status("moe_grouped_mlp_fused", *a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(w2=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(off=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(total=-1), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(G=0), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(D=1152), _lib.MOE_ERR_UNSUPPORTED),
    (dict(D=320), _lib.MOE_ERR_UNSUPPORTED),
    (dict(H=1000), _lib.MOE_ERR_UNSUPPORTED),
    (dict(dt=_lib.MOE_F32, ydt=_lib.MOE_F32), _lib.MOE_ERR_UNSUPPORTED),
    (dict(ydt=7), _lib.MOE_ERR_UNSUPPORTED),
    (dict(G=129), _lib.MOE_ERR_UNSUPPORTED),
    (dict(ri=FAKE, src=0), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(ri=FAKE, src=1 << 23), _lib.MOE_ERR_UNSUPPORTED),
])
def test_mlp_fused_rejects(kw, status):
    ensure_built()
    assert _mlp_fused(**kw) == status
    assert _lib.last_error()


def _gate_balance(**kw):
    a = dict(x=FAKE, dt=_lib.MOE_BF16, wg=FAKE, bias=None, B=4, T=16, D=128,
             E=8, K=2, alpha=ctypes.c_float(0.01),
             mode=_lib.MOE_BAL_PER_SEQUENCE, probs=FAKE, idx=FAKE, w=FAKE,
             counts=FAKE, ps=FAKE, loss=FAKE, ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    return _lib.call_status("moe_gate_topk_balance", *a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(loss=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(counts=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(K=0), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(K=9), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(T=0), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(B=-1), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(mode=2), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(E=65, K=2), _lib.MOE_ERR_UNSUPPORTED),
    (dict(D=100), _lib.MOE_ERR_UNSUPPORTED),
    (dict(dt=5), _lib.MOE_ERR_UNSUPPORTED),
    (dict(wsb=0), _lib.MOE_ERR_WORKSPACE_TOO_SMALL),
    (dict(ws=None), _lib.MOE_ERR_INVALID_ARGUMENT),
])
def test_gate_balance_rejects(kw, status):
    ensure_built()
    assert _gate_balance(**kw) == status
    assert _lib.last_error()


def test_gate_balance_workspace():
    lib = ensure_built()
    # 16-token groups x E partials, fp32 and int32 halves
    assert lib.moe_gate_balance_workspace_size(32, 1024, 8) == 2 * 2048 * 8 * 4
    assert lib.moe_gate_balance_workspace_size(0, 16, 8) == 0
    assert lib.moe_gate_balance_workspace_size(3, 100, 8) >= 2 * 19 * 8 * 4


def _gate_route(**kw):
    a = dict(x=FAKE, dt=_lib.MOE_BF16, wg=FAKE, bias=None, B=4, T=16, D=128,
             E=8, K=2, alpha=ctypes.c_float(0.01),
             mode=_lib.MOE_BAL_PER_SEQUENCE, probs=FAKE, idx=FAKE, w=FAKE,
             counts=FAKE, ps=FAKE, loss=FAKE, ecounts=FAKE, eoffs=FAKE,
             row_token=FAKE, slot_row=FAKE, ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    return _lib.call_status("moe_gate_route", *a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(loss=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(counts=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(ecounts=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(eoffs=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(row_token=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(slot_row=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(idx=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(K=0), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(K=9), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(T=0), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(B=-1), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(mode=2), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(E=65, K=2), _lib.MOE_ERR_UNSUPPORTED),
    (dict(D=100), _lib.MOE_ERR_UNSUPPORTED),
    (dict(dt=5), _lib.MOE_ERR_UNSUPPORTED),
    # K*N (and B*T*E) at 2^31
    (dict(B=1 << 15, T=1 << 15, E=2, K=2, wsb=1 << 62), _lib.MOE_ERR_UNSUPPORTED),
    (dict(wsb=0), _lib.MOE_ERR_WORKSPACE_TOO_SMALL),
    (dict(ws=None), _lib.MOE_ERR_INVALID_ARGUMENT),
])
def test_gate_route_rejects(kw, status):
    ensure_built()
    assert _gate_route(**kw) == status
    assert _lib.last_error()


def test_gate_route_workspace():
    lib = ensure_built()
    # the gate's partials, then the permutation's workspace
    for B, T, E in [(32, 1024, 8), (3, 100, 16), (0, 16, 8), (1, 16, 1)]:
        N = B * T
        assert (lib.moe_gate_route_workspace_size(B, T, E) ==
                lib.moe_gate_balance_workspace_size(B, T, E) +
                lib.moe_permute_workspace_size(N, E, 2))
    assert lib.moe_gate_route_workspace_size(-1, 16, 8) == 0


def _ffn_split(**kw):
    a = dict(x=FAKE, ri=None, src=0, dt=_lib.MOE_BF16, total=16, offs=FAKE,
             G=1, D=128, H=256, w1=FAKE, b1=None, w2=FAKE, b2=None, h=FAKE,
             u=None, y=FAKE, ydt=_lib.MOE_BF16, stages=_lib.MOE_FFN_BOTH,
             ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return _lib.call_status("moe_grouped_ffn_split", *a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(wsb=0), _lib.MOE_ERR_WORKSPACE_TOO_SMALL),
    (dict(ws=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(ws=ctypes.c_void_p(0x1008)), _lib.MOE_ERR_INVALID_ARGUMENT),
    # the checks of moe_grouped_ffn
    (dict(G=0), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(stages=0), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(D=100), _lib.MOE_ERR_UNSUPPORTED),
    (dict(h=None), _lib.MOE_ERR_INVALID_ARGUMENT),
])
def test_grouped_ffn_split_rejects(kw, status):
    ensure_built()
    assert _ffn_split(**kw) == status
    assert _lib.last_error()


def test_grouped_ffn_split_workspace():
    lib = ensure_built()
    n = lib.moe_grouped_ffn_split_workspace_size()
    # header + one 256 x 192 fp32 tile per compute unit (at least 8 CUs)
    assert n >= 3 * 8 * 1024 + 8 * 256 * 192 * 4
    assert (n - 3 * 8 * 1024) % (8 * 256 * 192 * 4) == 0


def test_binding_raises_on_error():
    ensure_built()
    with pytest.raises(_lib.MoEError, match="MOE_ERR_INVALID_ARGUMENT"):
        _lib.call("moe_gate_topk", None, 1, None, None, 1, 8, 8, 2, 0, None,
                  None, None, None, 0, None)


def _hist(**kw):
    a = dict(idx=FAKE, B=4, T=16, E=8, Kmax=2, tags=None, n_tags=0, pos=FAKE,
             tag=None, stream=None)
    a.update(kw)
    return _lib.call_status("moe_routing_histogram", *a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(idx=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(pos=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(B=-1), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(T=0), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(E=0), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(Kmax=0), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(tags=FAKE, n_tags=0, tag=FAKE), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(tags=FAKE, n_tags=10, tag=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(E=65), _lib.MOE_ERR_UNSUPPORTED),
    (dict(Kmax=65), _lib.MOE_ERR_UNSUPPORTED),
    (dict(B=1 << 20, T=1 << 10, Kmax=2), _lib.MOE_ERR_UNSUPPORTED),
])
def test_routing_histogram_rejects(kw, status):
    ensure_built()
    assert _hist(**kw) == status
    assert _lib.last_error()


def _fdc(**kw):
    a = dict(h=FAKE, dt=_lib.MOE_BF16, N=64, D=128, H=256, w2=FAKE, b2=None,
             yr=FAKE, sr=FAKE, w=FAKE, Kmax=2, y=FAKE, stream=None)
    a.update(kw)
    return _lib.call_status("moe_ffn_down_combine", *a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(h=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(sr=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(y=None), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(N=-1), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(Kmax=0), _lib.MOE_ERR_INVALID_ARGUMENT),
    (dict(dt=_lib.MOE_F32), _lib.MOE_ERR_UNSUPPORTED),
    (dict(Kmax=17), _lib.MOE_ERR_UNSUPPORTED),
    (dict(D=100), _lib.MOE_ERR_UNSUPPORTED),
    (dict(N=1 << 31), _lib.MOE_ERR_UNSUPPORTED),
])
def test_ffn_down_combine_rejects(kw, status):
    ensure_built()
    assert _fdc(**kw) == status
    assert _lib.last_error()


def test_backward_entry_points_reject():
    ensure_built()
    lib = _lib.load()
    assert lib.moe_ffn_backward_workspace_size(1000, 8, 128, 256) > 0
    assert lib.moe_ffn_backward_workspace_size(-1, 8, 128, 256) == 0
    assert lib.moe_gate_backward_workspace_size(1000, 8, 128) > 0
    cb = dict(dy=FAKE, dydt=_lib.MOE_BF16, yr=FAKE, ydt=_lib.MOE_BF16, sr=FAKE,
              w=FAKE, N=10, D=64, Kmax=2, dyr=FAKE, sg=FAKE, stream=None)
    for kw, st in [(dict(dy=None), _lib.MOE_ERR_INVALID_ARGUMENT),
                   (dict(sg=None), _lib.MOE_ERR_INVALID_ARGUMENT),
                   (dict(Kmax=0), _lib.MOE_ERR_INVALID_ARGUMENT),
                   (dict(D=60), _lib.MOE_ERR_UNSUPPORTED),
                   (dict(Kmax=65), _lib.MOE_ERR_UNSUPPORTED)]:
        a = dict(cb); a.update(kw)
        assert _lib.call_status("moe_combine_backward", *a.values()) == st
    fb = dict(x=FAKE, ri=None, src=0, dt=_lib.MOE_BF16, total=100, offs=FAKE,
              G=8,
              D=128, H=256, w1=FAKE, b1=None, w2=FAKE, dyr=FAKE, u=None,
              h=None, ws=FAKE, wsb=1 << 40, dx=FAKE, dxdt=_lib.MOE_BF16,
              dw1=FAKE, dw2=FAKE, stream=None)
    for kw, st in [(dict(w1=None), _lib.MOE_ERR_INVALID_ARGUMENT),
                   (dict(dw2=None), _lib.MOE_ERR_INVALID_ARGUMENT),
                   (dict(G=0), _lib.MOE_ERR_INVALID_ARGUMENT),
                   (dict(dt=_lib.MOE_F32), _lib.MOE_ERR_UNSUPPORTED),
                   (dict(G=129), _lib.MOE_ERR_UNSUPPORTED),
                   (dict(H=100), _lib.MOE_ERR_UNSUPPORTED),
                   (dict(total=1 << 31), _lib.MOE_ERR_UNSUPPORTED),
                   # the weight-gradient GEMMs' 32-bit byte offsets:
                   # (total + 64) * max(D, H) * 2 must stay below 2^32
                   (dict(total=(1 << 23) - 64), _lib.MOE_ERR_UNSUPPORTED),
                   (dict(total=(1 << 23) - 65, wsb=16),
                    _lib.MOE_ERR_WORKSPACE_TOO_SMALL),
                   (dict(wsb=16), _lib.MOE_ERR_WORKSPACE_TOO_SMALL),
                   # a group's W2 block is read with 32-bit byte offsets:
                   # D * H * 2 must stay below 2^32
                   (dict(D=1 << 16, H=1 << 15), _lib.MOE_ERR_UNSUPPORTED),
                   (dict(D=1 << 16, H=(1 << 15) - 8, wsb=16),
                    _lib.MOE_ERR_WORKSPACE_TOO_SMALL),
                   (dict(ri=FAKE, src=0), _lib.MOE_ERR_INVALID_ARGUMENT),
                   # D = 128: src <= 2^24 - 2 passes the gather check and
                   # reaches the workspace check
                   (dict(ri=FAKE, src=(1 << 24) - 1),
                    _lib.MOE_ERR_UNSUPPORTED),
                   (dict(ri=FAKE, src=(1 << 24) - 2, wsb=16),
                    _lib.MOE_ERR_WORKSPACE_TOO_SMALL)]:
        a = dict(fb); a.update(kw)
        assert _lib.call_status("moe_grouped_ffn_backward", *a.values()) == st
    gb = dict(x=FAKE, xdt=_lib.MOE_BF16, wg=FAKE, P=FAKE, idx=FAKE, sg=FAKE,
              counts=FAKE, B=2, T=16, D=64, E=8, Kmax=2, K=2, alpha=0.01,
              dloss=1.0, mode=_lib.MOE_BAL_PER_SEQUENCE, dxr=None, sr=None,
              dxs=None, dxdt=_lib.MOE_BF16, dx=FAKE, dwg=FAKE, db=None,
              ws=FAKE, wsb=1 << 30, stream=None)
    for kw, st in [(dict(wg=None), _lib.MOE_ERR_INVALID_ARGUMENT),
                   (dict(counts=None), _lib.MOE_ERR_INVALID_ARGUMENT),
                   (dict(K=9), _lib.MOE_ERR_INVALID_ARGUMENT),
                   (dict(mode=5), _lib.MOE_ERR_INVALID_ARGUMENT),
                   (dict(dxr=FAKE), _lib.MOE_ERR_INVALID_ARGUMENT),
                   (dict(E=65, K=2), _lib.MOE_ERR_UNSUPPORTED),
                   (dict(D=60), _lib.MOE_ERR_UNSUPPORTED),
                   (dict(wsb=8), _lib.MOE_ERR_WORKSPACE_TOO_SMALL)]:
        a = dict(gb); a.update(kw)
        assert _lib.call_status("moe_gate_backward", *a.values()) == st
