"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects invalid arguments on the host before any HIP call.

Only argument combinations that fail validation are passed here; the fake
device pointers are never dereferenced.
"""

import ctypes
import os
import re
import subprocess

import pytest

import vision_transformer_dynamic_amd as bra
from vision_transformer_dynamic_amd import build as bra_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bra.h")

EINVAL, EUNSUP = bra.BRA_EINVAL, bra.BRA_EUNSUPPORTED
P = 0x10000  # aligned fake device pointers (never dereferenced)
P2, P3, P4, PW = 0x20000, 0x30000, 0x40000, 0x50000
PF, PB = 0x60000, 0x70000  # local-context filter weight and bias
WS = 0x1000000  # workspace (1 MiB by default), clear of every tensor above
# Maps of the default shape (1 x 16 x 16 x 32 fp32) are 32 KiB; the fake
# pointers are 64 KiB apart, so offsets below place one tensor partly inside
# another.
MAP = 16 * 16 * 32 * 4


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bra.library_path()):
        bra_build.build()
    return bra.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bra_[a-z_]+)\s*\(", text)))


def test_header_declares_exactly_the_binding_exports():
    assert _declared_functions() == sorted(bra.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", bra.library_path()],
                         stdout=subprocess.PIPE, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (bra_[a-z_]+)$", out, flags=re.M))
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings(lib):
    for code in range(6):
        s = lib.bra_status_string(code)
        assert isinstance(s, bytes) and len(s) > 3
    assert lib.bra_status_string(0) == b"success"
    assert lib.bra_status_string(99) == b"unknown status"


def test_workspace_bytes(lib):
    # [Qr | Kr | idx], each rounded up to 256 bytes
    B, H, W, C, S, k = 64, 56, 56, 64, 7, 1
    pooled = 4 * B * 49 * C
    idx = -(-4 * B * 49 * k // 256) * 256
    assert lib.bra_workspace_bytes(B, H, W, C, S, k) == 2 * pooled + idx
    assert lib.bra_workspace_bytes(1, 16, 16, 32, 4, 2) == 2 * 2048 + 256
    assert lib.bra_workspace_bytes(1, 16, 16, 32, 5, 2) == 0  # S does not divide H
    assert lib.bra_workspace_bytes(1, 16, 16, 32, 4, 17) == 0  # topk > S*S


def _fwd(lib, B=1, H=16, W=16, C=32, heads=1, S=4, k=2, dt=0, q=P, kk=P2, v=P3, o=P4, ws=WS, wsb=1 << 20):
    return lib.bra_forward_ws(q, kk, v, o, B, H, W, C, heads, S, k, dt, ws, wsb, None)


def _route(lib, B=1, H=16, W=16, C=32, S=4, k=2, dt=0, q=P, kk=P2, idx=P3, ws=WS, wsb=1 << 20):
    return lib.bra_route_ws(q, kk, idx, B, H, W, C, S, k, dt, ws, wsb, None)


# the forms without a workspace argument (they would allocate one: only calls
# that fail validation, before any HIP call, are made here)
def _fwd_alloc(lib, B=1, H=16, W=16, C=32, heads=1, S=4, k=2, dt=0, q=P, kk=P2, v=P3, o=P4):
    return lib.bra_forward(q, kk, v, o, B, H, W, C, heads, S, k, dt, None)


def _route_alloc(lib, B=1, H=16, W=16, C=32, S=4, k=2, dt=0, q=P, kk=P2, idx=P3):
    return lib.bra_route(q, kk, idx, B, H, W, C, S, k, dt, None)


def _attend(lib, B=1, H=16, W=16, C=32, heads=1, S=4, k=2, dt=0, q=P, kk=P2, v=P3, idx=P4, o=PW):
    return lib.bra_attend(q, kk, v, idx, o, B, H, W, C, heads, S, k, dt, None)


def _fwd_lce(lib, B=1, H=16, W=16, C=32, heads=1, S=4, k=2, dt=0, q=P, kk=P2, v=P3, o=P4, ws=WS, wsb=1 << 20,
             wt=PF, bias=PB):
    return lib.bra_forward_lce(q, kk, v, wt, bias, o, B, H, W, C, heads, S, k, dt, ws, wsb, None)


def _attend_lce(lib, B=1, H=16, W=16, C=32, heads=1, S=4, k=2, dt=0, q=P, kk=P2, v=P3, idx=P4, o=PW, wt=PF,
                bias=PB):
    return lib.bra_attend_lce(q, kk, v, idx, wt, bias, o, B, H, W, C, heads, S, k, dt, None)


def _bwd(lib, B=1, H=16, W=16, C=32, heads=1, S=4, k=2, dt=0, q=P, kk=P2, v=P3, o=P4, do=PF, idx=PB,
         dq=0x80000, dk=0x90000, dv=0xA0000, ws=WS, wsb=1 << 20):
    return lib.bra_attend_backward(q, kk, v, o, do, idx, dq, dk, dv, B, H, W, C, heads, S, k, dt, ws, wsb, None)


@pytest.mark.parametrize("call", [_fwd, _route, _fwd_alloc, _route_alloc, _attend, _fwd_lce, _attend_lce, _bwd])
@pytest.mark.parametrize(
    "kwargs,status",
    [
        (dict(H=18), EINVAL),            # S does not divide H
        (dict(W=10), EINVAL),            # S does not divide W
        (dict(k=0), EINVAL),
        (dict(k=17), EINVAL),            # topk > S*S
        (dict(B=0), EINVAL),
        (dict(C=-32), EINVAL),
        (dict(S=0), EINVAL),
        (dict(q=0), EINVAL),             # null pointer
        (dict(q=P + 2), EINVAL),         # misaligned pointer
        (dict(kk=0), EINVAL),
        (dict(dt=7), EUNSUP),            # unknown dtype
        (dict(S=17, H=17, W=17), EUNSUP),  # 289 regions
        (dict(C=36), EUNSUP),            # C not a multiple of 8 (route) / d != 32
    ],
)
def test_host_validation(lib, call, kwargs, status):
    assert call(lib, **kwargs) == status


@pytest.mark.parametrize("call", [_fwd, _fwd_alloc, _attend, _fwd_lce, _attend_lce, _bwd])
@pytest.mark.parametrize(
    "kwargs,status",
    [
        (dict(heads=3), EINVAL),         # heads does not divide C
        (dict(heads=0), EINVAL),
        (dict(C=64, heads=1), EUNSUP),   # head dim 64
        (dict(C=64, heads=4), EUNSUP),   # head dim 16
        (dict(v=0), EINVAL),
        (dict(o=P), EINVAL),             # output aliases Q
    ],
)
def test_host_validation_heads_and_outputs(lib, call, kwargs, status):
    if call is _bwd and "o" in kwargs:
        kwargs = dict(dq=kwargs["o"])  # the backward's o is an input: alias an output instead
    assert call(lib, **kwargs) == status


def test_attend_null_index_table(lib):
    assert _attend(lib, idx=0) == EINVAL
    assert _attend(lib, idx=P4 + 2) == EINVAL
    assert _attend_lce(lib, idx=0) == EINVAL


@pytest.mark.parametrize("call", [_fwd_lce, _attend_lce])
@pytest.mark.parametrize(
    "kwargs",
    [
        dict(wt=0),                      # the filter is required
        dict(wt=PF + 2),                 # weight not 4-byte aligned
        dict(bias=PB + 2),               # fp32 bias not element aligned
        dict(dt=1, bias=PB + 1),         # bf16 bias not element aligned
        dict(wt=0x40010, o=0x40000),     # weight inside O
        dict(bias=0x40100, o=0x40000),   # bias inside O
        dict(wt=0x40000 - 64, o=0x40000),  # weight runs into O
    ],
)
def test_lce_filter_validation(lib, call, kwargs):
    assert call(lib, **kwargs) == EINVAL


def _qkv(lib, B=1, H=16, W=16, C=32, S=4, dt=0, x=P, w=P2, b=0, q=P3, k=P4, v=PW, qr=PF, kr=PB):
    return lib.bra_qkv_pool(x, w, b, q, k, v, qr, kr, B, H, W, C, S, dt, None)


def _fqkv(lib, B=1, H=16, W=16, C=32, heads=1, S=4, k=2, dt=0, x=P, w=P2, b=0, q=P3, kk=P4, v=PW, o=PF,
          ws=WS, wsb=1 << 20):
    return lib.bra_forward_qkv(x, w, b, q, kk, v, o, B, H, W, C, heads, S, k, dt, ws, wsb, None)


@pytest.mark.parametrize("call", [_qkv, _fqkv])
@pytest.mark.parametrize(
    "kwargs,status",
    [
        (dict(C=40), EUNSUP),             # C not a multiple of 32
        (dict(C=512, H=8, W=8, S=2), EUNSUP),  # C above the projection's limit
        (dict(C=256, H=8, W=8, S=2), EUNSUP),  # fp32 above 128
        (dict(x=0), EINVAL),
        (dict(x=P + 8), EINVAL),          # misaligned input
        (dict(w=P2 + 4), EINVAL),         # misaligned weight
        (dict(b=PB + 2), EINVAL),         # misaligned fp32 bias
        (dict(q=P), EINVAL),              # output aliases the input
        (dict(q=P2), EINVAL),             # output overlaps the weight
        (dict(S=5), EINVAL),
        (dict(dt=3), EUNSUP),
    ],
)
def test_projection_validation(lib, call, kwargs, status):
    if call is _fqkv and "C" in kwargs and kwargs["C"] in (256, 512):
        kwargs = dict(kwargs, heads=kwargs["C"] // 32)
    assert call(lib, **kwargs) == status


def test_projection_pooled_outputs_validation(lib):
    assert _qkv(lib, qr=0) == EINVAL
    assert _qkv(lib, kr=PF + 64) == EINVAL  # region means overlap
    assert _qkv(lib, qr=0x90004) == EINVAL  # region means not 16-byte aligned
    assert _fqkv(lib, o=P3) == EINVAL       # O aliases Q
    assert _fqkv(lib, wsb=16) == EINVAL


@pytest.mark.parametrize("kwargs", [dict(dq=P), dict(dk=P3), dict(dv=PF), dict(dq=0x90000), dict(dk=0xA0000),
                                    dict(do=0), dict(idx=0), dict(idx=PB + 2), dict(dv=0xA0000 + 8),
                                    dict(dq=P + 256), dict(dk=0x80000 + MAP - 16), dict(dv=PF + 16)])
def test_backward_validation(lib, kwargs):
    assert _bwd(lib, **kwargs) == EINVAL


def test_backward_workspace_bytes(lib):
    B, H, W, C, heads, S, k = 2, 16, 16, 64, 2, 4, 2
    tok = B * H * W * heads
    up = lambda x: -(-x // 256) * 256
    assert lib.bra_backward_workspace_bytes(B, H, W, C, heads, S, k) == 2 * up(4 * tok) + 3 * up(4 * B * 16) + up(4 * B * 16 * 16)
    assert lib.bra_backward_workspace_bytes(B, H, W, C, 0, S, k) == 0
    assert lib.bra_backward_workspace_bytes(B, H, W, C, 3, S, k) == 0


@pytest.mark.parametrize("call", [_fwd, _route, _fwd_lce, _bwd])
def test_workspace_validation(lib, call):
    assert call(lib, wsb=16) == EINVAL           # too small
    assert call(lib, ws=WS + 64) == EINVAL       # not 256-byte aligned
    assert call(lib, ws=0, wsb=16) == EINVAL     # size without a buffer
    assert call(lib, ws=P2 - 256) == EINVAL      # workspace runs into K (1 MiB from 0x1ff00)


@pytest.mark.parametrize("call", [_fwd, _route])
def test_workspace_forms_need_a_workspace(lib, call):
    # the *_ws entry points never allocate: no buffer is an error
    assert call(lib, ws=0, wsb=0) == EINVAL



@pytest.mark.parametrize("call", [_fwd, _fwd_alloc, _attend, _fwd_lce, _attend_lce])
@pytest.mark.parametrize("o", [P + 16, P2 + MAP - 16, P3 - MAP + 16])
def test_output_may_not_partly_overlap_inputs(lib, call, o):
    assert call(lib, o=o) == EINVAL


def test_index_table_may_not_overlap_output_or_inputs(lib):
    assert _attend(lib, idx=PW + 64) == EINVAL          # idx inside O
    assert _attend_lce(lib, idx=PW + 64) == EINVAL
    assert _route(lib, idx=P + 64) == EINVAL            # idx inside Q
    assert _route_alloc(lib, idx=P2 + 1024) == EINVAL   # idx inside K
    assert _bwd(lib, idx=0x80000 + 64) == EINVAL        # idx inside dQ


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(bra, "_lib", None)
    monkeypatch.setenv("BRA_LIBRARY", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="not built"):
        bra.load_library()


def _fwd_static(lib, B=1, H=16, W=16, C=32, heads=1, S=4, k=2, dt=0, q=P, kk=P2, v=P3, o=P4):
    return lib.bra_forward_static(q, kk, v, o, B, H, W, C, heads, S, k, dt, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(H=18), EINVAL), (dict(k=0), EINVAL), (dict(q=0), EINVAL), (dict(o=P + 2), EINVAL),
    (dict(heads=3), EINVAL), (dict(C=64, heads=1), EUNSUP), (dict(dt=7), EUNSUP),
])
def test_static_entry_point_validation(lib, kwargs, status):
    assert _fwd_static(lib, **kwargs) == status


def test_static_entry_point_rejects_sizes_beyond_its_buffer(lib):
    # 1024 images of 56 x 56 x 64 at S = 7: 25.7 MB of region means
    assert lib.bra_workspace_bytes(1024, 56, 56, 64, 7, 1) > bra.STATIC_SCRATCH_BYTES
    assert _fwd_static(lib, B=1024, H=56, W=56, C=64, heads=2, S=7, k=1, dt=1) == bra.BRA_ESCRATCH
    assert lib.bra_workspace_bytes(512, 56, 56, 64, 7, 1) <= bra.STATIC_SCRATCH_BYTES
