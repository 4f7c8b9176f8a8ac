"""The C-ABI library on a host without a GPU: it loads, exports every entry point that
include/gdr2.h declares, answers the size queries, and rejects invalid arguments on the host
before any launch (no GPU call is made by any test here)."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_gdr_amd import library_path, load_library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr2.h")

NULL = None
OK, E_NULL, E_SHAPE, E_DTYPE, E_UNSUP, E_ALIGN, E_ALIAS, E_WS = 0, 1, 2, 3, 4, 5, 6, 7


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr2_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    assert os.path.exists(library_path()), "build the library first (gated_delta_rule_gdr_amd/build.py)"
    lib = load_library()
    names = declared_functions()
    assert "gdr2_fwd_chunked" in names and "gdr2_bwd_chunked" in names and "gdr2_decode_step" in names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in gdr2.h but not exported"


def test_version_and_strings():
    lib = load_library()
    assert lib.gdr2_abi_version() == 4
    for s in range(11):
        assert lib.gdr2_status_string(s) and lib.gdr2_status_string(s) != b"unknown status"
    assert lib.gdr2_dtype_size(0) == 4 and lib.gdr2_dtype_size(1) == 2 and lib.gdr2_dtype_size(7) == 0
    assert lib.gdr2_num_chunks(0) == 0 and lib.gdr2_num_chunks(1) == 1 and lib.gdr2_num_chunks(64) == 1
    assert lib.gdr2_num_chunks(65) == 2


def test_workspace_sizes():
    lib = load_library()
    B, T, H, dk, dv = 4, 4096, 16, 128, 128
    nc = 64
    per = B * H * nc
    fws = lib.gdr2_fwd_workspace_bytes(B, T, H, dk, dv, 1)
    # -Y, Qbar, Ktilde [64][dk]; P, T [64][64]; U [64][dv] in bf16; gamma fp32; states [dv][dk] bf16
    expect = per * (3 * 64 * dk * 2 + 2 * 64 * 64 * 2 + 64 * dv * 2 + dk * 4 + dv * dk * 2)
    assert fws == expect
    assert lib.gdr2_bwd_workspace_bytes(B, T, H, dk, dv, 1) == per * dk * dv * 2
    assert lib.gdr2_fwd_workspace_bytes(1, 0, 1, 64, 64, 0) == 0


def test_forward_only_and_recompute_workspace_sizes():
    """The forward-only workspace is the training forward's without the chunk-entry states; the
    recomputing backward needs the training forward's workspace followed by the backward's."""
    lib = load_library()
    for (B, T, H, dk, dv, dt) in [(4, 4096, 16, 128, 128, 1), (1, 100, 3, 64, 128, 0), (2, 1, 1, 64, 64, 1)]:
        per = B * H * ((T + 63) // 64)
        es = 2 if dt == 1 else 4
        r = lambda n: (n + 255) // 256 * 256
        fws = lib.gdr2_fwd_workspace_bytes(B, T, H, dk, dv, dt)
        inf = lib.gdr2_fwd_infer_workspace_bytes(B, T, H, dk, dv, dt)
        assert fws - inf == r(per * dv * dk * es)
        assert lib.gdr2_bwd_recompute_workspace_bytes(B, T, H, dk, dv, dt) == fws + lib.gdr2_bwd_workspace_bytes(B, T, H, dk, dv, dt)


def test_sizes_that_would_overflow_are_rejected():
    """Shape products are bounded before they are formed: sizes whose products overflow 64 bits
    get GDR2_E_SHAPE (and workspace queries 0) instead of wrapping around."""
    lib = load_library()
    P = lambda a: _fake(a)
    big = 1 << 40
    ins = [P(0x10000 + i * 0x8000) for i in range(6)]
    for (B, T, H) in [(big, 8, big), (1 << 31, 8, 1 << 31), (1, 1 << 41, 1), (1 << 20, 1 << 30, 1),
                      (big, big, big), ((1 << 62), 1, 4)]:
        assert lib.gdr2_fwd_workspace_bytes(B, T, H, 128, 128, 1) == 0
        assert lib.gdr2_fwd_infer_workspace_bytes(B, T, H, 128, 128, 1) == 0
        assert lib.gdr2_bwd_workspace_bytes(B, T, H, 128, 128, 1) == 0
        assert lib.gdr2_bwd_recompute_workspace_bytes(B, T, H, 128, 128, 1) == 0
        assert lib.gdr2_fwd_chunked(B, T, H, 128, 128, 1, *ins, NULL, P(0x90000), NULL,
                                    P(0x200000), 1 << 30, NULL) == E_SHAPE
        assert lib.gdr2_fwd_infer(B, T, H, 128, 128, 1, *ins, NULL, P(0x90000), NULL,
                                  P(0x200000), 1 << 30, NULL) == E_SHAPE
        assert lib.gdr2_bwd_chunked_recompute(B, T, H, 128, 128, 1, *ins, NULL, P(0x300000), NULL,
                                              *[P(0x400000 + i * 0x1000) for i in range(6)], NULL,
                                              P(0x500000), 1 << 30, NULL) == E_SHAPE
    assert lib.gdr2_decode_step(big, big, 64, 64, 1, *ins, NULL, P(0x100000), P(0x200000), NULL) == E_SHAPE
    assert lib.gdr2_decode_step(1 << 16, 1 << 15, 64, 64, 1, *ins, NULL, P(0x100000), P(0x200000), NULL) == E_SHAPE


def test_forward_only_rejects_before_launch():
    lib = load_library()
    P = lambda a: _fake(a)
    B, T, H, dk, dv = 1, 8, 1, 64, 64
    need = lib.gdr2_fwd_infer_workspace_bytes(B, T, H, dk, dv, 1)

    def call(dt=1, q=0x10000, o=0x90000, ws=0x200000, wsb=1 << 30, gates=0):
        ins = [P(q + i * 0x8000) if q else NULL for i in range(6)]
        return lib.gdr2_fwd_infer_ex(B, T, H, dk, dv, dt, gates, NULL, *ins, NULL, P(o) if o else NULL,
                                     NULL, P(ws) if ws else NULL, wsb, NULL)
    assert call(dt=3) == E_DTYPE
    assert call(gates=8) == E_UNSUP
    assert call(q=0) == E_NULL
    assert call(o=0) == E_NULL
    assert call(ws=0) == E_WS
    assert call(wsb=need - 1) == E_WS
    assert call(o=0x10008) == E_ALIGN
    assert call(o=0x18000) == E_ALIAS
    # the overlap test covers the forward-only workspace's own extent: ending 64 bytes into w
    assert call(ws=0x10000 + 5 * 0x8000 + 64 - need) == E_ALIAS


def test_recompute_backward_rejects_before_launch():
    from gated_delta_rule_gdr_amd import Prologue
    lib = load_library()
    P = lambda a: _fake(a)
    B, T, H, dk, dv = 1, 8, 1, 64, 64
    need = lib.gdr2_bwd_recompute_workspace_bytes(B, T, H, dk, dv, 1)
    ins = [P(0x10000 + i * 0x8000) for i in range(6)]

    def call(dt=1, S0=0, dO=0x300000, dq=0x400000, ws=0x900000, wsb=1 << 30, pro=None, gates=0):
        grads = [P(dq + i * 0x8000) if dq else NULL for i in range(6)]
        return lib.gdr2_bwd_chunked_recompute_ex(B, T, H, dk, dv, dt, gates, pro, *ins,
                                                 P(S0) if S0 else NULL, P(dO) if dO else NULL, NULL,
                                                 *grads, NULL, P(ws) if ws else NULL, wsb, NULL)
    assert call(dt=7) == E_DTYPE
    assert call(gates=16) == E_UNSUP
    assert call(pro=ctypes.byref(Prologue(0.0, 1e-6))) == 9
    assert call(dO=0) == E_NULL
    assert call(dq=0) == E_NULL
    assert call(ws=0) == E_WS
    assert call(wsb=need - 1) == E_WS
    assert call(S0=0x300008) == E_ALIGN
    assert call(dq=0x10000) == E_ALIAS
    assert call(ws=0x300000) == E_ALIAS      # workspace over dO
    assert call(S0=0x400000) == E_ALIAS      # an input under the gradient outputs


def test_noalloc_entry_point_rejects_before_launch():
    """The no-allocation forward-only call validates like gdr2_fwd_infer_ex (no workspace
    argument) and rejects problems whose factors exceed its static scratch with GDR2_E_TOO_LARGE;
    none of these calls reaches the device."""
    lib = load_library()
    P = lambda a: _fake(a)
    cap = lib.gdr2_fwd_infer_noalloc_max_bytes()
    assert cap == 128 << 20
    ins = [P(0x10000 + i * 0x8000) for i in range(6)]

    def call(B=1, T=8, H=1, dk=64, dv=64, dt=1, o=0x90000, gates=0, pro=None):
        return lib.gdr2_fwd_infer_noalloc_ex(B, T, H, dk, dv, dt, gates, pro, *ins, NULL,
                                             P(o) if o else NULL, NULL, NULL)
    assert call(dt=2) == E_DTYPE
    assert call(dk=32) == E_UNSUP
    assert call(gates=9) == E_UNSUP
    assert call(o=0) == E_NULL
    assert call(o=0x90008) == E_ALIGN
    assert call(o=0x10000) == E_ALIAS
    from gated_delta_rule_gdr_amd import Prologue
    assert call(pro=ctypes.byref(Prologue(1.0, 0.0))) == 9
    # largest sequence whose factors fit, and the next chunk over the limit (B = 1, H = 32, d = 128,
    # bf16: enough chains that the forward is not pipelined, so the forward-only workspace is
    # exactly the factors)
    per_chunk = lib.gdr2_fwd_infer_workspace_bytes(1, 64, 32, 128, 128, 1)
    n = cap // per_chunk
    while lib.gdr2_fwd_infer_workspace_bytes(1, 64 * n, 32, 128, 128, 1) > cap:
        n -= 1
    assert lib.gdr2_fwd_infer_workspace_bytes(1, 64 * (n + 1), 32, 128, 128, 1) > cap
    far = lambda T, H=32: lib.gdr2_fwd_infer_noalloc_ex(1, T, H, 128, 128, 1, 0, NULL,
                                                        *[P(0x100000000 * (i + 1)) for i in range(6)],
                                                        NULL, P(0x1000000000), NULL, NULL)
    assert far(64 * (n + 1)) == 10
    assert far(64 * n + 65) == 10
    # a pipelined shape (one chain, many chunks): the limit is on the factors alone, not on the
    # forward-only workspace, which also holds the fp32 hand-off buffer of one d x d state
    per_chunk1 = lib.gdr2_fwd_infer_workspace_bytes(1, 64, 1, 128, 128, 1)  # one chunk: not pipelined
    m = cap // per_chunk1
    assert lib.gdr2_fwd_infer_workspace_bytes(1, 64 * m, 1, 128, 128, 1) == m * per_chunk1 + 128 * 128 * 4
    assert far(64 * (m + 1), H=1) == 10
    assert far(64 * m, H=1) != 10


def _fake(addr):
    """A non-null, 16-byte aligned address that is never dereferenced (validation fails first)."""
    return ctypes.c_void_p(addr)


def _fwd(lib, B=1, T=8, H=1, dk=64, dv=64, dt=1, q=0x10000, o=0x90000, ws=0x200000, ws_bytes=1 << 30,
         stride=0x8000, S0=None, ST=None):
    ptrs = [_fake(q + i * stride) if q else NULL for i in range(6)]
    return lib.gdr2_fwd_chunked(B, T, H, dk, dv, dt, *ptrs, S0, _fake(o) if o else NULL, ST,
                                _fake(ws) if ws else NULL, ws_bytes, NULL)


def test_fwd_rejects_before_launch():
    lib = load_library()
    assert _fwd(lib, dt=5) == E_DTYPE
    assert _fwd(lib, T=-1) == E_SHAPE
    assert _fwd(lib, dk=96) == E_UNSUP
    assert _fwd(lib, dv=256) == E_UNSUP
    assert _fwd(lib, q=0) == E_NULL
    assert _fwd(lib, o=0) == E_NULL
    assert _fwd(lib, ws=0) == E_WS
    assert _fwd(lib, ws_bytes=16) == E_WS
    assert _fwd(lib, q=0x10004) == E_ALIGN
    assert _fwd(lib, o=0x10000) == E_ALIAS            # output on top of q
    assert _fwd(lib, ws=0x10000) == E_ALIAS           # workspace on top of the inputs
    assert _fwd(lib, B=0) == OK                         # nothing to do, nothing launched
    assert _fwd(lib, H=0) == OK


def test_bwd_rejects_before_launch():
    lib = load_library()
    P = lambda a: _fake(a)
    base = [P(0x10000 + i * 0x8000) for i in range(6)]

    def call(dt=1, fws=0x400000, dO=0x300000, dq=0x500000, ws=0x900000, ws_bytes=1 << 30, fws_bytes=1 << 30):
        grads = [P(dq + i * 0x8000) if dq else NULL for i in range(6)]
        return lib.gdr2_bwd_chunked(1, 8, 1, 64, 64, dt, *base, P(fws) if fws else NULL, fws_bytes,
                                    P(dO) if dO else NULL, NULL, grads[0], grads[1], grads[2],
                                    grads[3], grads[4], grads[5], NULL, P(ws) if ws else NULL,
                                    ws_bytes, NULL)
    assert call(dt=9) == E_DTYPE
    assert call(fws=0) == E_NULL
    assert call(dO=0) == E_NULL
    assert call(dq=0) == E_NULL
    assert call(ws=0) == E_WS
    assert call(fws_bytes=8) == E_WS
    assert call(dq=0x10000) == E_ALIAS
    assert call(ws=0x300000) == E_ALIAS


def test_decode_rejects_before_launch():
    lib = load_library()
    P = lambda a: _fake(a)
    ins = [P(0x10000 + i * 0x1000) for i in range(6)]
    assert lib.gdr2_decode_step(2, 2, 64, 64, 3, *ins, NULL, P(0x100000), P(0x200000), NULL) == E_DTYPE
    assert lib.gdr2_decode_step(2, 2, 64, 80, 1, *ins, NULL, P(0x100000), P(0x200000), NULL) == E_UNSUP
    assert lib.gdr2_decode_step(2, 2, 64, 64, 1, *ins, NULL, NULL, P(0x200000), NULL) == E_NULL
    assert lib.gdr2_decode_step(2, 2, 64, 64, 1, *ins, NULL, P(0x100008), P(0x200000), NULL) == E_ALIGN
    assert lib.gdr2_decode_step(2, 2, 64, 64, 1, *ins, NULL, P(0x10000), P(0x200000), NULL) == E_ALIAS
    # S_in may equal S_out exactly, but may not partially overlap it
    assert lib.gdr2_decode_step(2, 2, 64, 64, 1, *ins, P(0x100010), P(0x100000), P(0x200000), NULL) == E_ALIAS
    assert lib.gdr2_decode_step(0, 2, 64, 64, 1, *ins, NULL, P(0x100000), P(0x200000), NULL) == OK


def test_gate_shape_entry_points_validate():
    """The *_ex entry points: unknown gate bits are rejected; a channel-wise gate's extent is
    checked for overlap, and a scalar gate's smaller extent still is (every call here fails
    validation, so nothing is launched)."""
    lib = load_library()
    P = lambda a: _fake(a)
    B, T, H, dk, dv = 1, 8, 1, 64, 64

    def fwd(gates, b=0x18000, o=0x90000):
        ins = [P(0x10000), P(0x20000), P(0x30000), P(0x40000), P(b), P(0x60000)]
        return lib.gdr2_fwd_chunked_ex(B, T, H, dk, dv, 1, gates, NULL, *ins, NULL, P(o), NULL,
                                       P(0x200000), 1 << 30, NULL)
    assert fwd(8) == E_UNSUP
    assert fwd(1 << 31) == E_UNSUP
    # channel-wise b spans 8 x 64 bf16 = 1 KB from 0x18000: o at 0x18010 overlaps it
    assert fwd(0, b=0x18000, o=0x18010) == E_ALIAS
    # scalar b spans 16 bytes: o at 0x18000 still overlaps it
    assert fwd(1, b=0x18000, o=0x18000) == E_ALIAS
    # decode with every gate scalar: rejects bad bits, accepts the sizes
    ins = [P(0x10000 + i * 0x1000) for i in range(6)]
    assert lib.gdr2_decode_step_ex(2, 2, 64, 64, 1, 16, NULL, *ins, NULL, P(0x100000), P(0x200000), NULL) == E_UNSUP
    assert lib.gdr2_decode_step_ex(2, 2, 64, 64, 1, 7, NULL, *ins, NULL, P(0x10008), P(0x200000), NULL) == E_ALIGN


def test_prologue_parameters_validated_before_launch():
    """A fused-prologue parameter block with a non-positive or non-finite member is rejected with
    GDR2_E_VALUE by every *_ex entry point (otherwise valid calls, so the prologue check is what
    stops them; nothing is launched)."""
    from gated_delta_rule_gdr_amd import Prologue
    lib = load_library()
    P = lambda a: _fake(a)
    B, T, H, dk, dv = 1, 8, 1, 64, 64
    ins = [P(0x10000 + i * 0x1000) for i in range(6)]
    bad = [Prologue(0.0, 1e-6), Prologue(-1.0, 1e-6), Prologue(1.0, 0.0), Prologue(1.0, -1.0),
           Prologue(float("nan"), 1e-6), Prologue(1.0, float("inf"))]
    for pro in bad:
        r = ctypes.byref(pro)
        assert lib.gdr2_fwd_chunked_ex(B, T, H, dk, dv, 1, 0, r, *ins, NULL, P(0x90000), NULL,
                                       P(0x200000), 1 << 30, NULL) == 9
        assert lib.gdr2_fwd_factors_ex(B, T, H, dk, dv, 1, 0, r, *ins, P(0x200000), 1 << 30,
                                       NULL) == 9
        assert lib.gdr2_bwd_grads_ex(B, T, H, dk, dv, 1, 0, r, *ins, P(0x200000), 1 << 30,
                                     P(0x300000), *[P(0x400000 + i * 0x1000) for i in range(6)],
                                     P(0x500000), 1 << 30, NULL) == 9
        assert lib.gdr2_bwd_chunked_ex(B, T, H, dk, dv, 1, 0, r, *ins, P(0x200000), 1 << 30,
                                       P(0x300000), NULL,
                                       *[P(0x400000 + i * 0x1000) for i in range(6)], NULL,
                                       P(0x500000), 1 << 30, NULL) == 9
        assert lib.gdr2_decode_step_ex(2, 2, 64, 64, 1, 0, r, *ins, NULL, P(0x100000),
                                       P(0x200000), NULL) == 9


def test_out_gate_rejects_before_launch():
    lib = load_library()
    P = lambda a: _fake(a)
    F = ctypes.c_float
    fwd = lambda rows=64, dv=128, dt=1, eps=1e-6, o=0x10000, y=0x90000: lib.gdr2_out_gate_fwd(
        rows, dv, dt, P(o) if o else NULL, P(0x30000), P(0x50000), F(eps), P(y), NULL)
    assert fwd(dt=4) == E_DTYPE
    assert fwd(dv=96) == E_UNSUP
    assert fwd(eps=0.0) == 9 and fwd(eps=-1.0) == 9 and fwd(eps=float("nan")) == 9
    assert fwd(o=0) == E_NULL
    assert fwd(o=0x10008) == E_ALIGN
    assert fwd(y=0x30000) == E_ALIAS
    assert fwd(rows=0) == OK
    # one workgroup per 128 rows: beyond 2^37 rows the grid would not fit a launch
    assert fwd(rows=-1) == E_SHAPE and fwd(rows=(1 << 37) + 1) == E_SHAPE
    assert lib.gdr2_out_gate_bwd_workspace_bytes(1 << 18, 128) > 0
    bwd = lambda ws=0x400000, wsb=1 << 30, dw=0x200000: lib.gdr2_out_gate_bwd(
        64, 128, 1, P(0x10000), P(0x30000), P(0x50000), F(1e-6), P(0x60000), P(0x70000),
        P(0x80000), P(dw) if dw else NULL, P(ws) if ws else NULL, wsb, NULL)
    assert bwd(dw=0) == E_NULL
    assert bwd(ws=0) == E_WS
    assert bwd(wsb=4) == E_WS
    assert bwd(dw=0x10000) == E_ALIAS
