"""The boundary's calling conventions on the GPU: every call is queued on the caller's current
stream (here a side stream, with other work queued on the default stream meanwhile), and any
16-byte-aligned, contiguous buffer is accepted (inputs as views at a 16-byte offset into larger
allocations).  Both must give results bitwise identical to the plain call."""
import pytest
import torch

from gated_delta_rule_gdr_amd import gdr2_bwd_chunked, gdr2_decode_step, gdr2_fwd_chunked
from gated_delta_rule_gdr_amd.inputs import decode_inputs, layer_inputs
from tests._util import announce

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NAMES = ("q", "k", "v", "log_alpha", "b", "w")
GRADS = ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0")


def _gpu(x):
    return {n: (None if t is None else t.to(DEV)) for n, t in x.items()}


def _layer(g):
    o, ST, ws = gdr2_fwd_chunked(*(g[n] for n in NAMES), S0=g["S0"])
    gr = gdr2_bwd_chunked(*(g[n] for n in NAMES), g["dO"], ws, dS_T=g.get("dST"))
    return o, ST, gr


def _same(a, b):
    o, ST, gr = a
    o2, ST2, gr2 = b
    assert torch.equal(o, o2) and torch.equal(ST, ST2)
    for n in GRADS:
        assert torch.equal(gr[n], gr2[n]), n


def _offset_copy(t, nbytes=16):
    """A contiguous copy of t that starts nbytes into a larger allocation."""
    if t is None:
        return None
    pad = nbytes // t.element_size()
    buf = torch.zeros(t.numel() + pad, dtype=t.dtype, device=t.device)
    view = buf[pad:].view(t.shape)
    view.copy_(t)
    assert view.is_contiguous() and view.data_ptr() % 256 == nbytes % 256
    return view


def test_layer_on_a_side_stream():
    x = _gpu(layer_inputs(2, 200, 4, 128, 128, dtype="bf16", seed=61, s0_std=0.05, dST=True))
    announce("forward + backward on a side stream")
    ref = _layer(x)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    busy = torch.randn(2048, 2048, device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = _layer(x)
    for _ in range(4):  # unrelated work on the default stream meanwhile
        busy = busy @ busy.T.contiguous() * 1e-3
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    _same(ref, got)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_layer_on_offset_buffers(dtype, d):
    x = _gpu(layer_inputs(1, 130, 3, d, d, dtype=dtype, seed=62, s0_std=0.05, dST=True))
    announce(f"forward + backward on 16-byte-offset buffers {dtype} d={d}")
    ref = _layer(x)
    got = _layer({n: _offset_copy(t) for n, t in x.items()})
    torch.cuda.synchronize()
    _same(ref, got)


def test_decode_on_offset_buffers_and_side_stream():
    tok = _gpu(decode_inputs(0, N=8, H=4, dk=128, dv=128, dtype="bf16", seed_base=63))
    S0 = torch.randn(8, 4, 128, 128, device=DEV) * 0.02
    announce("decode on offset buffers and a side stream")
    o_ref, S_ref = gdr2_decode_step(*(tok[n] for n in NAMES), S_in=S0.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        S = _offset_copy(S0)
        o, S = gdr2_decode_step(*(_offset_copy(tok[n]) for n in NAMES), S_in=S, S_out=S)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)


@pytest.mark.parametrize("B,T,H,d,pro,scalar", [
    (4, 4096, 16, 128, False, ""), (2, 200, 3, 64, False, ""), (2, 130, 4, 128, True, ""),
    # few chains and many chunks: the chunked calls pipeline their chunk ranges over two streams
    (1, 64 * 256 + 17, 8, 128, False, ""), (1, 64 * 256 + 17, 8, 64, False, "bwa"),
    (1, 64 * 257, 8, 128, True, ""), (1, 32768, 16, 128, False, "")])
def test_phase_entry_points_match_the_chunked_calls(B, T, H, d, pro, scalar):
    """The four phase entry points in the sequence the benchmark times (factors, carry, state
    gradient, chunk gradients) give bitwise the results of gdr2_fwd_chunked + gdr2_bwd_chunked,
    at the full 1.3B-layer size too, so the timed path is the one the parity tests check.  For
    long sequences at a small batch the chunked calls split the chunks into ranges over a second
    stream, handing the carries' fp32 states from range to range: bitwise the same again."""
    import gated_delta_rule_gdr_amd as g2
    prologue = g2.Prologue(0.1, 1e-6) if pro else None
    x = _gpu(layer_inputs(B, T, H, d, d, dtype="bf16", seed=64, s0_std=0.05, dST=True, raw=pro,
                          scalar=scalar))
    announce(f"phase entry points vs chunked calls B={B} T={T} H={H} d={d} prologue={pro} scalar={scalar}")
    args = [x[n] for n in NAMES]
    o, ST, fws = gdr2_fwd_chunked(*args, S0=x["S0"], prologue=prologue)
    ref = gdr2_bwd_chunked(*args, x["dO"], fws, dS_T=x["dST"], prologue=prologue)
    bf = torch.bfloat16
    fws2 = torch.empty(g2.fwd_workspace_bytes(B, T, H, d, d, bf), dtype=torch.uint8, device=DEV)
    bws2 = torch.empty(g2.bwd_workspace_bytes(B, T, H, d, d, bf), dtype=torch.uint8, device=DEV)
    o2, ST2 = torch.empty_like(o), torch.empty_like(ST)
    dS0 = torch.empty_like(ref["dS0"])
    gr = {n: torch.empty_like(x[s]) for n, s in (("dq", "q"), ("dk", "k"), ("dv", "v"),
                                                ("dlog_alpha", "log_alpha"), ("db", "b"), ("dw", "w"))}
    g2.gdr2_fwd_factors(*args, fws2, prologue=prologue)
    g2.gdr2_fwd_carry(B, T, H, d, d, bf, fws2, o2, S0=x["S0"], S_T=ST2)
    g2.gdr2_bwd_state(B, T, H, d, d, bf, fws2, x["dO"], bws2, dS_T=x["dST"], dS0=dS0)
    g2.gdr2_bwd_grads(*args, fws2, x["dO"], bws2, gr, prologue=prologue)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(ST, ST2) and torch.equal(ref["dS0"], dS0)
    for n in GRADS[:-1]:
        assert torch.equal(ref[n], gr[n]), n


def test_split_long_sequences_from_two_host_threads():
    """Two host threads, each on its own stream, run the split (two-stream) long-sequence path at
    the same time; the library serialises their use of its shared second stream and events, so
    each thread's results equal those of the same call made alone."""
    import threading
    xs = [_gpu(layer_inputs(1, 64 * 256 + 9, 8, 128, 128, dtype="bf16", seed=70 + i, s0_std=0.05,
                            dST=True)) for i in range(2)]
    announce("split long-sequence path from two host threads")
    ref = [_layer(x) for x in xs]
    torch.cuda.synchronize()
    out, errs = [None, None], []

    def run(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(3):
                    out[i] = _layer(xs[i])
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errs.append(e)

    th = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    torch.cuda.synchronize()
    assert not errs, errs
    for i in range(2):
        _same(out[i], ref[i])
