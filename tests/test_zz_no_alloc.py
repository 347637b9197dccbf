"""fd_decode_attn_noalloc (the allocation-free entry point) against
fd_decode_attn with a caller's workspace, through the C ABI on the GPU.

Two calls in a row, the second on a smaller input, each checked against
the workspace call on the same inputs (the same kernels and partial layout
run, so the outputs must agree bit for bit) and against the float64 oracle
at the bf16 bar."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from split_kv_long_amd import binding as fb

pytestmark = pytest.mark.gpu

TOL = 2e-3        # bf16 inputs, fp32 accumulation


def inputs(w):
    d = torch.device("cuda")
    return dict(q=w.q.to(d), k=w.k.to(d), v=w.v.to(d),
                lens=w.seq_lens.to(d),
                bt=None if w.block_table is None else w.block_table.to(d))


def both_calls(w, S):
    t = inputs(w)
    shape = fb.make_shape(**w.shape_dict())
    B, Hq, D = w.batch, w.num_q_heads, w.head_dim
    res = []
    for noalloc in (False, True):
        out = torch.full((B, Hq, D), float("nan"), device="cuda")
        lse = torch.full((B, Hq), float("nan"), device="cuda")
        print(f"[gpu] {w.name} S={S} noalloc={noalloc}", flush=True)
        if noalloc:
            fb.fd_decode_attn_noalloc(shape, t["q"], t["k"], t["v"], t["bt"],
                                      t["lens"], S, out, lse)
        else:
            nb = fb.fd_workspace_size(shape, S)
            ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
            fb.fd_decode_attn(shape, t["q"], t["k"], t["v"], t["bt"],
                              t["lens"], S, ws, out, lse)
        torch.cuda.synchronize()
        res.append((out.cpu().double().numpy(), lse.cpu().double().numpy()))
    return res


def test_noalloc_matches_the_workspace_call_on_two_calls():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    big = workloads.make("long_gqa_64k")
    small = workloads.make("ragged_paged", seed=95, batch=3, max_seq_len=5000,
                           min_seq_len=1)
    for w in (big, small):                     # the second call is smaller
        S = fb.fd_plan_splits(fb.make_shape(**w.shape_dict()), cus,
                              w.sum_seq_len())
        assert S > 1                           # the partials use the scratch
        (o1, l1), (o2, l2) = both_calls(w, S)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), w.name
        a = w.numpy_view()
        ro, rl = oracle.decode_attention(
            a["q"], a["k"], a["v"], a["seq_lens"], dtype="bf16",
            block_table=a["block_table"], block_size=a["block_size"])
        assert np.abs(o2 - ro).max() <= TOL, w.name
        fin = np.isfinite(rl)
        assert np.abs(l2[fin] - rl[fin]).max() <= 1e-4, w.name


def test_noalloc_call_replays_in_a_graph():
    """What the entry point is for: captured in a HIP graph (nothing to
    allocate, nothing cleared), every replay with eager work between --
    including a workspace call of another shape -- reproduces the eager
    result bit for bit."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    w = workloads.make("long_gqa_64k", max_seq_len=16384)
    other = workloads.make("ragged_paged", seed=96, batch=2, max_seq_len=3000,
                           min_seq_len=1)
    t, to = inputs(w), inputs(other)
    shape = fb.make_shape(**w.shape_dict())
    S = fb.fd_plan_splits(shape, cus, w.sum_seq_len())
    assert S > 1
    out = torch.empty(w.batch, w.num_q_heads, w.head_dim, device="cuda")
    lse = torch.empty(w.batch, w.num_q_heads, device="cuda")

    def call():
        fb.fd_decode_attn_noalloc(shape, t["q"], t["k"], t["v"], t["bt"],
                                  t["lens"], S, out, lse)
    call()
    torch.cuda.synchronize()
    ref = (out.cpu().clone(), lse.cpu().clone())
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    print(f"[gpu] noalloc graph capture S={S}", flush=True)
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            call()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        both_calls(other, 3)                 # eager work, scratch reused
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.cpu(), ref[0]) and torch.equal(lse.cpu(), ref[1])
