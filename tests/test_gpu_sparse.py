"""Parity of the block-sparse path (key summary + top-delta + exact attention
over kept blocks) against the float64 oracle (needs a gfx950 GPU).

* The key summary is integer work decided in fp32 on both sides: codes and
  scales must match the oracle bit for bit.
* The kept-block set must equal the oracle's exactly: the estimates are
  integer dot products of the 8-bit query with the codes, scaled by the
  same float32 multiplications in the same order on both sides, so every
  keep decision is taken identically. The output must match exact
  attention over the kept blocks, to the bf16 bar (2e-3).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import sparse as osp
import workloads
from split_kv_long_amd import binding as fb

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

TOL = 2e-3
LSE_TOL = 1e-4


def shape_of(w):
    return fb.make_shape(**w.shape_dict())


def gpu_summary(w, t):
    d = torch.device("cuda")
    D = w.head_dim
    if w.paged:
        nrec = (w.k.shape[0], w.num_kv_heads, w.block_size // 16)
    else:
        nrec = (w.batch, w.num_kv_heads, -(-w.max_seq_len // 16))
    codes = torch.full(nrec + (8 * D,), 0xAA, dtype=torch.uint8, device=d)
    scales = torch.full(nrec, -1.0, device=d)
    print(f"[gpu] summary {w.name} paged={w.paged} D={D}", flush=True)
    fb.fd_build_key_summary(shape_of(w), t["k"], t["bt"], t["lens"], codes,
                            scales)
    torch.cuda.synchronize()
    return codes, scales


def device_inputs(w):
    d = torch.device("cuda")
    return dict(q=w.q.to(d), k=w.k.to(d), v=w.v.to(d), lens=w.seq_lens.to(d),
                bt=None if w.block_table is None else w.block_table.to(d))


def written_records(w):
    """(b-or-page, kvh, record) index arrays of every record the summary
    writes, and the matching (b-or-page, kvh, first row) of the oracle's
    row-layout codes."""
    a = w.numpy_view()
    rec, row = [], []
    for b in range(w.batch):
        n = int(a["seq_lens"][b])
        for kvh in range(w.num_kv_heads):
            for j in range(-(-n // 16)):
                if w.paged:
                    blk = a["block_table"][b, 16 * j // w.block_size]
                    sub = (16 * j % w.block_size) // 16
                    rec.append((blk, kvh, sub))
                    row.append((blk, kvh, 16 * sub))
                else:
                    rec.append((b, kvh, j))
                    row.append((b, kvh, 16 * j))
    return tuple(np.array(x) for x in zip(*rec)), row


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("d", [128, 64])
def test_summary_matches_oracle_bitwise(paged, d):
    lens = [1, 15, 16, 17, 100, 0, 333]
    w = workloads.make("sum", seed=71, batch=len(lens), num_q_heads=8,
                       num_kv_heads=2, head_dim=d, max_seq_len=333,
                       paged=paged, seq_lens=lens, poison_tail=True)
    t = device_inputs(w)
    codes, scales = gpu_summary(w, t)
    a = w.numpy_view()
    ref_c, ref_s = osp.key_summary(a["k"], a["seq_lens"], a["block_table"],
                                   w.block_size)
    got = codes.cpu().numpy()
    recs, rows = written_records(w)
    L = w.max_seq_len
    for i, (x, h, r0) in enumerate(rows):
        blk = osp.unpack_int4(osp.records_to_rows(got[recs][i], d))
        if w.paged:
            want = ref_c[x, h, r0:r0 + 16]
        else:                      # rows past L do not exist in the cache
            want = np.zeros((16, d), dtype=np.int64)
            want[:min(16, L - r0)] = ref_c[x, h, r0:r0 + 16]
        assert np.array_equal(blk, want), (x, h, r0)
    # nothing else was written
    mask = np.ones(got.shape[:-1], dtype=bool)
    mask[recs] = False
    assert np.all(got[mask] == 0xAA)
    gs = scales.cpu().numpy()
    for b in range(w.batch):
        n = lens[b]
        for kvh in range(2):
            for j in range(-(-n // 16)):
                s_ref = osp.block_scale(ref_s, b, kvh, j, a["block_table"],
                                        w.block_size)
                s_got = osp.block_scale(gs, b, kvh, j, a["block_table"],
                                        w.block_size)
                assert np.float32(s_got) == np.float32(s_ref), (b, kvh, j)


def sparse_case(seed, paged, d=128, hq=16, hkv=2, L=8192, lens=None):
    lens = lens or [L]
    return workloads.make("sparse", seed=seed, batch=len(lens),
                          num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                          max_seq_len=L, paged=paged, seq_lens=lens,
                          needles=[5, L // 3, L // 2 + 7, lens[-1] - 1],
                          needle_logit=14.0, poison_tail=True)


def run_sparse(w, t, codes, scales, delta, S):
    d = torch.device("cuda")
    B, Hq, D = w.batch, w.num_q_heads, w.head_dim
    out = torch.full((B, Hq, D), float("nan"), device=d)
    lse = torch.full((B, Hq), float("nan"), device=d)
    kept = torch.full((B, w.num_kv_heads, -(-w.max_seq_len // 16)), 7,
                      dtype=torch.uint8, device=d)
    shape = shape_of(w)
    nbytes = fb.fd_workspace_size(shape, S)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=d)
    print(f"[gpu] sparse {w.name} paged={w.paged} D={D} delta={delta} S={S}",
          flush=True)
    fb.fd_decode_attn_sparse(shape, t["q"], t["k"], t["v"], codes, scales,
                             t["bt"], t["lens"], delta, S, ws, out, lse, kept)
    torch.cuda.synchronize()
    return (out.cpu().double().numpy(), lse.cpu().double().numpy(),
            kept.cpu().numpy())


def exact_over_kept(w, kept):
    """Float64 attention of every head over the tokens of kept blocks."""
    a = w.numpy_view()
    q = oracle.decode_values(a["q"], "bf16")
    B, Hq, D = q.shape
    G = Hq // w.num_kv_heads
    sc = w.effective_scale
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        n = int(a["seq_lens"][b])
        for kvh in range(w.num_kv_heads):
            toks = np.array([t for t in range(n) if kept[b, kvh, t // 16]],
                            dtype=np.int64)
            if toks.size == 0:
                continue
            kr = np.concatenate([oracle.decode_values(oracle.history_rows(
                a["k"], b, kvh, t, t + 1, a["block_table"], a["block_size"]),
                "bf16") for t in toks])
            vr = np.concatenate([oracle.decode_values(oracle.history_rows(
                a["v"], b, kvh, t, t + 1, a["block_table"], a["block_size"]),
                "bf16") for t in toks])
            hs = slice(kvh * G, (kvh + 1) * G)
            o, l = oracle.softmax_attention(sc * (q[b, hs] @ kr.T), vr)
            out[b, hs], lse[b, hs] = o, l
    return out, lse


def check_sparse(w, delta, S, expect_dropped=True):
    t = device_inputs(w)
    codes, scales = gpu_summary(w, t)
    a = w.numpy_view()
    ref_c, ref_s = osp.key_summary(a["k"], a["seq_lens"], a["block_table"],
                                   w.block_size)
    out, lse, kept = run_sparse(w, t, codes, scales, delta, S)
    ro, rl, est, rkept = osp.sparse_decode_attention(
        a["q"], a["k"], a["v"], a["seq_lens"], ref_c, ref_s, delta=delta,
        num_splits=S, max_seq_len=w.max_seq_len, scale=w.scale,
        block_table=a["block_table"], block_size=a["block_size"])
    for b in range(w.batch):
        n = int(a["seq_lens"][b])
        nb = -(-n // 16)
        for kvh in range(w.num_kv_heads):
            assert np.all(kept[b, kvh, nb:] == 7)       # untouched
            got = kept[b, kvh, :nb].astype(bool)
            assert np.array_equal(got, rkept[b, kvh, :nb]), (b, kvh)
    if expect_dropped:
        assert 0 < kept[kept != 7].sum() < (kept != 7).sum()
    ref_out, ref_lse = exact_over_kept(w, kept.astype(bool) & (kept != 7))
    assert np.all(np.isfinite(out))
    err = float(np.abs(out - ref_out).max())
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isneginf(lse), ~fin)
    lerr = float(np.abs(lse[fin] - ref_lse[fin]).max())
    print(f"[gpu] sparse max|out-ref|={err:.3g} lse={lerr:.3g} "
          f"kept={int(kept[kept != 7].sum())}/{int((kept != 7).sum())}",
          flush=True)
    assert err <= TOL and lerr <= LSE_TOL
    return out, lse, kept


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("S", [1, 4, 16])
def test_sparse_top_delta_matches_oracle(paged, S):
    w = sparse_case(81, paged)
    check_sparse(w, 1.0, S)


@pytest.mark.parametrize("d,hq,hkv", [(64, 8, 8), (64, 32, 4), (128, 12, 3)])
def test_sparse_head_layouts_and_ragged(d, hq, hkv):
    w = sparse_case(82, True, d=d, hq=hq, hkv=hkv, L=4000,
                    lens=[4000, 1, 17, 2500])
    check_sparse(w, 2.0, 3, expect_dropped=False)


def test_sparse_delta_inf_is_dense():
    w = sparse_case(83, False, L=6000, lens=[6000, 4321])
    out, lse, kept = check_sparse(w, math.inf, 2, expect_dropped=False)
    assert np.all(kept[kept != 7] == 1)
    a = w.numpy_view()
    ref = oracle.decode_attention(a["q"], a["k"], a["v"], a["seq_lens"],
                                  dtype="bf16")
    assert np.abs(out - ref[0]).max() <= TOL


def test_sparse_delta_zero_keeps_the_needles():
    w = sparse_case(84, False, L=8192)
    out, lse, kept = check_sparse(w, 0.0, 4)
    for p in (5, 8192 // 3, 8192 // 2 + 7, 8191):
        assert kept[0, 0, p // 16] == 1 and kept[0, 1, p // 16] == 1


@pytest.mark.parametrize("bs", [32, 64])
def test_sparse_and_summary_with_larger_pages(bs):
    lens = [4000, 1, 17, 2500]
    w = workloads.make("sparse", seed=85, batch=len(lens), num_q_heads=8,
                       num_kv_heads=2, head_dim=128, max_seq_len=4000,
                       paged=True, block_size=bs, seq_lens=lens,
                       needles=[5, 1333, 3999], needle_logit=14.0,
                       poison_tail=True)
    check_sparse(w, 2.0, 3, expect_dropped=False)


def test_sparse_random_shapes():
    # Seeded sweep: batch, kv heads, group size (both head-group widths),
    # head_dim, ragged lengths, contiguous or paged, delta and split count;
    # kept sets must equal the oracle's and outputs match exact attention
    # over the kept blocks.
    import random
    rng = random.Random(909)
    for case in range(16):
        hkv, g = rng.choice([1, 2, 3]), rng.choice([1, 3, 8, 12, 16])
        L = rng.choice([17, 100, 511, 900, 1500])
        b = rng.choice([1, 2, 3])
        lens = [rng.randint(1, L) for _ in range(b)]
        lens[rng.randrange(b)] = L
        w = workloads.make(f"sparse_random{case}", seed=4000 + case,
                           batch=b, num_q_heads=g * hkv, num_kv_heads=hkv,
                           head_dim=rng.choice([64, 128]), max_seq_len=L,
                           paged=rng.random() < 0.5, seq_lens=lens,
                           needles=[0, L // 2, L - 1], needle_logit=10.0,
                           poison_tail=True)
        check_sparse(w, rng.choice([0.0, 0.5, 2.0, 5.0]),
                     rng.choice([1, 2, 3, 5, 8]), expect_dropped=False)
