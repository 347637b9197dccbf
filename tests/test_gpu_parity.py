"""Parity of the HIP library against the float64 oracle (needs a gfx950 GPU).

Every case draws seeded inputs from ``workloads``, runs them through the C ABI
(``split_kv_long_amd.binding``) and through ``oracle``, and compares every
output element. Bars: max |out - oracle| <= 1e-5 for fp32 inputs and 2e-3 for
bf16 inputs (fp32 accumulation); |lse - oracle| <= 1e-4; empty histories give
exactly 0 / -inf.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from split_kv_long_amd import binding as fb

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

# fp8_e4m3 / int8: bf16 query against an 8-bit cache, fp32 accumulation --
# the codes convert exactly to bf16, and the scales add one fp32 rounding
# per score and per probability, so the bf16 bar applies.
TOL = {"f32": 1e-5, "bf16": 2e-3, "fp8_e4m3": 2e-3, "int8": 2e-3}
LSE_TOL = 1e-4
LOG = os.environ.get("FD_PARITY_LOG")


def num_cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def shape_of(w):
    return fb.make_shape(**w.shape_dict())


def device_inputs(w):
    d = torch.device("cuda")
    return dict(q=w.q.to(d), k=w.k.to(d), v=w.v.to(d),
                seq_lens=w.seq_lens.to(d),
                bt=None if w.block_table is None else w.block_table.to(d),
                ks=None if w.k_scale is None else w.k_scale.to(d),
                vs=None if w.v_scale is None else w.v_scale.to(d))


def gpu_attention(w, S, t=None):
    t = t or device_inputs(w)
    shape = shape_of(w)
    out = torch.full((w.batch, w.num_q_heads, w.head_dim), float("nan"),
                     device="cuda")
    lse = torch.full((w.batch, w.num_q_heads), float("nan"), device="cuda")
    nbytes = fb.fd_workspace_size(shape, S)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    print(f"[gpu] {w.name} {w.cache_dtype} S={S}", flush=True)
    if w.cache_dtype in ("fp8_e4m3", "int8"):
        call = (fb.fd_decode_attn_fp8 if w.cache_dtype == "fp8_e4m3"
                else fb.fd_decode_attn_int8)
        call(shape, t["q"], t["k"], t["v"], t["ks"], t["vs"], t["bt"],
             t["seq_lens"], S, ws, out, lse)
    else:
        fb.fd_decode_attn(shape, t["q"], t["k"], t["v"], t["bt"],
                          t["seq_lens"], S, ws, out, lse)
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), lse.cpu().double().numpy()


def oracle_attention(w):
    a = w.numpy_view()
    return oracle.decode_attention(a["q"], a["k"], a["v"], a["seq_lens"],
                                   dtype=a["dtype"], scale=a["scale"],
                                   block_table=a["block_table"],
                                   block_size=a["block_size"],
                                   kv_dtype=a["kv_dtype"],
                                   k_scale=a["k_scale"], v_scale=a["v_scale"])


def assert_parity(name, dtype, out, lse, ref_out, ref_lse):
    tol = TOL[dtype]
    assert np.all(np.isfinite(out)), f"{name}: non-finite output"
    err = float(np.abs(out - ref_out).max())
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isneginf(lse), ~fin), f"{name}: -inf lse mismatch"
    lerr = float(np.abs(lse[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
    if LOG:
        with open(LOG, "a") as f:
            f.write(json.dumps(dict(case=name, dtype=dtype, max_abs=err,
                                    lse_max_abs=lerr, tol=tol)) + "\n")
    assert err <= tol, f"{name}: max |out - oracle| = {err:.3g} > {tol}"
    assert lerr <= LSE_TOL, f"{name}: max |lse - oracle| = {lerr:.3g}"
    empty = ~fin
    assert np.all(out[empty] == 0.0)


def check(w, S):
    out, lse = gpu_attention(w, S)
    ref_out, ref_lse = oracle_attention(w)
    assert_parity(f"{w.name}/{w.cache_dtype}/S={S}", w.cache_dtype, out, lse,
                  ref_out, ref_lse)
    return out, lse


# ------------------------------------------------------- the five workloads

@pytest.mark.parametrize("name", workloads.ORDER)
def test_workload_at_planned_splits(name):
    w = workloads.make(name)
    S = fb.fd_plan_splits(shape_of(w), num_cus(), w.sum_seq_len())
    check(w, S)


@pytest.mark.parametrize("name,splits", [
    ("tiny_mha", [1, 4]),
    ("long_gqa_64k", [1, 2, 4, 8, 512]),
    ("ultra_long_256k", [8, 64, 256]),
    ("ragged_paged", [1, 16]),
    ("short_batch", [2, 8]),
])
def test_workload_at_forced_splits(name, splits):
    w = workloads.make(name)
    ref_out, ref_lse = oracle_attention(w)
    t = device_inputs(w)
    for S in splits:
        out, lse = gpu_attention(w, S, t)
        assert_parity(f"{name}/S={S}", w.cache_dtype, out, lse, ref_out,
                      ref_lse)


# ---------------------------------------------------------------- edge cases

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("paged", [False, True])
def test_ragged_tails_with_poisoned_cache(dtype, paged):
    lens = [1, 15, 16, 17, 31, 33, 100, 511, 0, 257]
    w = workloads.make("ragged", seed=21, batch=len(lens), num_q_heads=16,
                       num_kv_heads=2, head_dim=128, max_seq_len=512,
                       dtype=dtype, paged=paged, seq_lens=lens,
                       poison_tail=True)
    for S in (1, 3, 8, 32):
        check(w, S)


@pytest.mark.parametrize("batch", [1, 3])
def test_subtile_rounds_per_wave(batch):
    # A bf16 wave streams the subtiles w, w + NW, ... of its split and
    # requests the next one as the current one lands, alternating two
    # register sets; these lengths end that loop after 1 to 7 rounds, on
    # either set, with full, partial and fully masked last subtiles.
    for L in (96, 128, 200, 256, 401, 640, 777, 896):
        lens = [L] if batch == 1 else [L, max(L - 37, 1), L // 2]
        w = workloads.make(f"rounds{L}", seed=40 + L, batch=batch,
                           num_q_heads=16, num_kv_heads=2, head_dim=128,
                           max_seq_len=L, seq_lens=lens, poison_tail=True)
        for S in (1, 2, 3):
            check(w, S)


def test_random_shapes():
    # A seeded sweep over the shape space: dtype, head_dim, kv heads, group
    # size (both head-group widths), batch, ragged lengths with one full
    # history, contiguous or paged (16- to 64-token pages), split count.
    import random
    rng = random.Random(2026)
    for case in range(60):
        kv = rng.choice(["bf16", "bf16", "fp8_e4m3", "f32"])
        hkv, g = rng.choice([1, 2, 3, 4]), rng.choice([1, 2, 4, 5, 8, 12, 16, 24])
        b = rng.choice([1, 1, 2, 3, 5, 9])
        L = rng.choice([1, 15, 33, 100, 257, 511, 700, 1024, 1500, 3000])
        lens = [rng.randint(0, L) for _ in range(b)]
        lens[rng.randrange(b)] = L
        paged = rng.random() < 0.5
        w = workloads.make(f"random{case}", seed=3000 + case, batch=b,
                           num_q_heads=g * hkv, num_kv_heads=hkv,
                           head_dim=rng.choice([64, 128]), max_seq_len=L,
                           dtype="f32" if kv == "f32" else "bf16",
                           paged=paged,
                           block_size=rng.choice([16, 32, 64]) if paged else 16,
                           seq_lens=lens, poison_tail=True,
                           kv_dtype="fp8_e4m3" if kv == "fp8_e4m3" else None)
        check(w, rng.choice([1, 2, 3, 4, 7, 8, 16, 33, 64]))


def test_more_splits_than_tiles():
    lens = [3, 64, 40, 17]
    w = workloads.make("few_tiles", seed=22, batch=4, num_q_heads=8,
                       num_kv_heads=2, head_dim=128, max_seq_len=64,
                       seq_lens=lens, poison_tail=True)
    for S in (4, 16, 64):          # P = 16: most splits of short rows empty
        check(w, S)


def test_empty_histories():
    w = workloads.make("empty", seed=23, batch=3, num_q_heads=4,
                       num_kv_heads=1, head_dim=64, max_seq_len=32,
                       seq_lens=[0, 0, 0])
    for S in (1, 2):
        out, lse = gpu_attention(w, S)
        assert np.all(out == 0.0) and np.all(np.isneginf(lse))


@pytest.mark.parametrize("paged", [False, True])
def test_needles_at_boundaries(paged):
    L, S = 4096, 8
    P = oracle.split_length(L, S)
    n = L - 5
    positions = sorted({0, n - 1, P - 1, P, 3 * P - 1, 3 * P, 7 * P - 1,
                        (n - 1) // 16 * 16})
    for p in positions:
        w = workloads.make("needle", seed=24, batch=1, num_q_heads=16,
                           num_kv_heads=2, head_dim=128, max_seq_len=L,
                           seq_lens=[n], paged=paged, needles=[p],
                           needle_logit=40.0, poison_tail=True)
        out, lse = check(w, S)
        ref_v = w.v.float()
        for kvh in range(2):
            h = kvh * 8
            if paged:
                row = ref_v[int(w.block_table[0, p // 16]), kvh, p % 16]
            else:
                row = ref_v[0, kvh, p]
            assert np.abs(out[0, h] - row.double().numpy()).max() < 2e-3, p


def test_paged_matches_contiguous_bitwise():
    w = workloads.make("ragged_paged", seed=25, batch=6, max_seq_len=3000,
                       min_seq_len=1)
    c = workloads.to_contiguous(w)
    for S in (1, 5):
        o1, l1 = gpu_attention(w, S)
        o2, l2 = gpu_attention(c, S)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("hq,hkv,d", [(8, 8, 128), (12, 3, 128), (16, 1, 128),
                                      (64, 2, 128), (40, 2, 64), (32, 8, 64),
                                      (4, 4, 64)])
def test_head_layouts_bf16(hq, hkv, d):
    w = workloads.make("heads", seed=26, batch=2, num_q_heads=hq,
                       num_kv_heads=hkv, head_dim=d, max_seq_len=700,
                       seq_lens=[700, 333])
    for S in (1, 3):
        check(w, S)


@pytest.mark.parametrize("hq,hkv,d", [(16, 2, 128), (6, 3, 64), (40, 2, 64),
                                     (34, 1, 128)])
def test_head_layouts_f32(hq, hkv, d):
    """fp32 caches, including groups of more than 16 query heads per kv
    head (two head groups, the second partial: 20 = 16 + 4, 34 = 16 + 16
    + 2)."""
    w = workloads.make("heads32", seed=27, batch=2, num_q_heads=hq,
                       num_kv_heads=hkv, head_dim=d, max_seq_len=300,
                       seq_lens=[300, 129], dtype="f32")
    for S in (1, 4):
        check(w, S)


def test_custom_scale_and_large_logits():
    w = workloads.make("ultra_long_256k", max_seq_len=8192, scale=0.3,
                       hot_key_fraction=0.002)
    check(w, 1)
    check(w, 16)


@pytest.mark.parametrize("rise,period", [(30.0, 8192), (-40.0, 8192),
                                         (200.0, 512)])
def test_drifting_logits(rise, period):
    """Logits that drift along the history: the first head of each group
    gains `rise` (natural-log units) over every `period` tokens, so the
    running maximum creeps up in small steps (30 over the whole history),
    only falls (-40), or jumps on every 32-token tile and drops at each
    period boundary (a sawtooth of 200 per 512 tokens)."""
    import dataclasses
    L = 8192
    w = workloads.make("drift", seed=29, batch=2, num_q_heads=16,
                       num_kv_heads=2, head_dim=128, max_seq_len=L,
                       seq_lens=[L, 5000])
    G = 8
    scl = w.effective_scale
    k = w.k.float()
    q = w.q.float()
    ramp = (torch.arange(L) % period).float() / (period - 1)
    for b in range(2):
        for h in range(2):
            qv = q[b, h * G]
            u = qv / float(qv @ qv)             # q.u = 1 for the first head
            k[b, h] += (rise / scl) * ramp[:, None] * u[None, :]
    w = dataclasses.replace(w, k=k.to(torch.bfloat16).contiguous())
    ref_out, ref_lse = oracle_attention(w)
    t = device_inputs(w)
    for S in (1, 4, 32):
        out, lse = gpu_attention(w, S, t)
        assert_parity(f"drift{rise}/{period}/S={S}", "bf16", out, lse,
                      ref_out, ref_lse)


@pytest.mark.parametrize("bs", [16, 64])
def test_partials_and_combine_entry_points(bs):
    # With 64-token pages the splits are whole pages: 192 tokens for
    # L = 900, S = 7 (16-token rounding would give 144).
    w = workloads.make("ragged_paged", seed=28, batch=3, num_q_heads=16,
                       num_kv_heads=4, head_dim=128, max_seq_len=900,
                       min_seq_len=1, poison_tail=True, block_size=bs)
    S = 7
    t = device_inputs(w)
    shape = shape_of(w)
    B, Hq, D = w.batch, w.num_q_heads, w.head_dim
    op = torch.empty(B, Hq, S, D, device="cuda")
    lp = torch.empty(B, Hq, S, device="cuda")
    fb.fd_decode_partials(shape, t["q"], t["k"], t["v"], t["bt"],
                          t["seq_lens"], S, op, lp)
    torch.cuda.synchronize()
    a = w.numpy_view()
    ref_op, ref_lp = oracle.split_partials(
        a["q"], a["k"], a["v"], a["seq_lens"], S, dtype="bf16",
        max_seq_len=900, block_table=a["block_table"],
        block_size=a["block_size"])
    got_op, got_lp = op.cpu().double().numpy(), lp.cpu().double().numpy()
    assert_parity("partials", "bf16", got_op.reshape(B, Hq * S, D),
                  got_lp.reshape(B, Hq * S), ref_op.reshape(B, Hq * S, D),
                  ref_lp.reshape(B, Hq * S))
    # combine of the oracle's partials (rounded to fp32) on the GPU
    op2 = torch.from_numpy(ref_op.astype(np.float32)).cuda()
    lp2 = torch.from_numpy(ref_lp.astype(np.float32)).cuda()
    out = torch.empty(B, Hq, D, device="cuda")
    lse = torch.empty(B, Hq, device="cuda")
    fb.fd_combine_partials(B, Hq, D, S, op2, lp2, out, lse)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.combine_partials(ref_op.astype(np.float32),
                                               ref_lp.astype(np.float32))
    assert_parity("combine", "f32", out.cpu().double().numpy(),
                  lse.cpu().double().numpy(), ref_out, ref_lse)


@pytest.mark.parametrize("lens", [[16384], [16384, 9000, 4100, 1]])
def test_sequence_sharded_partials_then_combine(lens):
    # The sequence-sharded layout on one GPU: the history is cut into four
    # contiguous shards (what four GPUs would each hold); every shard runs
    # the split step on its own cache with its own split count, the
    # partials are concatenated along the split axis (what an all-gather
    # would deliver), and one combine gives attention over the whole
    # history. Shards past a sequence's end contribute empty partials.
    L, R = 16384, 4
    w = workloads.make("sharded", seed=29, batch=len(lens), num_q_heads=16,
                       num_kv_heads=2, head_dim=128, max_seq_len=L,
                       seq_lens=lens, poison_tail=True)
    B, Hq, D = w.batch, w.num_q_heads, w.head_dim
    d = torch.device("cuda")
    q = w.q.to(d)
    Ls = L // R
    ops, lps = [], []
    for r in range(R):
        k = w.k[:, :, r * Ls:(r + 1) * Ls].contiguous().to(d)
        v = w.v[:, :, r * Ls:(r + 1) * Ls].contiguous().to(d)
        sl = torch.clamp(w.seq_lens - r * Ls, 0, Ls).to(torch.int32).to(d)
        shape = fb.make_shape(B, Hq, w.num_kv_heads, D, Ls, "bf16")
        S_r = 8 + 8 * r                        # shards need not agree on S
        op = torch.empty(B, Hq, S_r, D, device=d)
        lp = torch.empty(B, Hq, S_r, device=d)
        print(f"[gpu] shard {r} S={S_r}", flush=True)
        fb.fd_decode_partials(shape, q, k, v, None, sl, S_r, op, lp)
        ops.append(op)
        lps.append(lp)
    op = torch.cat(ops, dim=2).contiguous()
    lp = torch.cat(lps, dim=2).contiguous()
    S = op.shape[2]
    out = torch.empty(B, Hq, D, device=d)
    lse = torch.empty(B, Hq, device=d)
    fb.fd_combine_partials(B, Hq, D, S, op, lp, out, lse)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_attention(w)
    assert_parity("sharded", "bf16", out.cpu().double().numpy(),
                  lse.cpu().double().numpy(), ref_out, ref_lse)


def test_deterministic_bitwise():
    w = workloads.make("long_gqa_64k", max_seq_len=16384)
    t = device_inputs(w)
    o1, l1 = gpu_attention(w, 32, t)
    o2, l2 = gpu_attention(w, 32, t)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_convenience_wrapper_plans_and_allocates():
    import split_kv_long_amd as fd
    w = workloads.make("long_gqa_64k", max_seq_len=5000)
    t = device_inputs(w)
    out, lse = fd.decode_attention(t["q"], t["k"], t["v"], t["seq_lens"],
                                   return_lse=True)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_attention(w)
    assert_parity("wrapper", "bf16", out.cpu().double().numpy(),
                  lse.cpu().double().numpy(), ref_out, ref_lse)


# ------------------------------------------------- 8-bit E4M3 cache (fp8)

def test_fp8_64k_at_planned_and_forced_splits():
    w = workloads.make("long_gqa_64k_fp8")
    ref_out, ref_lse = oracle_attention(w)
    t = device_inputs(w)
    planned = fb.fd_plan_splits(shape_of(w), num_cus(), w.sum_seq_len())
    for S in sorted({planned, 1, 8, 64, 512}):
        out, lse = gpu_attention(w, S, t)
        assert_parity(f"fp8-64k/S={S}", "fp8_e4m3", out, lse, ref_out,
                      ref_lse)


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("d", [128, 64])
def test_fp8_ragged_tails_with_poisoned_cache(paged, d):
    lens = [1, 15, 16, 17, 31, 33, 100, 511, 0, 257, 1000]
    w = workloads.make("ragged8", seed=41, batch=len(lens), num_q_heads=16,
                       num_kv_heads=2, head_dim=d, max_seq_len=1000,
                       paged=paged, seq_lens=lens, poison_tail=True,
                       kv_dtype="fp8_e4m3")
    for S in (1, 3, 8, 32):
        check(w, S)


@pytest.mark.parametrize("hq,hkv,d", [(8, 8, 128), (12, 3, 128),
                                      (64, 2, 128), (40, 2, 64), (4, 4, 64)])
def test_fp8_head_layouts(hq, hkv, d):
    w = workloads.make("heads8", seed=42, batch=2, num_q_heads=hq,
                       num_kv_heads=hkv, head_dim=d, max_seq_len=2100,
                       seq_lens=[2100, 777], kv_dtype="fp8_e4m3")
    for S in (1, 5):
        check(w, S)


def test_fp8_long_ragged_paged_batch():
    w = workloads.make("ragged_paged", seed=43, batch=6, max_seq_len=20000,
                       kv_dtype="fp8_e4m3")
    check(w, fb.fd_plan_splits(shape_of(w), num_cus(), w.sum_seq_len()))
    check(w, 1)


def test_fp8_partials_entry_point():
    w = workloads.make("ragged_paged", seed=44, batch=3, num_q_heads=16,
                       num_kv_heads=4, head_dim=128, max_seq_len=900,
                       min_seq_len=1, poison_tail=True, kv_dtype="fp8_e4m3")
    S = 7
    t = device_inputs(w)
    B, Hq, D = w.batch, w.num_q_heads, w.head_dim
    op = torch.empty(B, Hq, S, D, device="cuda")
    lp = torch.empty(B, Hq, S, device="cuda")
    fb.fd_decode_partials_fp8(shape_of(w), t["q"], t["k"], t["v"], t["ks"],
                              t["vs"], t["bt"], t["seq_lens"], S, op, lp)
    torch.cuda.synchronize()
    a = w.numpy_view()
    ref_op, ref_lp = oracle.split_partials(
        a["q"], a["k"], a["v"], a["seq_lens"], S, dtype="bf16",
        max_seq_len=900, block_table=a["block_table"],
        block_size=a["block_size"], kv_dtype="fp8_e4m3",
        k_scale=a["k_scale"], v_scale=a["v_scale"])
    assert_parity("fp8-partials", "fp8_e4m3",
                  op.cpu().double().numpy().reshape(B, Hq * S, D),
                  lp.cpu().double().numpy().reshape(B, Hq * S),
                  ref_op.reshape(B, Hq * S, D), ref_lp.reshape(B, Hq * S))


def test_fp8_paged_matches_contiguous_bitwise():
    w = workloads.make("ragged_paged", seed=45, batch=5, max_seq_len=3000,
                       min_seq_len=1, kv_dtype="fp8_e4m3")
    c = workloads.to_contiguous(w)
    for S in (1, 6):
        o1, l1 = gpu_attention(w, S)
        o2, l2 = gpu_attention(c, S)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("kv", ["fp8_e4m3", "int8"])
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("hq,d", [(16, 128), (32, 128), (40, 64)])
def test_8bit_single_sequence_long_splits(kv, paged, hq, d):
    """A single sequence's 8-bit splits of 2048 tokens or more (8 subtiles
    per wave and up) take the reissue schedule (for int8 the subtile's
    scales are part of each register set): full histories, lengths ending
    inside a subtile and inside the last split, NaN-poisoned slots past
    the length, one and two head passes (S = 4 is the threshold itself at
    L = 8192), and odd and even subtile counts per wave."""
    for i, (L, n) in enumerate(((8192, 8192), (8192, 8179), (12288, 9001))):
        w = workloads.make("8bitlong", seed=46 + i, batch=1, num_q_heads=hq,
                           num_kv_heads=2, head_dim=d, max_seq_len=L,
                           paged=paged, seq_lens=[n], poison_tail=True,
                           kv_dtype=kv)
        for S in (1, 2, 4):
            check(w, S)


# ------------------------------- 8-bit integer cache, per-position scales

def test_int8_64k_at_planned_and_forced_splits():
    w = workloads.make("long_gqa_64k_int8")
    ref_out, ref_lse = oracle_attention(w)
    t = device_inputs(w)
    planned = fb.fd_plan_splits(shape_of(w), num_cus(), w.sum_seq_len())
    for S in sorted({planned, 1, 8, 64, 512}):
        out, lse = gpu_attention(w, S, t)
        assert_parity(f"int8-64k/S={S}", "int8", out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("d", [128, 64])
def test_int8_ragged_tails_with_poisoned_cache(paged, d):
    """Unattended slots hold code 127 and NaN scales: any read of them that
    reaches the arithmetic turns the output NaN."""
    lens = [1, 15, 16, 17, 31, 33, 100, 511, 0, 257, 1000]
    w = workloads.make("ragged_i8", seed=141, batch=len(lens),
                       num_q_heads=16, num_kv_heads=2, head_dim=d,
                       max_seq_len=1000, paged=paged, seq_lens=lens,
                       poison_tail=True, kv_dtype="int8")
    for S in (1, 3, 8, 32):
        check(w, S)


def test_int8_single_sequence_short_tail_poisoned():
    # Batch one takes the speculative first requests: rows past the length
    # are read before it is known, and their NaN scales must stay masked.
    for L, n in ((1000, 1), (1000, 17), (4096, 4000), (700, 699)):
        w = workloads.make("spec_i8", seed=142 + n, batch=1, num_q_heads=16,
                           num_kv_heads=2, head_dim=128, max_seq_len=L,
                           seq_lens=[n], poison_tail=True, kv_dtype="int8")
        for S in (1, 4, 16):
            check(w, S)


@pytest.mark.parametrize("hq,hkv,d", [(8, 8, 128), (12, 3, 128),
                                      (64, 2, 128), (40, 2, 64), (4, 4, 64)])
def test_int8_head_layouts(hq, hkv, d):
    w = workloads.make("heads_i8", seed=143, batch=2, num_q_heads=hq,
                       num_kv_heads=hkv, head_dim=d, max_seq_len=2100,
                       seq_lens=[2100, 777], kv_dtype="int8")
    for S in (1, 5):
        check(w, S)


def test_int8_long_ragged_paged_batch():
    w = workloads.make("ragged_paged", seed=144, batch=6, max_seq_len=20000,
                       kv_dtype="int8")
    check(w, fb.fd_plan_splits(shape_of(w), num_cus(), w.sum_seq_len()))
    check(w, 1)


def test_int8_partials_entry_point():
    w = workloads.make("ragged_paged", seed=145, batch=3, num_q_heads=16,
                       num_kv_heads=4, head_dim=128, max_seq_len=900,
                       min_seq_len=1, poison_tail=True, kv_dtype="int8")
    S = 7
    t = device_inputs(w)
    B, Hq, D = w.batch, w.num_q_heads, w.head_dim
    op = torch.empty(B, Hq, S, D, device="cuda")
    lp = torch.empty(B, Hq, S, device="cuda")
    print("[gpu] int8 partials", flush=True)
    fb.fd_decode_partials_int8(shape_of(w), t["q"], t["k"], t["v"], t["ks"],
                               t["vs"], t["bt"], t["seq_lens"], S, op, lp)
    torch.cuda.synchronize()
    a = w.numpy_view()
    ref_op, ref_lp = oracle.split_partials(
        a["q"], a["k"], a["v"], a["seq_lens"], S, dtype="bf16",
        max_seq_len=900, block_table=a["block_table"],
        block_size=a["block_size"], kv_dtype="int8",
        k_scale=a["k_scale"], v_scale=a["v_scale"])
    assert_parity("int8-partials", "int8",
                  op.cpu().double().numpy().reshape(B, Hq * S, D),
                  lp.cpu().double().numpy().reshape(B, Hq * S),
                  ref_op.reshape(B, Hq * S, D), ref_lp.reshape(B, Hq * S))


def test_int8_paged_matches_contiguous_bitwise():
    w = workloads.make("ragged_paged", seed=146, batch=5, max_seq_len=3000,
                       min_seq_len=1, kv_dtype="int8")
    c = workloads.to_contiguous(w)
    for S in (1, 6):
        o1, l1 = gpu_attention(w, S)
        o2, l2 = gpu_attention(c, S)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("bs", [32, 256])
def test_int8_larger_page_sizes(bs):
    lens = [1, 31, 33, 255, 257, 1000, 0, 2047]
    w = workloads.make("pages_i8", seed=147, batch=len(lens),
                       num_q_heads=16, num_kv_heads=2, head_dim=128,
                       max_seq_len=2048, paged=True, block_size=bs,
                       seq_lens=lens, poison_tail=True, kv_dtype="int8")
    for S in (1, 3, 8):
        check(w, S)


def test_int8_random_shapes():
    import random
    rng = random.Random(2027)
    for case in range(24):
        hkv, g = rng.choice([1, 2, 3, 4]), rng.choice([1, 2, 4, 5, 8, 12, 16, 24])
        b = rng.choice([1, 1, 2, 3, 5, 9])
        L = rng.choice([1, 15, 33, 100, 257, 511, 700, 1024, 1500, 3000])
        lens = [rng.randint(0, L) for _ in range(b)]
        lens[rng.randrange(b)] = L
        paged = rng.random() < 0.5
        w = workloads.make(f"random_i8_{case}", seed=5000 + case, batch=b,
                           num_q_heads=g * hkv, num_kv_heads=hkv,
                           head_dim=rng.choice([64, 128]), max_seq_len=L,
                           paged=paged,
                           block_size=rng.choice([16, 32, 64]) if paged else 16,
                           seq_lens=lens, poison_tail=True, kv_dtype="int8")
        check(w, rng.choice([1, 2, 3, 4, 7, 8, 16, 33, 64]))


def test_convenience_wrapper_int8_cache():
    import split_kv_long_amd as fd
    w = workloads.make("long_gqa_64k_int8", max_seq_len=5000)
    t = device_inputs(w)
    out, lse = fd.decode_attention(t["q"], t["k"], t["v"], t["seq_lens"],
                                   return_lse=True, k_scale=t["ks"],
                                   v_scale=t["vs"])
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_attention(w)
    assert_parity("wrapper-int8", "int8", out.cpu().double().numpy(),
                  lse.cpu().double().numpy(), ref_out, ref_lse)


# ------------------------------------------------------------ large sizes

def test_million_token_history_and_max_splits():
    """A 2^20-token history (512 MB of bf16 K/V for one kv head) at the
    planned split count and at the largest split count the ABI allows
    (65535: 16-token splits, half of them past the history's end)."""
    L = 1 << 20
    w = workloads.make("million", seed=91, batch=1, num_q_heads=8,
                       num_kv_heads=1, head_dim=128, max_seq_len=L,
                       seq_lens=[L - 3], needles=[L // 2 + 1], needle_logit=9.0)
    ref_out, ref_lse = oracle_attention(w)
    t = device_inputs(w)
    planned = fb.fd_plan_splits(shape_of(w), num_cus(), w.sum_seq_len())
    for S in (planned, 65535):
        out, lse = gpu_attention(w, S, t)
        assert_parity(f"million/S={S}", "bf16", out, lse, ref_out, ref_lse)


def test_large_ragged_batch():
    """4096 short ragged sequences (lengths 0..48): batch x kv heads covers
    the GPU many times over, so the planner does not split; forced splits
    must agree too."""
    g = torch.Generator().manual_seed(92)
    lens = torch.randint(0, 49, (4096,), generator=g).tolist()
    w = workloads.make("bigbatch", seed=92, batch=4096, num_q_heads=8,
                       num_kv_heads=2, head_dim=64, max_seq_len=48,
                       seq_lens=lens, paged=True, poison_tail=True)
    ref_out, ref_lse = oracle_attention(w)
    t = device_inputs(w)
    planned = fb.fd_plan_splits(shape_of(w), num_cus(), w.sum_seq_len())
    assert planned == 1
    for S in (1, 3):
        out, lse = gpu_attention(w, S, t)
        assert_parity(f"bigbatch/S={S}", "bf16", out, lse, ref_out, ref_lse)


def test_int8_million_token_history_and_max_splits():
    """A 2^20-token int8 history (256 MB of codes + 8 MB of scales for one
    kv head) at the planned split count and at 65535 splits."""
    L = 1 << 20
    w = workloads.make("million_i8", seed=191, batch=1, num_q_heads=8,
                       num_kv_heads=1, head_dim=128, max_seq_len=L,
                       seq_lens=[L - 3], needles=[L // 2 + 1],
                       needle_logit=9.0, kv_dtype="int8")
    ref_out, ref_lse = oracle_attention(w)
    t = device_inputs(w)
    planned = fb.fd_plan_splits(shape_of(w), num_cus(), w.sum_seq_len())
    for S in (planned, 65535):
        out, lse = gpu_attention(w, S, t)
        assert_parity(f"million-int8/S={S}", "int8", out, lse, ref_out,
                      ref_lse)


@pytest.mark.parametrize("kv", ["int8", "fp8_e4m3"])
def test_8bit_large_ragged_batch(kv):
    """Hundreds of ragged sequences (uniform splits, no length-aware
    pieces above 64 sequences), paged with poisoned tails, at the planned
    and forced split counts."""
    g = torch.Generator().manual_seed(193)
    lens = torch.randint(0, 700, (300,), generator=g)
    lens[::37] = 2000
    w = workloads.make("bigbatch8", seed=193, batch=300, num_q_heads=8,
                       num_kv_heads=2, head_dim=128, max_seq_len=2000,
                       seq_lens=lens.tolist(), paged=True, poison_tail=True,
                       kv_dtype=kv)
    ref_out, ref_lse = oracle_attention(w)
    t = device_inputs(w)
    planned = fb.fd_plan_splits(shape_of(w), num_cus(), w.sum_seq_len())
    for S in sorted({planned, 1, 4}):
        out, lse = gpu_attention(w, S, t)
        assert_parity(f"bigbatch8-{kv}/S={S}", kv, out, lse, ref_out,
                      ref_lse)


@pytest.mark.parametrize("batch", [2, 64, 65])
def test_int8_length_aware_pieces_at_the_batch_limit(batch):
    """int8 batches run the pieces kernel with 4 waves up to 64 sequences
    and the uniform splits with 8 above."""
    g = torch.Generator().manual_seed(194 + batch)
    lens = torch.randint(1, 3000, (batch,), generator=g)
    lens[0] = 3000
    w = workloads.make("pieces_i8", seed=194 + batch, batch=batch,
                       num_q_heads=32, num_kv_heads=8, head_dim=128,
                       max_seq_len=3000, seq_lens=lens.tolist(), paged=True,
                       poison_tail=True, kv_dtype="int8")
    S = max(2, fb.fd_plan_splits(shape_of(w), num_cus(), w.sum_seq_len()))
    check(w, S)


@pytest.mark.parametrize("batch", [63, 64, 65])
def test_length_aware_pieces_at_the_batch_limit(batch):
    """Batched calls cut sequences by their lengths when the batch fits one
    lane of a wave (<= 64 sequences) and fall back to
    uniform splits above; empty sequences and single-token ones included."""
    g = torch.Generator().manual_seed(93)
    lens = torch.randint(0, 700, (batch,), generator=g)
    lens[:3] = torch.tensor([0, 1, 699])
    w = workloads.make("bal", seed=93, batch=batch, num_q_heads=4,
                       num_kv_heads=1, head_dim=128, max_seq_len=700,
                       seq_lens=lens.tolist(), paged=True, poison_tail=True)
    ref_out, ref_lse = oracle_attention(w)
    t = device_inputs(w)
    for S in (2, 5, 44):
        out, lse = gpu_attention(w, S, t)
        assert_parity(f"bal{batch}/S={S}", "bf16", out, lse, ref_out, ref_lse)


# ------------------------------------------------- graphs and streams

@pytest.mark.parametrize("name,over", [
    ("long_gqa_64k", dict(max_seq_len=8192)),
    ("ragged_paged", dict(batch=6, max_seq_len=5000, min_seq_len=1)),
    ("long_gqa_64k_fp8", dict(max_seq_len=8192)),
    ("long_gqa_64k_int8", dict(max_seq_len=8192)),
])
def test_graph_replays_match_eager(name, over):
    """The calls enqueue kernels only (no allocation, no memset), so they
    can be captured in a graph: every replay, with eager work and
    synchronisations in between, must reproduce the eager result bitwise."""
    w = workloads.make(name, **over)
    t = device_inputs(w)
    S = max(2, fb.fd_plan_splits(shape_of(w), num_cus(), w.sum_seq_len()))
    eager_out, eager_lse = gpu_attention(w, S, t)
    shape = shape_of(w)
    out = torch.zeros(w.batch, w.num_q_heads, w.head_dim, device="cuda")
    lse = torch.zeros(w.batch, w.num_q_heads, device="cuda")
    ws = torch.empty(max(fb.fd_workspace_size(shape, S), 16),
                     dtype=torch.uint8, device="cuda")

    def call():
        if w.cache_dtype in ("fp8_e4m3", "int8"):
            q8 = (fb.fd_decode_attn_fp8 if w.cache_dtype == "fp8_e4m3"
                  else fb.fd_decode_attn_int8)
            q8(shape, t["q"], t["k"], t["v"], t["ks"], t["vs"], t["bt"],
               t["seq_lens"], S, ws, out, lse)
        else:
            fb.fd_decode_attn(shape, t["q"], t["k"], t["v"], t["bt"],
                              t["seq_lens"], S, ws, out, lse)
    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    print(f"[gpu] graph capture {name} S={S}", flush=True)
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            call()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws.fill_(0xFF)                       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().double().numpy(), eager_out), rep
        assert np.array_equal(lse.cpu().double().numpy(), eager_lse), rep


def test_concurrent_streams():
    """Two calls with their own workspaces on two streams (default
    priority) overlap and both match the oracle."""
    ws_ = [workloads.make("long_gqa_64k", max_seq_len=4096),
           workloads.make("ragged_paged", seed=94, batch=5, max_seq_len=3000,
                          min_seq_len=1)]
    refs = [oracle_attention(w) for w in ws_]
    ts = [device_inputs(w) for w in ws_]
    outs = []
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for w, t, st in zip(ws_, ts, streams):
        shape = shape_of(w)
        S = fb.fd_plan_splits(shape, num_cus(), w.sum_seq_len())
        out = torch.empty(w.batch, w.num_q_heads, w.head_dim, device="cuda")
        lse = torch.empty(w.batch, w.num_q_heads, device="cuda")
        ws = torch.empty(max(fb.fd_workspace_size(shape, S), 16),
                         dtype=torch.uint8, device="cuda")
        st.wait_stream(torch.cuda.current_stream())
        print(f"[gpu] stream call {w.name} S={S}", flush=True)
        with torch.cuda.stream(st):
            for _ in range(5):
                fb.fd_decode_attn(shape, t["q"], t["k"], t["v"], t["bt"],
                                  t["seq_lens"], S, ws, out, lse)
        outs.append((out, lse))
    torch.cuda.synchronize()
    for w, (out, lse), (ro, rl) in zip(ws_, outs, refs):
        assert_parity(f"stream-{w.name}", w.cache_dtype,
                      out.cpu().double().numpy(), lse.cpu().double().numpy(),
                      ro, rl)


def test_convenience_wrapper_e4m3_cache():
    import split_kv_long_amd as fd
    w = workloads.make("long_gqa_64k_fp8", max_seq_len=5000)
    t = device_inputs(w)
    out, lse = fd.decode_attention(t["q"], t["k"], t["v"], t["seq_lens"],
                                   return_lse=True, k_scale=t["ks"],
                                   v_scale=t["vs"])
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_attention(w)
    assert_parity("wrapper-fp8", "fp8_e4m3", out.cpu().double().numpy(),
                  lse.cpu().double().numpy(), ref_out, ref_lse)


@pytest.mark.parametrize("bs", [32, 256])
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_larger_page_sizes(bs, kv):
    """Pages of 32 and 256 tokens: splits are rounded to whole pages, and
    16-token subtiles start inside a page."""
    lens = [1, 31, 33, 255, 257, 1000, 0, 2047]
    w = workloads.make("pages", seed=95, batch=len(lens), num_q_heads=16,
                       num_kv_heads=2, head_dim=128, max_seq_len=2048,
                       paged=True, block_size=bs, seq_lens=lens,
                       poison_tail=True,
                       kv_dtype=None if kv == "bf16" else kv)
    for S in (1, 3, 8):
        check(w, S)
