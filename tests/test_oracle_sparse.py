"""Pins for the block-sparse oracle (low-bit key summary, top-delta block
filter per split, exact attention over the kept blocks).

The "Faster Than Flash" page prints no worked example, so each pin checks
the oracle against something it does not compute itself: the nearest-integer
property of the quantizer, hand-packed nibbles, the dense oracle (delta =
inf, one block per split), torch's float64 SDPA with a mask built from the
kept blocks, brute-force estimates by explicit loops, invariants of the
keep rule, hand-derived estimates and kept sets on inputs every step
represents exactly (``tests/golden/sparse_keep.json``), and the bound the
4-bit keys and 8-bit query put on an estimate's error against the block's
true largest logit. The last tests plant plausible mistakes in copies of
the keep step and show each is caught (the unit mistakes -- the estimate
left without its logit scale, delta used without conversion -- by a pin
other than the brute-force restatement).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import sparse as osp
import workloads


def _bf16(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------- quantizer

def test_quantizer_nearest_integer_and_range():
    rng = np.random.default_rng(0)
    for trial in range(50):
        n = int(rng.integers(1, 17))
        x = rng.standard_normal((n, 64)) * 10 ** rng.uniform(-3, 3)
        bits = _bf16(x)
        xv = oracle.decode_values(bits, "bf16")
        codes, scale = osp.quantize_block(bits)
        amax = np.abs(xv).max()
        assert codes.min() >= -7 and codes.max() <= 7
        # nearest integer to 7 x / amax (float64; ties may go either way)
        assert np.all(np.abs(7.0 * xv / amax - codes) <= 0.5 + 1e-6)
        i = np.unravel_index(np.abs(xv).argmax(), xv.shape)
        assert abs(codes[i]) == 7
        assert abs(float(scale) * 7 - amax) <= 1e-6 * amax


def test_quantizer_zero_block():
    codes, scale = osp.quantize_block(_bf16(np.zeros((16, 8))))
    assert not codes.any() and scale == 0


def test_int4_packing_by_hand():
    assert osp.pack_int4(np.array([1, -1])).tolist() == [0xF1]
    assert osp.pack_int4(np.array([-8, 7])).tolist() == [0x78]
    assert osp.pack_int4(np.array([0, 3, -2, 5])).tolist() == [0x30, 0x5E]
    allc = np.arange(-8, 8)
    pairs = np.stack(np.meshgrid(allc, allc), -1).reshape(-1, 2)
    assert np.array_equal(osp.unpack_int4(osp.pack_int4(pairs)), pairs)


def test_summary_records_by_hand():
    """Record bytes D/8 * (n + 16 p) .. hold piece p of row n."""
    D = 64                                        # 8-byte pieces, 512 B
    rec = np.arange(8 * D, dtype=np.int64) % 251
    rows = osp.records_to_rows(rec.astype(np.uint8), D)
    assert rows.shape == (16, D // 2)
    for n in (0, 5, 15):
        for p in range(4):
            assert rows[n, 8 * p:8 * p + 8].tolist() == \
                [(8 * (n + 16 * p) + i) % 251 for i in range(8)]


def test_key_summary_paged_equals_contiguous():
    w = workloads.make("ragged_paged", seed=51, batch=3, num_q_heads=4,
                       num_kv_heads=2, head_dim=32, max_seq_len=100,
                       min_seq_len=1)
    c = workloads.to_contiguous(w)
    a, b = w.numpy_view(), c.numpy_view()
    cp, sp = osp.key_summary(a["k"], a["seq_lens"], a["block_table"], 16)
    cc, sc = osp.key_summary(b["k"], b["seq_lens"])
    for bb in range(3):
        n = int(a["seq_lens"][bb])
        for h in range(2):
            rows = oracle.history_rows(cp, bb, h, 0, n, a["block_table"], 16)
            assert np.array_equal(rows, cc[bb, h, :n])
            for j in range(-(-n // 16)):
                blk = a["block_table"][bb, j]
                assert sp[blk, h, 0] == sc[bb, h, j]


# ---------------------------------------------------------- checks proper

def _case(seed, B=2, Hq=4, Hkv=2, D=32, L=200, lens=(200, 77), needles=None):
    w = workloads.make("sp", seed=seed, batch=B, num_q_heads=Hq,
                       num_kv_heads=Hkv, head_dim=D, max_seq_len=L,
                       seq_lens=list(lens), needles=needles,
                       needle_logit=12.0)
    a = w.numpy_view()
    codes, scales = osp.key_summary(a["k"], a["seq_lens"])
    return a, codes, scales


def check_dense_limit(fn):
    """delta = inf keeps everything: the dense oracle's result."""
    a, codes, scales = _case(60)
    for S in (1, 3):
        out, lse, _, kept = fn(a["q"], a["k"], a["v"], a["seq_lens"], codes,
                               scales, delta=math.inf, num_splits=S,
                               max_seq_len=200)
        ref = oracle.decode_attention(a["q"], a["k"], a["v"], a["seq_lens"],
                                      dtype="bf16")
        assert np.allclose(out, ref[0], atol=1e-13)
        assert np.allclose(lse, ref[1], atol=1e-13)


def check_one_block_per_split_is_dense(fn):
    """With one 16-token block per split every split keeps its only block."""
    a, codes, scales = _case(61, L=96, lens=(96, 50))
    out, lse, _, kept = fn(a["q"], a["k"], a["v"], a["seq_lens"], codes,
                           scales, delta=0.0, num_splits=6, max_seq_len=96)
    ref = oracle.decode_attention(a["q"], a["k"], a["v"], a["seq_lens"],
                                  dtype="bf16")
    assert np.allclose(out, ref[0], atol=1e-13)


def check_brute_force_keep(fn):
    """Estimates by explicit loops (int8 query, integer dots, float32
    products in the stated order) and the keep rule written out per block."""
    a, codes, scales = _case(62, B=1, Hq=4, Hkv=2, D=16, L=80, lens=(75,))
    q = oracle.decode_values(a["q"], "bf16")
    sl2 = np.float32(float(np.float32(1.0 / math.sqrt(16))) * 1.4426950408889634)
    for delta in (0.0, 0.3, 1.0):
        d2 = np.float32(float(np.float32(delta)) * 1.4426950408889634)
        out, lse, est, kept = fn(a["q"], a["k"], a["v"], a["seq_lens"],
                                 codes, scales, delta=delta, num_splits=2,
                                 max_seq_len=80)
        # P = 48: split 0 = blocks 0..2, split 1 = blocks 3..4 (75 tokens)
        for kvh in range(2):
            e = {}
            for h in (2 * kvh, 2 * kvh + 1):
                amax = max(abs(float(x)) for x in q[0, h])
                inv = np.float32(np.float32(127) / np.float32(amax))
                sq = np.float32(np.float32(amax) / np.float32(127))
                q8 = [int(np.rint(np.float32(np.float32(x) * inv)))
                      for x in q[0, h]]
                assert max(abs(x) for x in q8) == 127
                for j in range(5):
                    best = None
                    for t in range(16 * j, min(16 * j + 16, 75)):
                        acc = 0
                        for d in range(16):
                            acc += q8[d] * int(codes[0, kvh, t, d])
                        best = acc if best is None else max(best, acc)
                    v = np.float32(np.float32(best) * sq)
                    v = np.float32(v * np.float32(scales[0, kvh, j]))
                    e[h, j] = np.float32(v * sl2)
                    assert est[0, h, j] == e[h, j]
            for blocks in ((0, 1, 2), (3, 4)):
                for j in blocks:
                    want = any(e[h, j] >= np.float32(
                        max(e[h, i] for i in blocks) - d2)
                        for h in (2 * kvh, 2 * kvh + 1))
                    assert kept[0, kvh, j] == want, (delta, kvh, j)


def test_query_quantizer_nearest_integer_and_range():
    rng = np.random.default_rng(3)
    for trial in range(50):
        x = rng.standard_normal(64) * 10 ** rng.uniform(-3, 3)
        bits = _bf16(x)
        xv = oracle.decode_values(bits, "bf16")
        q8, s = osp.quantize_query(bits)
        amax = np.abs(xv).max()
        assert q8.min() >= -127 and q8.max() <= 127
        assert np.all(np.abs(127.0 * xv / amax - q8) <= 0.5 + 1e-5)
        assert abs(q8[np.abs(xv).argmax()]) == 127
        assert abs(float(s) * 127 - amax) <= 1e-6 * amax
    q8, s = osp.quantize_query(_bf16(np.zeros(8)))
    assert not q8.any() and s == 0


def check_masked_sdpa(fn):
    """The result is torch's float64 SDPA restricted to the kept tokens."""
    a, codes, scales = _case(63, needles=[5, 130])
    out, lse, _, kept = fn(a["q"], a["k"], a["v"], a["seq_lens"], codes,
                           scales, delta=1.5, num_splits=4, max_seq_len=200)
    q = torch.from_numpy(oracle.decode_values(a["q"], "bf16"))
    k = torch.from_numpy(oracle.decode_values(a["k"], "bf16"))
    v = torch.from_numpy(oracle.decode_values(a["v"], "bf16"))
    assert 0 < kept.sum() < kept.size
    for b in range(2):
        n = int(a["seq_lens"][b])
        for h in range(4):
            kvh = h // 2
            mask = torch.tensor([bool(kept[b, kvh, t // 16]) for t in range(n)])
            ref = torch.nn.functional.scaled_dot_product_attention(
                q[b, h][None, None, None], k[b, kvh, :n][None, None],
                v[b, kvh, :n][None, None], attn_mask=mask[None, None, None])
            assert np.allclose(out[b, h], ref[0, 0, 0].numpy(), atol=1e-12)


def check_keep_invariants(fn):
    a, codes, scales = _case(64, L=512, lens=(512, 300), needles=[200])
    prev = None
    for delta in (0.0, 0.5, 2.0, 8.0):
        _, _, est, kept = fn(a["q"], a["k"], a["v"], a["seq_lens"], codes,
                             scales, delta=delta, num_splits=4,
                             max_seq_len=512)
        if prev is not None:
            assert np.all(kept >= prev)            # monotone in delta
        prev = kept
        for b, n in ((0, 512), (1, 300)):
            for s in range(4):
                j0, j1 = 8 * s, min(8 * s + 8, -(-n // 16))
                if j1 <= j0:
                    continue
                for h in range(4):           # every head's top block kept
                    top = j0 + int(np.nanargmax(est[b, h, j0:j1]))
                    assert kept[b, h // 2, top]
    # the needle (logit 12 for head 0) dominates its split at delta 0
    _, _, est, kept = fn(a["q"], a["k"], a["v"], a["seq_lens"], codes,
                         scales, delta=0.0, num_splits=4, max_seq_len=512)
    assert kept[0, 0, 200 // 16] and kept[1, 0, 200 // 16]


GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "sparse_keep.json")))


def _golden_inputs():
    """The inputs of tests/golden/sparse_keep.json, built from its recipe."""
    c = GOLDEN["construction"]
    D, L = c["head_dim"], c["seq_len"]
    q = np.zeros((1, 2, D), np.float32)
    q[0, 0, 0] = q[0, 1, 1] = 31.75
    k = np.zeros((1, 1, L, D), np.float32)
    for j in range(c["blocks"]):
        for t in range(16):
            i = 16 * j + t
            k[0, 0, i, 0] = max(c["c0"][j] - t % 3, -7) / 4
            k[0, 0, i, 1] = max(c["c1"][j] - t % 2, -7) / 4
            if t == 0:
                k[0, 0, i, 63] = -7 / 4
    v = np.ones((1, 1, L, D), np.float32)
    v[0, 0, :, 0] = np.arange(L)
    qb, kb, vb = _bf16(q), _bf16(k), _bf16(v)
    # every value is exact in bfloat16, so the hand derivation applies
    assert np.array_equal(oracle.decode_values(kb, "bf16"), k)
    assert np.array_equal(oracle.decode_values(qb, "bf16"), q)
    return qb, kb, vb


def check_hand_derived_keep(fn):
    """Estimates equal the hand-derived largest logits times log2 e, and
    the kept sets match the ones worked out by hand from the logits."""
    qb, kb, vb = _golden_inputs()
    codes, scales = osp.key_summary(kb, [64])
    assert np.all(scales == np.float32(0.25))       # amax 7/4 in every block
    logit = np.array([GOLDEN["max_logit"]["head0"],
                      GOLDEN["max_logit"]["head1"]])
    for case in GOLDEN["keep"]:
        delta = math.inf if case["delta"] == "inf" else float(case["delta"])
        _, _, est, kept = fn(qb, kb, vb, [64], codes, scales, delta=delta,
                             num_splits=case["num_splits"], max_seq_len=64)
        assert kept[0, 0, :4].astype(int).tolist() == case["kept"], case
        want = logit * 1.4426950408889634
        assert np.allclose(est[0, :, :4], want,
                           rtol=GOLDEN["est_tol_rel"], atol=0), case


def check_estimate_error_bound(fn):
    """|est * ln 2 - T| <= the quantization bound, T = the block's largest
    logit over its attended tokens (float64 from the bf16 values). With
    amax_q = 127 s_q, amax_j = 7 scale_j, each key off its code by at most
    scale_j / 2 and the query by s_q / 2, a dot product moves by at most
    D * s_q * scale_j * (127/2 + 7/2 + 1/4), and so does a maximum."""
    for seed, D, L, lens in ((65, 64, 160, (160, 97)), (66, 128, 96, (96,))):
        a, codes, scales = _case(seed, B=len(lens), Hq=4, Hkv=2, D=D, L=L,
                                 lens=lens)
        _, _, est, _ = fn(a["q"], a["k"], a["v"], a["seq_lens"], codes,
                          scales, delta=1.0, num_splits=2, max_seq_len=L)
        q = oracle.decode_values(a["q"], "bf16")
        k = oracle.decode_values(a["k"], "bf16")
        sc = 1.0 / math.sqrt(D)
        checked = 0
        for b, n in enumerate(lens):
            for h in range(4):
                sq = np.abs(q[b, h]).max() / 127.0
                for j in range(-(-n // 16)):
                    rows = k[b, h // 2, 16 * j:min(16 * j + 16, n)]
                    sj = np.abs(rows).max() / 7.0
                    T = sc * (rows @ q[b, h]).max()
                    bound = sc * D * sq * sj * 67.25 * (1 + 1e-5) \
                        + 1e-6 * abs(T) + 1e-30
                    assert abs(float(est[b, h, j]) * math.log(2) - T) \
                        <= bound, (seed, b, h, j)
                    checked += 1
        assert checked > 20


CHECKS = [check_dense_limit, check_one_block_per_split_is_dense,
          check_brute_force_keep, check_masked_sdpa, check_keep_invariants,
          check_hand_derived_keep, check_estimate_error_bound]


def test_reference_passes_every_check():
    for chk in CHECKS:
        chk(osp.sparse_decode_attention)


def _mutant(kind):
    """sparse_decode_attention with one plausible mistake in the keep step."""
    def fn(q, k, v, seq_lens, codes, scales, *, delta, num_splits,
           max_seq_len, scale=None, block_table=None, block_size=0):
        qf = oracle.decode_values(q, "bf16")
        B, Hq, D = qf.shape
        Hkv = k.shape[1]
        G = Hq // Hkv
        sc = 1.0 / math.sqrt(D)
        P = oracle.split_length(max_seq_len, num_splits)
        nblk = -(-max_seq_len // 16)
        out = np.zeros((B, Hq, D))
        lse = np.full((B, Hq), -np.inf)
        est = np.full((B, Hq, nblk), np.nan)
        kept = np.zeros((B, Hkv, nblk), dtype=bool)
        for b in range(B):
            n = int(seq_lens[b])
            for kvh in range(Hkv):
                heads = slice(kvh * G, (kvh + 1) * G)
                qq = [osp.quantize_query(q[b, h])
                      for h in range(kvh * G, (kvh + 1) * G)]
                q8 = np.stack([x[0] for x in qq])
                sl2 = osp.log2_units(sc)
                for j in range(-(-n // 16)):
                    c = codes[b, kvh, 16 * j:min(16 * j + 16, n)].astype(np.int64)
                    sj = np.float32(1.0) if kind == "no_block_scale" else \
                        np.float32(scales[b, kvh, j])
                    dots = q8 @ c.T
                    red = dots.mean(axis=1) if kind == "mean_not_max" \
                        else dots.max(axis=1)
                    for g in range(G):
                        e = np.float32(np.float32(red[g]) * qq[g][1])
                        e = np.float32(e * sj)
                        est[b, kvh * G + g, j] = (
                            e if kind == "no_logit_scale"
                            else np.float32(e * sl2))
                for s_ in range(num_splits):
                    j0 = s_ * P // 16
                    j1 = -(-min((s_ + 1) * P, n) // 16)
                    if kind == "split_off_by_one":
                        j1 = max(j0, j1 - 1)
                    if j1 <= j0:
                        continue
                    e = est[b, heads, j0:j1].astype(np.float32)
                    M = e.max(axis=1, keepdims=True)
                    if kind == "global_threshold":
                        M = np.nanmax(est[b, heads], axis=1,
                                      keepdims=True).astype(np.float32)
                    d2 = osp.log2_units(delta) if math.isfinite(delta) \
                        else np.float32(np.inf)
                    if kind == "delta_not_converted":
                        d2 = np.float32(delta)
                    ok = e >= (M - d2).astype(np.float32)
                    kept[b, kvh, j0:j1] = (ok.all(axis=0) if kind == "all_heads"
                                           else ok.any(axis=0))
                toks = [t for t in range(n) if kept[b, kvh, t // 16]]
                if not toks:
                    continue
                kr = oracle.decode_values(k[b, kvh, toks], "bf16")
                vr = oracle.decode_values(v[b, kvh, toks], "bf16")
                o, l = oracle.softmax_attention(sc * (qf[b, heads] @ kr.T), vr)
                out[b, heads] = o
                lse[b, heads] = l
        return out, lse, est, kept
    return fn


MUTANTS = ["no_block_scale", "mean_not_max", "split_off_by_one",
           "global_threshold", "all_heads", "no_logit_scale",
           "delta_not_converted"]


def test_mutant_copy_without_mistake_passes():
    fn = _mutant("none")
    for chk in CHECKS:
        chk(fn)


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_is_caught(kind):
    fn = _mutant(kind)
    failed = []
    for chk in CHECKS:
        try:
            with np.errstate(all="ignore"):
                chk(fn)
        except (AssertionError, IndexError, ValueError):
            failed.append(chk.__name__)
    assert failed, f"mutant {kind} passed every sparse pin"


@pytest.mark.parametrize("kind", ["no_logit_scale", "delta_not_converted"])
def test_unit_mistakes_caught_without_the_restatement(kind):
    """The estimate's units and delta's conversion are pinned by the
    hand-derived cases and the error bound, not only by the brute-force
    check that restates the oracle's own arithmetic."""
    fn = _mutant(kind)
    failed = []
    for chk in CHECKS:
        if chk is check_brute_force_keep:
            continue
        try:
            with np.errstate(all="ignore"):
                chk(fn)
        except (AssertionError, IndexError, ValueError):
            failed.append(chk.__name__)
    assert failed, f"mutant {kind} passed every pin but the restatement"


# ------------------------------------------------------------- E4M3 caches
# Every E4M3 value is a bf16 value, and a power-of-two scale only moves the
# exponent, so with such scales the E4M3 path must reproduce the bf16 path
# (pinned above) on the dequantized values exactly: the same summary codes,
# scales equal to the bf16 summary's, the same estimates and kept sets, the
# same result.

KS = np.array([2.0 ** -3, 2.0 ** 2])      # per kv head
VS = np.array([2.0 ** 1, 2.0 ** -4])


def _e4m3_view(seed, lens=(200, 77), L=200, paged=False):
    w = workloads.make("sp8", seed=seed, batch=len(lens), num_q_heads=4,
                       num_kv_heads=2, head_dim=32, max_seq_len=L,
                       seq_lens=list(lens), needles=[3, L // 2],
                       needle_logit=12.0, kv_dtype="fp8_e4m3", paged=paged)
    return w.numpy_view()


def _bf16_equivalent(codes, per_head):
    """E4M3 codes times a power of two per kv head (axis 1), as bf16 bits."""
    x = oracle.fp8_e4m3_to_f64(codes) * per_head[None, :, None, None]
    return _bf16(x)


@pytest.mark.parametrize("paged", [False, True])
def test_e4m3_summary_is_the_bf16_summary_of_the_scaled_keys(paged):
    a = _e4m3_view(61, paged=paged)
    bt, bs = a["block_table"], a["block_size"] if paged else 0
    c8, s8 = osp.key_summary(a["k"], a["seq_lens"], bt, bs,
                             kv_dtype="fp8_e4m3", k_scale=KS)
    kb = _bf16_equivalent(a["k"], KS)
    cb, sb = osp.key_summary(kb, a["seq_lens"], bt, bs)
    assert np.array_equal(c8, cb)
    assert np.array_equal(s8, sb)
    assert np.any(s8 != 0)
    # Planted mistake: the key scale left out of the summary. The codes do
    # not see it (they are scale-free), the block scales do.
    _, s_bad = osp.key_summary(a["k"], a["seq_lens"], bt, bs,
                               kv_dtype="fp8_e4m3", k_scale=np.ones(2))
    assert not np.array_equal(s_bad, sb)


@pytest.mark.parametrize("delta,S", [(0.5, 1), (2.0, 3), (math.inf, 2)])
def test_e4m3_sparse_attention_equals_bf16_on_the_same_values(delta, S):
    a = _e4m3_view(62)
    c8, s8 = osp.key_summary(a["k"], a["seq_lens"], kv_dtype="fp8_e4m3",
                             k_scale=KS)
    r8 = osp.sparse_decode_attention(
        a["q"], a["k"], a["v"], a["seq_lens"], c8, s8, delta=delta,
        num_splits=S, max_seq_len=200, scale=a["scale"],
        kv_dtype="fp8_e4m3", k_scale=KS, v_scale=VS)
    kb, vb = _bf16_equivalent(a["k"], KS), _bf16_equivalent(a["v"], VS)
    cb, sb = osp.key_summary(kb, a["seq_lens"])
    rb = osp.sparse_decode_attention(
        a["q"], kb, vb, a["seq_lens"], cb, sb, delta=delta, num_splits=S,
        max_seq_len=200, scale=a["scale"])
    for x8, xb in zip(r8, rb):
        assert np.array_equal(x8, xb, equal_nan=True)
    if math.isinf(delta):       # every block kept: the dense E4M3 oracle
        ref = oracle.decode_attention(
            a["q"], a["k"], a["v"], a["seq_lens"], dtype="bf16",
            kv_dtype="fp8_e4m3", k_scale=KS, v_scale=VS, scale=a["scale"])
        assert np.abs(r8[0] - ref[0]).max() < 1e-12
        assert np.abs(r8[1] - ref[1]).max() < 1e-12


# ------------------------------------------------------------- int8 caches
# An int8 code has at most 8 significant bits, so code x 2^e is a bf16
# value: with power-of-two per-position scales the int8 path must equal the
# bf16 path on the dequantized values exactly, as for E4M3 above.

def _int8_view(seed, paged=False, lens=(200, 77), L=200):
    w = workloads.make("sp8", seed=seed, batch=len(lens), num_q_heads=4,
                       num_kv_heads=2, head_dim=32, max_seq_len=L,
                       seq_lens=list(lens), needles=[3, L // 2],
                       needle_logit=12.0, kv_dtype="int8", paged=paged)
    a = w.numpy_view()
    rng = np.random.default_rng(seed)
    a["k_scale"] = 2.0 ** rng.integers(-6, 3, size=a["k_scale"].shape)
    a["v_scale"] = 2.0 ** rng.integers(-6, 3, size=a["v_scale"].shape)
    return a


def _bf16_per_position(codes, scale):
    """int8 codes times their per-position scale (cache layout without
    head_dim, rows possibly padded), as bf16 bits."""
    n = codes.shape[2]
    x = oracle.int8_to_f64(codes) * scale[:, :, :n, None]
    return _bf16(x)


@pytest.mark.parametrize("paged", [False, True])
def test_int8_summary_is_the_bf16_summary_of_the_scaled_keys(paged):
    a = _int8_view(63, paged=paged)
    bt, bs = a["block_table"], a["block_size"] if paged else 0
    c8, s8 = osp.key_summary(a["k"], a["seq_lens"], bt, bs, kv_dtype="int8",
                             k_scale=a["k_scale"])
    cb, sb = osp.key_summary(_bf16_per_position(a["k"], a["k_scale"]),
                             a["seq_lens"], bt, bs)
    assert np.array_equal(c8, cb)
    assert np.array_equal(s8, sb)
    assert np.any(s8 != 0)
    # Planted mistake: every position takes its neighbour's scale.
    shifted = np.roll(a["k_scale"], 1, axis=2)
    c_bad, s_bad = osp.key_summary(a["k"], a["seq_lens"], bt, bs,
                                   kv_dtype="int8", k_scale=shifted)
    assert not (np.array_equal(c_bad, cb) and np.array_equal(s_bad, sb))


@pytest.mark.parametrize("delta,S,paged", [(0.5, 1, False), (2.0, 3, True),
                                           (math.inf, 2, False)])
def test_int8_sparse_attention_equals_bf16_on_the_same_values(delta, S, paged):
    a = _int8_view(64, paged=paged)
    bt, bs = a["block_table"], a["block_size"] if paged else 0
    c8, s8 = osp.key_summary(a["k"], a["seq_lens"], bt, bs, kv_dtype="int8",
                             k_scale=a["k_scale"])
    r8 = osp.sparse_decode_attention(
        a["q"], a["k"], a["v"], a["seq_lens"], c8, s8, delta=delta,
        num_splits=S, max_seq_len=200, scale=a["scale"], block_table=bt,
        block_size=bs, kv_dtype="int8", k_scale=a["k_scale"],
        v_scale=a["v_scale"])
    kb = _bf16_per_position(a["k"], a["k_scale"])
    vb = _bf16_per_position(a["v"], a["v_scale"])
    cb, sb = osp.key_summary(kb, a["seq_lens"], bt, bs)
    rb = osp.sparse_decode_attention(
        a["q"], kb, vb, a["seq_lens"], cb, sb, delta=delta, num_splits=S,
        max_seq_len=200, scale=a["scale"], block_table=bt, block_size=bs)
    for x8, xb in zip(r8, rb):
        assert np.array_equal(x8, xb, equal_nan=True)
    if math.isinf(delta):       # every block kept: the dense int8 oracle
        ref = oracle.decode_attention(
            a["q"], a["k"], a["v"], a["seq_lens"], dtype="bf16",
            kv_dtype="int8", k_scale=a["k_scale"], v_scale=a["v_scale"],
            scale=a["scale"], block_table=bt, block_size=bs)
        assert np.abs(r8[0] - ref[0]).max() < 1e-12
        assert np.abs(r8[1] - ref[1]).max() < 1e-12


# ------------------------------------------------------------- split bounds

def test_split_boundaries_follow_the_page_size():
    # Splits are whole pages: P = ceil(ceil(L / S) / g) * g with
    # g = max(16, page size), the dense path's boundaries. With 64-token
    # pages, L = 5000 and S = 3 that is 1728 (16-token rounding would give
    # 1680); the per-split maxima, and so the kept sets, depend on it.
    assert oracle.split_length(5000, 3, 16) == 1680
    assert oracle.split_length(5000, 3, 32) == 1696
    assert oracle.split_length(5000, 3, 64) == 1728
    w = workloads.make("spb", seed=65, batch=1, num_q_heads=2,
                       num_kv_heads=1, head_dim=32, max_seq_len=5000,
                       seq_lens=[5000], paged=True, block_size=64,
                       needles=[1700], needle_logit=12.0)
    a = w.numpy_view()
    codes, scales = osp.key_summary(a["k"], a["seq_lens"], a["block_table"],
                                    64)
    _, _, est, kept = osp.sparse_decode_attention(
        a["q"], a["k"], a["v"], a["seq_lens"], codes, scales, delta=0.0,
        num_splits=3, max_seq_len=5000, scale=a["scale"],
        block_table=a["block_table"], block_size=64)
    # delta = 0 keeps, per split, each head's best block: recompute with
    # the page-aligned boundaries by explicit loops.
    want = np.zeros(kept.shape[2], dtype=bool)
    P = 1728
    for s in range(3):
        j0, j1 = s * P // 16, min(-(-min((s + 1) * P, 5000) // 16),
                                  kept.shape[2])
        for h in range(2):
            e = est[0, h, j0:j1].astype(np.float32)
            want[j0:j1] |= e >= e.max()
    assert np.array_equal(kept[0, 0], want)
    # The needle's block (1700 // 16 = 106) is in split 0 here, in split 1
    # with 16-token rounding (1680): it must be the best of split 0.
    assert kept[0, 0, 106]
