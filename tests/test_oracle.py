"""Pins for the float64 oracle, independent of the oracle's own formulas.

Each pin checks the oracle against something it does not compute itself:
hand-derived closed forms, a library routine (torch's scaled dot-product
attention in float64), brute force over every way to split a tiny history,
exact special cases and invariants of softmax attention. The last test plants
plausible mistakes in copies of the oracle and shows each is caught.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oa
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _rand(rng, *shape):
    return rng.standard_normal(shape).astype(np.float32)


# ---------------------------------------------------------------- pin checks
# Each check takes the attention function under test so the same check can be
# run against deliberately broken copies.

def check_closed_forms(attn):
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        q = np.array(c["q"], dtype=np.float32)
        k = np.array(c["k"], dtype=np.float32)
        v = np.array(c["v"], dtype=np.float32)
        out, lse = attn(q, k, v, np.array(c["seq_lens"]), dtype="f32",
                        scale=c["scale"])
        exp_out = np.array(c["out"], dtype=np.float64)
        exp_lse = np.array([[float(x) for x in row] for row in c["lse"]])
        assert np.allclose(out, exp_out, rtol=0, atol=c["tol"]), c["name"]
        fin = np.isfinite(exp_lse)
        assert np.array_equal(np.isneginf(lse), np.isneginf(exp_lse)), c["name"]
        assert np.allclose(lse[fin], exp_lse[fin], rtol=0, atol=c["tol"]), c["name"]


def check_library_sdpa(attn, seed=0):
    """torch scaled_dot_product_attention in float64, KV heads repeated."""
    rng = np.random.default_rng(seed)
    for (B, Hq, Hkv, D, L) in [(2, 8, 2, 16, 37), (1, 4, 4, 8, 5),
                               (3, 6, 3, 32, 70)]:
        q = _rand(rng, B, Hq, D)
        k = _rand(rng, B, Hkv, L, D)
        v = _rand(rng, B, Hkv, L, D)
        lens = rng.integers(1, L + 1, size=B)
        for scale in (None, 0.3):
            out, lse = attn(q, k, v, lens, dtype="f32", scale=scale)
            G = Hq // Hkv
            for b in range(B):
                n = int(lens[b])
                qt = torch.from_numpy(q[b].astype(np.float64))[None, :, None, :]
                kt = torch.from_numpy(k[b, :, :n].astype(np.float64))
                vt = torch.from_numpy(v[b, :, :n].astype(np.float64))
                kt = kt.repeat_interleave(G, dim=0)[None]
                vt = vt.repeat_interleave(G, dim=0)[None]
                ref = torch.nn.functional.scaled_dot_product_attention(
                    qt, kt, vt, scale=scale)[0, :, 0, :].numpy()
                assert np.allclose(out[b], ref, rtol=0, atol=1e-12)
                sc = scale if scale else 1.0 / math.sqrt(D)
                s = torch.einsum("hd,hnd->hn", qt[0, :, 0], kt[0]) * sc
                ref_lse = torch.logsumexp(s, dim=-1).numpy()
                assert np.allclose(lse[b], ref_lse, rtol=0, atol=1e-12)


def check_gqa_equals_repeated_mha(attn, seed=1):
    rng = np.random.default_rng(seed)
    B, Hkv, G, D, L = 2, 3, 4, 16, 25
    q = _rand(rng, B, Hkv * G, D)
    k = _rand(rng, B, Hkv, L, D)
    v = _rand(rng, B, Hkv, L, D)
    lens = np.array([25, 11])
    out, lse = attn(q, k, v, lens, dtype="f32")
    out2, lse2 = attn(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1),
                      lens, dtype="f32")
    assert np.allclose(out, out2, atol=1e-14) and np.allclose(lse, lse2, atol=1e-14)


def check_paged_equals_contiguous(attn, seed=4):
    w = workloads.make("ragged_paged", seed=seed, batch=3, num_q_heads=4,
                       num_kv_heads=2, head_dim=16, max_seq_len=70,
                       min_seq_len=1, poison_tail=True)
    c = workloads.to_contiguous(w)
    a, b = w.numpy_view(), c.numpy_view()
    o1, l1 = attn(a["q"], a["k"], a["v"], a["seq_lens"], dtype="bf16",
                  block_table=a["block_table"], block_size=a["block_size"])
    o2, l2 = attn(b["q"], b["k"], b["v"], b["seq_lens"], dtype="bf16")
    assert np.all(np.isfinite(o1))
    assert np.allclose(o1, o2, atol=1e-14) and np.allclose(l1, l2, atol=1e-14)


def check_single_token(attn, seed=5):
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng, 1, 2, 8), _rand(rng, 1, 2, 4, 8), _rand(rng, 1, 2, 4, 8)
    out, lse = attn(q, k, v, np.array([1]), dtype="f32", scale=0.7)
    assert np.array_equal(out[0], v[0, :, 0].astype(np.float64))
    s0 = 0.7 * np.einsum("hd,hd->h", q[0].astype(np.float64),
                         k[0, :, 0].astype(np.float64))
    assert np.allclose(lse[0], s0, rtol=0, atol=1e-15)


def check_equal_keys_mean(attn, seed=6):
    rng = np.random.default_rng(seed)
    L, D = 33, 16
    q = _rand(rng, 1, 3, D)
    k = np.repeat(_rand(rng, 1, 1, 1, D), L, axis=2)
    v = _rand(rng, 1, 1, L, D)
    out, lse = attn(q, k, v, np.array([L]), dtype="f32")
    mean = v[0, 0].astype(np.float64).mean(axis=0)
    assert np.allclose(out[0], mean[None], rtol=0, atol=1e-12)
    s = np.einsum("hd,d->h", q[0].astype(np.float64),
                  k[0, 0, 0].astype(np.float64)) / math.sqrt(D)
    assert np.allclose(lse[0], s + math.log(L), atol=1e-12)


def check_dominant_logit(attn, seed=7):
    rng = np.random.default_rng(seed)
    L, D = 40, 8
    for gap, j in ((50.0, 0), (50.0, L - 1), (800.0, 17)):
        q = np.zeros((1, 1, D), np.float32)
        q[0, 0, 0] = 1.0
        k = np.zeros((1, 1, L, D), np.float32)
        k[0, 0, :, 0] = rng.uniform(-1, 1, L).astype(np.float32)
        k[0, 0, j, 0] = gap + 1.0
        v = _rand(rng, 1, 1, L, D)
        out, lse = attn(q, k, v, np.array([L]), dtype="f32", scale=1.0)
        bound = L * math.exp(-(gap - 0.0)) * np.abs(v).max() + 1e-15
        assert np.all(np.isfinite(out))
        assert np.allclose(out[0, 0], v[0, 0, j], rtol=0, atol=bound)
        assert abs(lse[0, 0] - (gap + 1.0)) < 1e-9


# ------------------------------------------------------------ the pins proper

def test_bf16_decode_matches_torch_on_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = oracle.bf16_bits_to_f64(bits)
    ref = (torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
           .to(torch.float64).numpy())
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    # and the sign bit really is the sign
    assert oracle.bf16_bits_to_f64(np.array([0xBF80], np.uint16))[0] == -1.0


def test_closed_forms():
    check_closed_forms(oracle.decode_attention)


def test_library_sdpa():
    check_library_sdpa(oracle.decode_attention)


def test_gqa_equals_repeated_mha():
    check_gqa_equals_repeated_mha(oracle.decode_attention)


def test_paged_equals_contiguous():
    check_paged_equals_contiguous(oracle.decode_attention)


def test_single_token_is_exact():
    check_single_token(oracle.decode_attention)


def test_equal_keys_give_mean_of_values():
    check_equal_keys_mean(oracle.decode_attention)


def test_dominant_logit_gives_its_value_row():
    check_dominant_logit(oracle.decode_attention)


def test_permuting_history_jointly_is_invariant():
    rng = np.random.default_rng(8)
    q, k, v = _rand(rng, 1, 4, 8), _rand(rng, 1, 2, 19, 8), _rand(rng, 1, 2, 19, 8)
    perm = rng.permutation(19)
    o1, l1 = oracle.decode_attention(q, k, v, [19], dtype="f32")
    o2, l2 = oracle.decode_attention(q, k[:, :, perm], v[:, :, perm], [19],
                                     dtype="f32")
    assert np.allclose(o1, o2, atol=1e-14) and np.allclose(l1, l2, atol=1e-14)


def test_convex_and_affine_in_values():
    rng = np.random.default_rng(9)
    q, k, v = _rand(rng, 2, 2, 8), _rand(rng, 2, 1, 30, 8), _rand(rng, 2, 1, 30, 8)
    lens = np.array([30, 7])
    out, _ = oracle.decode_attention(q, k, v, lens, dtype="f32")
    for b in range(2):
        vv = v[b, 0, :lens[b]]
        assert np.all(out[b] <= vv.max(axis=0) + 1e-12)
        assert np.all(out[b] >= vv.min(axis=0) - 1e-12)
    a, c = 2.5, -1.25
    out2, _ = oracle.decode_attention(q, k, (a * v.astype(np.float64) + c),
                                      lens, dtype="f32")
    # a*v + c is rounded to float32 inside the oracle's f32 decode
    out3, _ = oracle.decode_attention(
        q, k, (a * v.astype(np.float64) + c).astype(np.float32), lens,
        dtype="f32")
    assert np.allclose(out2, out3, atol=0)
    assert np.allclose(out3, a * out + c, atol=1e-5)


def test_shift_of_all_scores_moves_only_lse():
    rng = np.random.default_rng(10)
    s = rng.standard_normal((3, 12))
    vals = rng.standard_normal((12, 5))
    o1, l1 = oracle.softmax_attention(s, vals)
    o2, l2 = oracle.softmax_attention(s + 123.0, vals)
    assert np.allclose(o1, o2, atol=1e-13)
    assert np.allclose(l2 - l1, 123.0, atol=1e-12)


def test_split_then_combine_brute_force():
    """Every split of a tiny history into <= 4 contiguous chunks (empty ones
    included), in every chunk order: combining the chunk partials equals
    attention over the whole history."""
    rng = np.random.default_rng(11)
    for n in range(1, 11):
        s = rng.standard_normal((2, n)) * 3.0
        vals = rng.standard_normal((n, 4))
        full_o, full_l = oracle.softmax_attention(s, vals)
        for parts in range(1, 5):
            for cuts in itertools.combinations_with_replacement(range(n + 1),
                                                                parts - 1):
                edges = (0,) + cuts + (n,)
                chunks = [(edges[i], edges[i + 1]) for i in range(parts)]
                os_, ls_ = [], []
                for (a, b) in chunks:
                    o, l = oracle.softmax_attention(s[:, a:b], vals[a:b])
                    os_.append(o)
                    ls_.append(l)
                orders = list(itertools.permutations(range(parts)))
                for order in orders[:6]:
                    op = np.stack([os_[i] for i in order], axis=1)
                    lp = np.stack([ls_[i] for i in order], axis=1)
                    o, l = oracle.combine_partials(op, lp)
                    assert np.allclose(o, full_o, rtol=0, atol=1e-12)
                    assert np.allclose(l, full_l, rtol=0, atol=1e-12)


def test_combine_of_all_empty_is_zero_and_neg_inf():
    o, l = oracle.combine_partials(np.full((2, 3, 4), 5.0),
                                   np.full((2, 3), -np.inf))
    assert np.array_equal(o, np.zeros((2, 4))) and np.all(np.isneginf(l))


@pytest.mark.parametrize("S", [1, 2, 3, 5, 16, 40])
def test_split_partials_recombine_to_unsplit(S):
    w = workloads.make("ragged_paged", seed=12, batch=3, num_q_heads=8,
                       num_kv_heads=2, head_dim=16, max_seq_len=150,
                       min_seq_len=0)
    a = w.numpy_view()
    kw = dict(dtype="bf16", block_table=a["block_table"],
              block_size=a["block_size"])
    op, lp = oracle.split_partials(a["q"], a["k"], a["v"], a["seq_lens"], S,
                                   max_seq_len=150, **kw)
    P = oracle.split_length(150, S)
    for b in range(3):
        n = int(a["seq_lens"][b])
        nonempty = -(-n // P)
        assert np.all(np.isfinite(lp[b, :, :nonempty]))
        assert np.all(np.isneginf(lp[b, :, nonempty:]))
    o, l = oracle.combine_partials(op, lp)
    ro, rl = oracle.decode_attention(a["q"], a["k"], a["v"], a["seq_lens"], **kw)
    assert np.allclose(o, ro, atol=1e-12)
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(l))
    assert np.allclose(l[fin], rl[fin], atol=1e-12)


def test_split_length():
    assert oracle.split_length(65536, 128) == 512
    assert oracle.split_length(512, 4) == 128
    assert oracle.split_length(100, 3) == 48
    assert oracle.split_length(262144, 32) == 8192
    for L in (1, 15, 16, 17, 1000, 65536):
        for S in (1, 2, 3, 7, 64):
            P = oracle.split_length(L, S)
            assert P % 16 == 0 and P * S >= L and P - 16 < -(-L // S)


# ------------------------------------------------ planted mistakes are caught

def _mutant(kind):
    """A copy of decode_attention with one plausible mistake planted."""
    def attn(q, k, v, seq_lens, *, dtype, scale=None, block_table=None,
             block_size=0, token_range=None):
        qf = oa.decode_values(q, dtype)
        B, Hq, D = qf.shape
        Hkv = k.shape[1]
        G = Hq // Hkv
        sc = scale if scale else 1.0 / math.sqrt(D)
        if kind == "no_scale":
            sc = 1.0
        out = np.zeros((B, Hq, D))
        lse = np.full((B, Hq), -np.inf)
        for b in range(B):
            n = int(seq_lens[b])
            if kind == "off_by_one_len":
                n = min(n + 1, k.shape[2] if block_table is None else n + 1)
            if n <= 0:
                continue
            for h in range(Hq):
                kvh = (h % Hkv) if kind == "gqa_modulo" else h // G
                if block_table is not None and block_size:
                    pos = np.arange(n)
                    slot = (pos // block_size if kind == "paged_slot_swap"
                            else pos % block_size)
                    blk = np.asarray(block_table)[b, pos // block_size]
                    if kind == "paged_slot_swap":
                        slot = np.minimum(slot, block_size - 1)
                    kr = oa.decode_values(k[blk, kvh, slot], dtype)
                    vr = oa.decode_values(v[blk, kvh, slot], dtype)
                else:
                    kr = oa.decode_values(k[b, kvh, :n], dtype)
                    vr = oa.decode_values(v[b, kvh, :n], dtype)
                s = sc * (kr @ qf[b, h])
                if kind == "no_max_subtract":
                    w = np.exp(s)
                else:
                    m = s.max()
                    w = np.exp(s - m)
                z = w.sum()
                if kind == "unnormalised":
                    z = 1.0
                o = (w @ vr) / z
                if kind == "key_value_swap":
                    o = (w @ kr) / z
                out[b, h] = o
                base = 0.0 if kind == "no_max_subtract" else m
                lse[b, h] = (base + (math.log2(w.sum()) if kind == "log2_lse"
                                     else math.log(w.sum())))
        return out, lse
    return attn


CHECKS = [check_closed_forms, check_library_sdpa, check_gqa_equals_repeated_mha,
          check_paged_equals_contiguous, check_single_token,
          check_equal_keys_mean, check_dominant_logit]
MUTANTS = ["no_scale", "gqa_modulo", "no_max_subtract", "unnormalised",
           "key_value_swap", "log2_lse", "paged_slot_swap", "off_by_one_len"]


def test_reference_copy_passes_every_check():
    attn = _mutant("none")
    for chk in CHECKS:
        chk(attn)


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_is_caught(kind):
    attn = _mutant(kind)
    failed = []
    for chk in CHECKS:
        try:
            with np.errstate(all="ignore"):
                chk(attn)
        except (AssertionError, IndexError, ValueError, FloatingPointError):
            failed.append(chk.__name__)
    assert failed, f"mutant {kind} passed every pin"


# ----------------------------------------------- 8-bit float (E4M3) caches

FP8_HAND = {
    # code: value, each derived by hand from the E4M3 layout
    # (sign | 4-bit exponent, bias 7 | 3-bit mantissa).
    0x00: 0.0,
    0x38: 1.0,                 # e = 7, m = 0
    0x3C: 1.5,                 # e = 7, m = 4
    0x40: 2.0,                 # e = 8
    0x7E: 448.0,               # e = 15, m = 6: largest finite
    0x08: 2.0 ** -6,           # smallest normal
    0x01: 2.0 ** -9,           # smallest subnormal: (1/8) * 2^-6
    0x07: 7 * 2.0 ** -9,       # largest subnormal
    0xB8: -1.0,
    0xC4: -3.0,                # e = 8, m = 4
}


def test_fp8_decode_hand_values():
    got = oracle.fp8_e4m3_to_f64(np.array(list(FP8_HAND), dtype=np.uint8))
    assert np.array_equal(got, np.array(list(FP8_HAND.values())))
    nan = oracle.fp8_e4m3_to_f64(np.array([0x7F, 0xFF], dtype=np.uint8))
    assert np.all(np.isnan(nan))
    neg0 = oracle.fp8_e4m3_to_f64(np.array([0x80], dtype=np.uint8))
    assert neg0[0] == 0.0 and math.copysign(1.0, neg0[0]) < 0


def check_fp8_codes(decode):
    """Every code against torch's float8_e4m3fn (the same OCP format)."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = decode(codes.numpy())
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def _fp8_case(seed, B=2, Hq=8, Hkv=2, D=16, L=29):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    k8 = (torch.randn(B, Hkv, L, D, generator=g) * 3).to(torch.float8_e4m3fn)
    v8 = (torch.randn(B, Hkv, L, D, generator=g) * 3).to(torch.float8_e4m3fn)
    ks = torch.rand(Hkv, generator=g) * 0.5 + 0.05
    vs = torch.rand(Hkv, generator=g) * 2.0 + 0.5
    lens = np.array([L, L // 2 + 1][:B])
    return q, k8, v8, ks, vs, lens


def check_fp8_sdpa(attn_q8, seed=30):
    """Attention over an E4M3 cache with per-kv-head scales against torch's
    float64 scaled_dot_product_attention on the cache torch dequantizes."""
    q, k8, v8, ks, vs, lens = _fp8_case(seed)
    B, Hq, D = q.shape
    Hkv = k8.shape[1]
    G = Hq // Hkv
    out, lse = attn_q8(q.view(torch.uint16).numpy(),
                       k8.view(torch.uint8).numpy(),
                       v8.view(torch.uint8).numpy(), lens,
                       ks.numpy(), vs.numpy())
    kd = k8.to(torch.float64) * ks.double()[None, :, None, None]
    vd = v8.to(torch.float64) * vs.double()[None, :, None, None]
    for b in range(B):
        n = int(lens[b])
        qt = q[b].double()[None, :, None, :]
        kt = kd[b, :, :n].repeat_interleave(G, dim=0)[None]
        vt = vd[b, :, :n].repeat_interleave(G, dim=0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)
        assert np.allclose(out[b], ref[0, :, 0].numpy(), rtol=0, atol=1e-12)
        s = (qt[0, :, 0, None, :] * kt[0]).sum(-1) / math.sqrt(D)
        assert np.allclose(lse[b], torch.logsumexp(s, -1).numpy(), atol=1e-12)


def check_fp8_equals_bf16_of_same_values(attn_q8, seed=31):
    """Power-of-two scales: every dequantized value is exact in bf16, so the
    quantized path must equal the (separately pinned) bf16 path on it."""
    q, k8, v8, _, _, lens = _fp8_case(seed)
    Hkv = k8.shape[1]
    ks = torch.tensor([0.25, 2.0])[:Hkv]
    vs = torch.tensor([4.0, 0.5])[:Hkv]
    out, lse = attn_q8(q.view(torch.uint16).numpy(),
                       k8.view(torch.uint8).numpy(),
                       v8.view(torch.uint8).numpy(), lens,
                       ks.numpy(), vs.numpy())
    kb = (k8.to(torch.float32) * ks[None, :, None, None]).to(torch.bfloat16)
    vb = (v8.to(torch.float32) * vs[None, :, None, None]).to(torch.bfloat16)
    assert torch.equal(kb.float(), k8.float() * ks[None, :, None, None])
    o2, l2 = oracle.decode_attention(q.view(torch.uint16).numpy(),
                                     kb.view(torch.uint16).numpy(),
                                     vb.view(torch.uint16).numpy(), lens,
                                     dtype="bf16")
    assert np.array_equal(out, o2) and np.array_equal(lse, l2)


def _attn_q8(q, k, v, lens, ks, vs):
    return oracle.decode_attention(q, k, v, lens, dtype="bf16",
                                   kv_dtype="fp8_e4m3", k_scale=ks,
                                   v_scale=vs)


def test_fp8_codes_match_torch():
    check_fp8_codes(oracle.fp8_e4m3_to_f64)


def test_fp8_attention_matches_torch_sdpa():
    check_fp8_sdpa(_attn_q8)


def test_fp8_attention_equals_bf16_on_exact_values():
    check_fp8_equals_bf16_of_same_values(_attn_q8)


def test_fp8_split_partials_recombine():
    q, k8, v8, ks, vs, lens = _fp8_case(32, L=100)
    args = (q.view(torch.uint16).numpy(), k8.view(torch.uint8).numpy(),
            v8.view(torch.uint8).numpy(), lens)
    ref = _attn_q8(*args, ks.numpy(), vs.numpy())
    op, lp = oracle.split_partials(*args, 7, dtype="bf16", max_seq_len=100,
                                   kv_dtype="fp8_e4m3", k_scale=ks.numpy(),
                                   v_scale=vs.numpy())
    out, lse = oracle.combine_partials(op, lp)
    assert np.allclose(out, ref[0], atol=1e-13)
    assert np.allclose(lse, ref[1], atol=1e-13)


def _fp8_decode_mutant(kind):
    def decode(codes):
        c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
        sign = np.where(c & 0x80, -1.0, 1.0)
        e = (c >> 3) & 0xF
        m = (c & 0x7).astype(np.float64)
        bias = 8 if kind == "bias8" else 7
        if kind == "subnormal_as_normal":
            mag = (1.0 + m / 8.0) * np.exp2((e - bias).astype(np.float64))
        else:
            mag = np.where(e == 0, (m / 8.0) * 2.0 ** (1 - bias),
                           (1.0 + m / 8.0) * np.exp2((e - bias).astype(np.float64)))
        if kind != "no_nan":
            mag = np.where((e == 15) & (c & 7 == 7), np.nan, mag)
        return sign * mag
    return decode


FP8_MUTANTS = ["bias8", "subnormal_as_normal", "no_nan", "scale_swap",
               "no_v_scale", "k_scale_on_both"]


@pytest.mark.parametrize("kind", FP8_MUTANTS)
def test_fp8_planted_mistake_is_caught(kind, monkeypatch):
    decode = oracle.fp8_e4m3_to_f64
    if kind in ("bias8", "subnormal_as_normal", "no_nan"):
        decode = _fp8_decode_mutant(kind)
        monkeypatch.setattr(oa, "fp8_e4m3_to_f64", decode)

    def attn(q, k, v, lens, ks, vs):
        if kind == "scale_swap":
            ks, vs = vs, ks
        elif kind == "no_v_scale":
            vs = None
        elif kind == "k_scale_on_both":
            vs = ks
        return _attn_q8(q, k, v, lens, ks, vs)

    failed = []
    for chk, arg in ((check_fp8_codes, decode), (check_fp8_sdpa, attn),
                     (check_fp8_equals_bf16_of_same_values, attn)):
        try:
            with np.errstate(all="ignore"):
                chk(arg)
        except AssertionError:
            failed.append(chk.__name__)
    assert failed, f"mutant {kind} passed every fp8 pin"


# --- 8-bit integer cache, one scale per (position, kv head) ---------------

INT8_HAND = {
    # byte: value, from two's complement by hand (b >= 128 means b - 256)
    0x00: 0.0, 0x01: 1.0, 0x7F: 127.0, 0x80: -128.0, 0x81: -127.0,
    0xFE: -2.0, 0xFF: -1.0, 0x40: 64.0, 0xC0: -64.0,
}


def test_int8_decode_hand_values():
    got = oracle.int8_to_f64(np.array(list(INT8_HAND), dtype=np.uint8))
    assert np.array_equal(got, np.array(list(INT8_HAND.values())))
    signed = np.array([-128, -1, 0, 1, 127], dtype=np.int8)
    assert np.array_equal(oracle.int8_to_f64(signed),
                          np.array([-128.0, -1.0, 0.0, 1.0, 127.0]))


def _int8_case(seed, B=2, Hq=8, Hkv=2, D=16, L=29):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    k8 = torch.randint(-128, 128, (B, Hkv, L, D), generator=g,
                       dtype=torch.int8)
    v8 = torch.randint(-128, 128, (B, Hkv, L, D), generator=g,
                       dtype=torch.int8)
    ks = torch.rand(B, Hkv, L, generator=g) * 0.04 + 0.002
    vs = torch.rand(B, Hkv, L, generator=g) * 0.1 + 0.01
    lens = np.array([L, L // 2 + 1][:B])
    return q, k8, v8, ks, vs, lens


def _attn_i8(q, k, v, lens, ks, vs, block_table=None, block_size=0):
    return oracle.decode_attention(q, k, v, lens, dtype="bf16",
                                   kv_dtype="int8", k_scale=ks, v_scale=vs,
                                   block_table=block_table,
                                   block_size=block_size)


def _i8_args(q, k8, v8, lens):
    return (q.view(torch.uint16).numpy(), k8.numpy(), v8.numpy(), lens)


def check_int8_sdpa(attn_i8, seed=40):
    """Attention over an int8 cache with per-position scales against torch's
    float64 scaled_dot_product_attention on the cache torch dequantizes."""
    q, k8, v8, ks, vs, lens = _int8_case(seed)
    B, Hq, D = q.shape
    G = Hq // k8.shape[1]
    out, lse = attn_i8(*_i8_args(q, k8, v8, lens), ks.numpy(), vs.numpy())
    kd = k8.to(torch.float64) * ks.double()[..., None]
    vd = v8.to(torch.float64) * vs.double()[..., None]
    for b in range(B):
        n = int(lens[b])
        qt = q[b].double()[None, :, None, :]
        kt = kd[b, :, :n].repeat_interleave(G, dim=0)[None]
        vt = vd[b, :, :n].repeat_interleave(G, dim=0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)
        assert np.allclose(out[b], ref[0, :, 0].numpy(), rtol=0, atol=1e-12)
        s = (qt[0, :, 0, None, :] * kt[0]).sum(-1) / math.sqrt(D)
        assert np.allclose(lse[b], torch.logsumexp(s, -1).numpy(), atol=1e-12)


def check_int8_equals_bf16_of_same_values(attn_i8, seed=41):
    """Power-of-two scales per position: every dequantized value is exact in
    bf16 (an int8 has at most 8 significant bits), so the int8 path must
    equal the (separately pinned) bf16 path on those values, bit for bit."""
    q, k8, v8, _, _, lens = _int8_case(seed)
    g = torch.Generator().manual_seed(seed + 100)
    ks = torch.exp2(torch.randint(-9, -3, k8.shape[:3], generator=g).float())
    vs = torch.exp2(torch.randint(-8, 0, v8.shape[:3], generator=g).float())
    out, lse = attn_i8(*_i8_args(q, k8, v8, lens), ks.numpy(), vs.numpy())
    kb = (k8.float() * ks[..., None]).to(torch.bfloat16)
    vb = (v8.float() * vs[..., None]).to(torch.bfloat16)
    assert torch.equal(kb.float(), k8.float() * ks[..., None])
    assert torch.equal(vb.float(), v8.float() * vs[..., None])
    o2, l2 = oracle.decode_attention(q.view(torch.uint16).numpy(),
                                     kb.view(torch.uint16).numpy(),
                                     vb.view(torch.uint16).numpy(), lens,
                                     dtype="bf16")
    assert np.array_equal(out, o2) and np.array_equal(lse, l2)


def check_int8_paged_equals_contiguous(attn_i8, seed=42, bs=16):
    """The same codes and scales moved, with no arithmetic, into a pool of
    bs-slot blocks in shuffled order: the result must not change."""
    q, k8, v8, ks, vs, lens = _int8_case(seed, L=61)
    B, Hkv, L, D = k8.shape
    nblk = -(-L // bs)
    perm = torch.randperm(B * nblk, generator=torch.Generator().manual_seed(7))
    NB = B * nblk + 1
    kp = torch.full((NB, Hkv, bs, D), 99, dtype=torch.int8)
    vp = torch.full((NB, Hkv, bs, D), -99, dtype=torch.int8)
    ksp = torch.full((NB, Hkv, bs), 1e30)
    vsp = torch.full((NB, Hkv, bs), float("nan"))
    bt = np.zeros((B, nblk), dtype=np.int64)
    for b in range(B):
        for j in range(nblk):
            blk = int(perm[b * nblk + j])
            bt[b, j] = blk
            t0, t1 = j * bs, min((j + 1) * bs, L)
            kp[blk, :, :t1 - t0] = k8[b, :, t0:t1]
            vp[blk, :, :t1 - t0] = v8[b, :, t0:t1]
            ksp[blk, :, :t1 - t0] = ks[b, :, t0:t1]
            vsp[blk, :, :t1 - t0] = vs[b, :, t0:t1]
    ref = attn_i8(*_i8_args(q, k8, v8, lens), ks.numpy(), vs.numpy())
    got = attn_i8(*_i8_args(q, kp, vp, lens), ksp.numpy(), vsp.numpy(),
                  block_table=bt, block_size=bs)
    assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])


def test_int8_attention_matches_torch_sdpa():
    check_int8_sdpa(_attn_i8)


def test_int8_attention_equals_bf16_on_exact_values():
    check_int8_equals_bf16_of_same_values(_attn_i8)


def test_int8_paged_equals_contiguous():
    check_int8_paged_equals_contiguous(_attn_i8)


def test_int8_per_head_scales_broadcast():
    """A per-position scale array that is constant along positions gives
    the same result as the one-value-per-kv-head form."""
    q, k8, v8, _, _, lens = _int8_case(43)
    B, Hkv, L, _ = k8.shape
    kh = np.array([0.01, 0.03])[:Hkv]
    vh = np.array([0.2, 0.05])[:Hkv]
    a = _attn_i8(*_i8_args(q, k8, v8, lens), kh, vh)
    b = _attn_i8(*_i8_args(q, k8, v8, lens),
                 np.broadcast_to(kh[None, :, None], (B, Hkv, L)).copy(),
                 np.broadcast_to(vh[None, :, None], (B, Hkv, L)).copy())
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_int8_split_partials_recombine():
    q, k8, v8, ks, vs, lens = _int8_case(44, L=100)
    args = _i8_args(q, k8, v8, lens)
    ref = _attn_i8(*args, ks.numpy(), vs.numpy())
    op, lp = oracle.split_partials(*args, 7, dtype="bf16", max_seq_len=100,
                                   kv_dtype="int8", k_scale=ks.numpy(),
                                   v_scale=vs.numpy())
    out, lse = oracle.combine_partials(op, lp)
    assert np.allclose(out, ref[0], atol=1e-13)
    assert np.allclose(lse, ref[1], atol=1e-13)


INT8_MUTANTS = ["unsigned", "sign_magnitude", "scale_shift", "scale_swap",
                "scale_first_position", "scale_ignores_table"]


@pytest.mark.parametrize("kind", INT8_MUTANTS)
def test_int8_planted_mistake_is_caught(kind, monkeypatch):
    real_rows = oa.scale_rows
    if kind == "unsigned":
        monkeypatch.setattr(oa, "int8_to_f64", lambda c: np.asarray(
            c).view(np.uint8).astype(np.float64))
    elif kind == "sign_magnitude":
        def sm(c):
            u = np.asarray(c).view(np.uint8).astype(np.int64)
            return np.where(u & 0x80, -(u & 0x7F), u).astype(np.float64)
        monkeypatch.setattr(oa, "int8_to_f64", sm)
    elif kind == "scale_shift":
        def shifted(scale, b, kvh, lo, hi, block_table=None, block_size=0):
            sc = np.asarray(scale, dtype=np.float64)
            if sc.ndim == 1:
                return real_rows(scale, b, kvh, lo, hi, block_table,
                                 block_size)
            rolled = np.roll(sc, 1, axis=-1)
            return real_rows(rolled, b, kvh, lo, hi, block_table, block_size)
        monkeypatch.setattr(oa, "scale_rows", shifted)
    elif kind == "scale_first_position":
        def first(scale, b, kvh, lo, hi, block_table=None, block_size=0):
            r = real_rows(scale, b, kvh, lo, hi, block_table, block_size)
            return np.full_like(r, r[0, 0])
        monkeypatch.setattr(oa, "scale_rows", first)
    elif kind == "scale_ignores_table":
        def flat(scale, b, kvh, lo, hi, block_table=None, block_size=0):
            sc = np.asarray(scale, dtype=np.float64)
            if sc.ndim == 3 and block_table is not None:
                rows = sc.reshape(-1, sc.shape[1], 1)
                return rows[lo:hi, kvh] if hi <= rows.shape[0] else \
                    real_rows(scale, b, kvh, lo, hi, None, 0)
            return real_rows(scale, b, kvh, lo, hi, block_table, block_size)
        monkeypatch.setattr(oa, "scale_rows", flat)

    def attn(q, k, v, lens, ks, vs, block_table=None, block_size=0):
        if kind == "scale_swap":
            ks, vs = vs, ks
        return _attn_i8(q, k, v, lens, ks, vs, block_table, block_size)

    failed = []
    for chk in (check_int8_sdpa, check_int8_equals_bf16_of_same_values,
                check_int8_paged_equals_contiguous):
        try:
            with np.errstate(all="ignore"):
                chk(attn)
        except (AssertionError, IndexError, ValueError):
            failed.append(chk.__name__)
    if kind in ("unsigned", "sign_magnitude"):
        try:
            test_int8_decode_hand_values()
        except AssertionError:
            failed.append("hand_values")
    assert failed, f"mutant {kind} passed every int8 pin"
