"""The convenience wrapper's input checks (CPU: no kernel runs).

``split_kv_long_amd.decode_attention`` hands raw pointers to the library,
which reads them with the dtypes, strides and padding the C ABI documents
(``include/fd_decode.h``). These tests pin that the wrapper refuses inputs
the kernels would misread instead of computing garbage."""

import pytest
import torch

import split_kv_long_amd as fd

B, HQ, HKV, D, L = 2, 8, 2, 64, 40     # L % 16 != 0: int8 rows need padding


def tensors(cache=torch.bfloat16, paged=False):
    q = torch.zeros(B, HQ, D, dtype=torch.bfloat16 if cache != torch.float32
                    else torch.float32)
    if paged:
        k = torch.zeros(7, HKV, 16, D).to(cache)
        bt = torch.zeros(B, 3, dtype=torch.int32)
    else:
        k = torch.zeros(B, HKV, L, D).to(cache)
        bt = None
    v = k.clone()
    lens = torch.full((B,), L, dtype=torch.int32)
    return q, k, v, lens, bt


def check(**kw):
    q, k, v, lens, bt = tensors(kw.pop("cache", torch.bfloat16),
                                kw.pop("paged", False))
    args = dict(q=q, k_cache=k, v_cache=v, seq_lens=lens, block_table=bt)
    args.update(kw)
    return fd.validate_inputs(args.pop("q"), args.pop("k_cache"),
                              args.pop("v_cache"), args.pop("seq_lens"),
                              device="cpu", **args)


def test_valid_inputs_pass():
    s = check()
    assert (s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim,
            s.max_seq_len, s.block_size) == (B, HQ, HKV, D, L, 0)
    s = check(paged=True, max_seq_len=37)     # a paged bound may be smaller
    assert s.max_seq_len == 37 and s.block_size == 16


def test_contiguous_bound_must_equal_the_cache_length():
    # L is also the row stride of [B, Hkv, L, D]: a different bound would
    # read rows of the wrong sequence or past the cache.
    with pytest.raises(ValueError, match="row stride"):
        check(max_seq_len=L - 8)
    with pytest.raises(ValueError, match="row stride"):
        check(max_seq_len=L + 16)
    assert check(max_seq_len=L).max_seq_len == L


def test_lengths_and_block_table_dtypes():
    q, k, v, lens, bt = tensors()
    with pytest.raises(ValueError, match="int32"):
        fd.validate_inputs(q, k, v, lens.to(torch.int64), device="cpu")
    with pytest.raises(ValueError, match="int32"):
        fd.validate_inputs(q, k, v, lens[:1], device="cpu")
    q, k, v, lens, bt = tensors(paged=True)
    with pytest.raises(ValueError, match="block_table"):
        fd.validate_inputs(q, k, v, lens, bt.to(torch.int64), device="cpu")
    with pytest.raises(ValueError, match="contiguous"):
        fd.validate_inputs(q, k, v, lens, bt.t().contiguous().t(),
                           device="cpu")


def test_layout_and_device():
    q, k, v, lens, bt = tensors()
    with pytest.raises(ValueError, match="contiguous"):
        fd.validate_inputs(q.transpose(0, 1).contiguous().transpose(0, 1), k,
                           v, lens, device="cpu")
    with pytest.raises(ValueError, match="head_dim"):
        fd.validate_inputs(torch.zeros(B, HQ, 128, dtype=torch.bfloat16), k,
                           v, lens, device="cpu")
    with pytest.raises(ValueError, match="match"):
        fd.validate_inputs(q, k, v[:, :, :8].contiguous(), lens,
                           device="cpu")
    with pytest.raises(ValueError, match="device"):
        fd.validate_inputs(q, k, v, lens, device="meta")


def test_int8_scales_need_padded_rows():
    lp = -(-L // 16) * 16
    ok = torch.ones(B, HKV, lp)
    check(cache=torch.int8, k_scale=ok, v_scale=ok)
    bad = torch.ones(B, HKV, L)              # unpadded: rows misread
    with pytest.raises(ValueError, match="k_scale"):
        check(cache=torch.int8, k_scale=bad, v_scale=ok)
    with pytest.raises(ValueError, match="v_scale"):
        check(cache=torch.int8, k_scale=ok, v_scale=bad)
    with pytest.raises(ValueError, match="fp32"):
        check(cache=torch.int8, k_scale=ok.double(), v_scale=ok)
    with pytest.raises(ValueError, match="needs"):
        check(cache=torch.int8, k_scale=ok)
    paged = torch.ones(7, HKV, 16)
    check(cache=torch.int8, paged=True, k_scale=paged, v_scale=paged)
    with pytest.raises(ValueError, match="k_scale"):
        check(cache=torch.int8, paged=True, k_scale=ok, v_scale=paged)


def test_e4m3_scales_per_kv_head_and_no_scales_otherwise():
    s = torch.ones(HKV)
    check(cache=torch.float8_e4m3fn, k_scale=s, v_scale=s)
    with pytest.raises(ValueError, match="k_scale"):
        check(cache=torch.float8_e4m3fn, k_scale=torch.ones(HKV + 1),
              v_scale=s)
    with pytest.raises(ValueError, match="only taken"):
        check(k_scale=s, v_scale=s)


def test_sparse_split_count_fits_the_sparse_limits():
    from split_kv_long_amd import binding as fb
    for L, G, bs, S in [(65536, 8, 0, 128), (65536, 32, 0, 1),
                        (1 << 20, 128, 0, 4), (100, 4, 16, 1),
                        (8193, 16, 0, 1), (40000, 20, 64, 3)]:
        nb = -(-L // bs) if bs else 0
        sh = fb.make_shape(1, 2 * G, 2, 128, L, "bf16", bs, nb, nb, 0.0)
        got = fd.sparse_splits(sh, S)
        g = max(16, bs)
        P = -(-(-(-L // got)) // g) * g
        assert got >= S
        assert P <= 8192 and P * max(16, G) <= 8192 * 16, (L, G, got, P)
        if got > S:      # the doubling stopped at the first fit
            half = got // 2
            Ph = -(-(-(-L // half)) // g) * g
            assert Ph > 8192 or Ph * max(16, G) > 8192 * 16


def test_sparse_wrappers_refuse_fp32_caches():
    q, k, v, lens, bt = tensors(cache=torch.float32)
    with pytest.raises(ValueError, match="bf16, E4M3 or int8"):
        fd.build_key_summary(q, k, lens)
    with pytest.raises(ValueError, match="bf16, E4M3 or int8"):
        fd.sparse_decode_attention(q, k, v, lens, (None, None), 1.0)


def test_sparse_call_checks_the_summary_layout():
    # The kernel reads the summary by the shape's layout: a summary of
    # another shape, dtype or device is refused before any call.
    q, k, v, lens, bt = tensors()
    nrec = (B, HKV, -(-L // 16))
    good_c = torch.zeros(nrec + (8 * D,), dtype=torch.uint8)
    good_s = torch.zeros(nrec)

    def call(c, s):
        fd.sparse_decode_attention(q, k, v, lens, (c, s), 1.0, num_splits=1)

    with pytest.raises(ValueError, match="summary codes"):
        call(good_c[:, :, :-1], good_s)
    with pytest.raises(ValueError, match="summary codes"):
        call(good_c.to(torch.int8), good_s)
    with pytest.raises(ValueError, match="summary scales"):
        call(good_c, good_s.double())
    with pytest.raises(ValueError, match="summary scales"):
        call(good_c, torch.zeros(B, HKV, 16 * nrec[2]))
