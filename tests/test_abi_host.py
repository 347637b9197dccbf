"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before launching."""

import ctypes
import os
import re

import pytest

from split_kv_long_amd import binding as fb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h)
           for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

pytestmark = pytest.mark.skipif(not os.path.exists(fb.LIB_PATH),
                                reason="library not built")


def header_functions():
    """Every fd_* function the headers under include/ declare."""
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(fd_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    lib = fb.load()
    names = header_functions()
    assert set(names) == set(fb.SYMBOLS)
    for name in names:
        assert hasattr(lib, name), name


def test_shape_struct_matches_header():
    text = open(os.path.join(ROOT, "include", "fd_decode.h")).read()
    body = re.search(r"typedef struct fd_shape \{(.*?)\} fd_shape;", text, re.S)
    fields = re.findall(r"(int32_t|float)\s+(\w+);", body.group(1))
    assert [f for _, f in fields] == [f for f, _ in fb.FdShape._fields_]
    assert ctypes.sizeof(fb.FdShape) == 40


def test_status_strings_and_version():
    assert fb.fd_status_str(0) == "ok"
    for st in (-1, -2, -3, -4):
        assert fb.fd_status_str(st) and fb.fd_status_str(st) != "ok"
    assert fb.fd_status_str(7) == "unknown status"
    assert fb.fd_version() >= 10100


def shp(**kw):
    d = dict(batch=1, num_q_heads=16, num_kv_heads=2, head_dim=128,
             max_seq_len=65536, dtype="bf16")
    d.update(kw)
    return fb.make_shape(**d)


def plan(cus=256, sum_len=-1, **kw):
    return fb.fd_plan_splits(shp(**kw), cus, sum_len)


def test_planner_regimes():
    # batch-one long history: spread over the CUs, 512-token splits
    assert plan() == 128
    # uniform long history: one workgroup per CU, 8192-token splits
    assert plan(num_q_heads=64, num_kv_heads=8, max_seq_len=262144) == 32
    assert plan(max_seq_len=262144) == 128
    assert plan(max_seq_len=131072) == 128
    # a batch that already fills the GPU: no split
    assert plan(batch=64, num_q_heads=32, num_kv_heads=8, max_seq_len=1024) == 1
    # half the CUs busy and a short history: no split either ...
    assert plan(batch=64, max_seq_len=512) == 1
    # ... but a longer one still gains from splitting
    assert plan(batch=64, max_seq_len=2048) == 2
    # a short history: no split below two minimum-length (128-token) splits
    assert plan(max_seq_len=200) == 1
    # ... but a batch-one 512-token history already gains from 4 splits
    assert plan(max_seq_len=512) == 4
    # a ragged batch (known total below batch x bound): splits longer than
    # 1024 tokens are halved, about two workgroups per CU for the
    # length-aware pieces; the same batch taken as uniform is not
    ragged = dict(batch=16, num_q_heads=32, num_kv_heads=8, max_seq_len=32768)
    assert plan(sum_len=245263, **ragged) == 9
    assert plan(sum_len=16 * 32768, **ragged) == 2
    assert plan(**ragged) == 2
    # tiny fp32 MHA history of 512 tokens: the fp32 path is latency-bound,
    # so it takes the shorter fp32 minimum split (64 tokens) -> 8 splits
    assert plan(num_q_heads=8, num_kv_heads=8, head_dim=64, max_seq_len=512,
                dtype="f32") == 8
    assert plan(num_q_heads=8, num_kv_heads=8, head_dim=64, max_seq_len=100,
                dtype="f32") == 1


def test_planner_regimes_8bit():
    # batch one: as for bf16
    for dt in ("fp8_e4m3", "int8"):
        assert plan(dtype=dt) == 128
        assert plan(max_seq_len=512, dtype=dt) == 4
    # a short history with 8 or more units runs unsplit (half the bytes per
    # position: the split stops paying earlier than for bf16) ...
    for dt in ("fp8_e4m3", "int8"):
        assert plan(batch=4, max_seq_len=512, dtype=dt) == 1
        assert plan(batch=16, max_seq_len=512, dtype=dt) == 1
    assert plan(batch=4, max_seq_len=512) == 4              # bf16 splits
    # ... and from 1024 positions on it splits again
    assert plan(batch=4, max_seq_len=2048, dtype="fp8_e4m3") == 16
    # int8 batches of 2..64 halve their splits at any length (4-wave
    # pieces, about two per CU); E4M3 keeps the bf16 sizing
    assert plan(batch=16, max_seq_len=262144, dtype="int8") == 16
    assert plan(batch=16, max_seq_len=262144, dtype="fp8_e4m3") == 8
    assert plan(batch=64, max_seq_len=32768, dtype="int8") == 4
    assert plan(batch=64, max_seq_len=32768, dtype="fp8_e4m3") == 2
    assert plan(batch=4, max_seq_len=131072, dtype="int8") == 64
    # above 64 sequences the uniform splits (8 waves) keep the bf16 sizing
    assert plan(batch=65, max_seq_len=32768, dtype="int8") == \
        plan(batch=65, max_seq_len=32768, dtype="fp8_e4m3")
    # a ragged int8 batch is halved once, like any ragged batch
    ragged = dict(batch=16, num_q_heads=32, num_kv_heads=8, max_seq_len=32768)
    assert plan(sum_len=245263, dtype="int8", **ragged) == 9


def test_planner_properties():
    for L in (512, 1000, 4096, 65536, 262144, 1 << 20):
        for B in (1, 2, 4, 16):
            S = plan(batch=B, max_seq_len=L)
            assert S >= 1
            P = -(-(-(-L // S)) // 16) * 16
            assert S * P >= L
            if S > 1:
                assert P >= 128 and B * 2 * S >= 1
            assert S == plan(batch=B, max_seq_len=L)   # deterministic
    # splits never grow as the batch grows at fixed L
    prev = 10 ** 9
    for B in (1, 2, 4, 8, 16, 32, 64, 128):
        S = plan(batch=B, max_seq_len=32768)
        assert S <= prev
        prev = S
    # a known, smaller total work gives shorter splits, so at least as many
    full = plan(batch=16, num_q_heads=32, num_kv_heads=8, max_seq_len=32768)
    part = plan(batch=16, num_q_heads=32, num_kv_heads=8, max_seq_len=32768,
                sum_len=266240)
    assert part >= full


def test_workspace_size():
    s = shp()
    assert fb.fd_workspace_size(s, 1) == 0
    n = fb.fd_workspace_size(s, 128)
    assert n >= 16 * 128 * 129 * 4 and n % 256 == 0


@pytest.mark.parametrize("kw,status", [
    (dict(num_q_heads=10, num_kv_heads=4), fb.FD_ERR_INVALID_ARG),
    (dict(batch=0), fb.FD_ERR_INVALID_ARG),
    (dict(num_kv_heads=0), fb.FD_ERR_INVALID_ARG),
    (dict(head_dim=96), fb.FD_ERR_UNSUPPORTED),
    (dict(head_dim=100), fb.FD_ERR_INVALID_ARG),
    (dict(dtype=7), fb.FD_ERR_UNSUPPORTED),
    (dict(max_seq_len=-1), fb.FD_ERR_INVALID_ARG),
    (dict(block_size=8, max_blocks_per_seq=8192, num_blocks=10),
     fb.FD_ERR_INVALID_ARG),
    (dict(block_size=16, max_blocks_per_seq=10, num_blocks=10),
     fb.FD_ERR_INVALID_ARG),
    (dict(block_size=16, max_blocks_per_seq=4096, num_blocks=0),
     fb.FD_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fb.FD_ERR_INVALID_ARG),
])
def test_bad_shapes_are_rejected(kw, status):
    s = shp(**kw)
    lib = fb.load()
    out = ctypes.c_int(-99)
    assert lib.fd_plan_splits(ctypes.byref(s), 256, -1, ctypes.byref(out)) == status
    assert out.value == -99
    size = ctypes.c_size_t(12345)
    assert lib.fd_workspace_size(ctypes.byref(s), 4, ctypes.byref(size)) == status
    assert size.value == 12345
    # a decode call with the bad shape is rejected before any pointer is used
    assert lib.fd_decode_attn(ctypes.byref(s), 16, 16, 16, None, 16, 1, None,
                              0, 16, None, None) == status


FAKE = 1 << 20   # aligned, never dereferenced: every call below is rejected


def call(**kw):
    lib = fb.load()
    args = dict(shape=shp(), q=FAKE, k=FAKE, v=FAKE, bt=None, lens=FAKE,
                S=4, ws=FAKE, ws_bytes=1 << 30, out=FAKE, lse=None)
    args.update(kw)
    return lib.fd_decode_attn(ctypes.byref(args["shape"]), args["q"],
                              args["k"], args["v"], args["bt"], args["lens"],
                              args["S"], args["ws"], args["ws_bytes"],
                              args["out"], args["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fb.FD_ERR_INVALID_ARG),
    (dict(k=None), fb.FD_ERR_INVALID_ARG),
    (dict(lens=None), fb.FD_ERR_INVALID_ARG),
    (dict(out=None), fb.FD_ERR_INVALID_ARG),
    (dict(q=FAKE + 8), fb.FD_ERR_INVALID_ARG),
    (dict(v=FAKE + 2), fb.FD_ERR_INVALID_ARG),
    (dict(out=FAKE + 4), fb.FD_ERR_INVALID_ARG),
    (dict(lse=FAKE + 2), fb.FD_ERR_INVALID_ARG),
    (dict(S=0), fb.FD_ERR_INVALID_ARG),
    (dict(S=70000), fb.FD_ERR_INVALID_ARG),
    (dict(ws=None), fb.FD_ERR_WORKSPACE),
    (dict(ws_bytes=100), fb.FD_ERR_WORKSPACE),
    (dict(ws=FAKE + 8), fb.FD_ERR_INVALID_ARG),
    (dict(bt=FAKE), fb.FD_ERR_INVALID_ARG),      # table given, contiguous shape
    (dict(shape=shp(block_size=16, max_blocks_per_seq=4096, num_blocks=64)),
     fb.FD_ERR_INVALID_ARG),                      # paged shape, no table
])
def test_bad_calls_are_rejected_on_the_host(kw, status):
    assert call(**kw) == status


def test_partials_and_combine_reject_bad_args():
    lib = fb.load()
    s = shp()
    assert lib.fd_decode_partials(ctypes.byref(s), FAKE, FAKE, FAKE, None,
                                  FAKE, 4, None, FAKE, None) == fb.FD_ERR_INVALID_ARG
    assert lib.fd_decode_partials(ctypes.byref(s), FAKE, FAKE, FAKE, None,
                                  FAKE, 0, FAKE, FAKE, None) == fb.FD_ERR_INVALID_ARG
    assert lib.fd_combine_partials(1, 16, 96, 4, FAKE, FAKE, FAKE, None,
                                   None) == fb.FD_ERR_UNSUPPORTED
    assert lib.fd_combine_partials(0, 16, 128, 4, FAKE, FAKE, FAKE, None,
                                   None) == fb.FD_ERR_INVALID_ARG
    assert lib.fd_combine_partials(1, 16, 128, 4, FAKE + 4, FAKE, FAKE, None,
                                   None) == fb.FD_ERR_INVALID_ARG


def call_fp8(**kw):
    lib = fb.load()
    args = dict(shape=shp(dtype="fp8_e4m3"), q=FAKE, k=FAKE, v=FAKE,
                ks=FAKE, vs=FAKE, bt=None, lens=FAKE, S=4, ws=FAKE,
                ws_bytes=1 << 30, out=FAKE, lse=None)
    args.update(kw)
    return lib.fd_decode_attn_fp8(ctypes.byref(args["shape"]), args["q"],
                                  args["k"], args["v"], args["ks"], args["vs"],
                                  args["bt"], args["lens"], args["S"],
                                  args["ws"], args["ws_bytes"], args["out"],
                                  args["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(ks=None), fb.FD_ERR_INVALID_ARG),
    (dict(vs=None), fb.FD_ERR_INVALID_ARG),
    (dict(ks=FAKE + 2), fb.FD_ERR_INVALID_ARG),
    (dict(shape=shp()), fb.FD_ERR_INVALID_ARG),           # bf16 shape
    (dict(shape=shp(dtype="f32")), fb.FD_ERR_INVALID_ARG),
    (dict(k=FAKE + 8), fb.FD_ERR_INVALID_ARG),
    (dict(ws_bytes=100), fb.FD_ERR_WORKSPACE),
    (dict(shape=shp(dtype="fp8_e4m3", head_dim=96)), fb.FD_ERR_UNSUPPORTED),
])
def test_fp8_calls_are_rejected_on_the_host(kw, status):
    assert call_fp8(**kw) == status


def test_fp8_shape_needs_the_fp8_entry_points():
    lib = fb.load()
    s = shp(dtype="fp8_e4m3")
    # the plain entry points have no scales: an E4M3 shape is refused there
    assert call(shape=s) == fb.FD_ERR_INVALID_ARG
    assert lib.fd_decode_partials(ctypes.byref(s), FAKE, FAKE, FAKE, None,
                                  FAKE, 4, FAKE, FAKE, None) == fb.FD_ERR_INVALID_ARG
    assert lib.fd_decode_partials_fp8(ctypes.byref(shp()), FAKE, FAKE, FAKE,
                                      FAKE, FAKE, None, FAKE, 4, FAKE, FAKE,
                                      None) == fb.FD_ERR_INVALID_ARG
    assert lib.fd_decode_partials_fp8(ctypes.byref(s), FAKE, FAKE, FAKE,
                                      None, FAKE, None, FAKE, 4, FAKE, FAKE,
                                      None) == fb.FD_ERR_INVALID_ARG
    # planning and workspace sizing accept it
    assert fb.fd_plan_splits(s, 256, -1) >= 1
    assert fb.fd_workspace_size(s, 8) == fb.fd_workspace_size(shp(), 8)


def test_sparse_and_summary_reject_bad_args():
    lib = fb.load()
    s = shp(max_seq_len=8192)
    F = ctypes.c_float

    def sparse(**kw):
        args = dict(shape=s, q=FAKE, k=FAKE, v=FAKE, codes=FAKE, scales=FAKE,
                    bt=None, lens=FAKE, delta=4.0, S=4, ws=FAKE,
                    ws_bytes=1 << 30, out=FAKE, lse=None, kept=None)
        args.update(kw)
        return lib.fd_decode_attn_sparse(
            ctypes.byref(args["shape"]), args["q"], args["k"], args["v"],
            args["codes"], args["scales"], args["bt"], args["lens"],
            F(args["delta"]), args["S"], args["ws"], args["ws_bytes"],
            args["out"], args["lse"], args["kept"], None)

    assert sparse(codes=None) == fb.FD_ERR_INVALID_ARG
    assert sparse(codes=FAKE + 8) == fb.FD_ERR_INVALID_ARG
    assert sparse(scales=None) == fb.FD_ERR_INVALID_ARG
    assert sparse(delta=-1.0) == fb.FD_ERR_INVALID_ARG
    assert sparse(delta=float("nan")) == fb.FD_ERR_INVALID_ARG
    assert sparse(ws_bytes=10) == fb.FD_ERR_WORKSPACE
    # more than 8192 tokens per split, more than 128 query heads per kv
    # head, more than 131072 (tokens per split x heads per kv head), fp32 or
    # E4M3 caches: not supported on this path
    assert sparse(shape=shp(max_seq_len=16384), S=1) == fb.FD_ERR_UNSUPPORTED
    assert sparse(shape=shp(max_seq_len=8192, num_q_heads=258, num_kv_heads=2),
                  S=64) == fb.FD_ERR_UNSUPPORTED
    assert sparse(shape=shp(max_seq_len=8192, num_q_heads=64, num_kv_heads=2),
                  S=1) == fb.FD_ERR_UNSUPPORTED               # 8192 x 32
    assert sparse(shape=shp(max_seq_len=8192, num_q_heads=256, num_kv_heads=2),
                  S=4) == fb.FD_ERR_UNSUPPORTED               # 2048 x 128
    assert sparse(shape=shp(max_seq_len=8192, dtype="f32")) == fb.FD_ERR_UNSUPPORTED
    assert sparse(shape=shp(max_seq_len=8192, dtype="fp8_e4m3")
                  ) == fb.FD_ERR_UNSUPPORTED

    # The E4M3 calls: an E4M3 shape with both scales, nothing else.
    s8 = shp(max_seq_len=8192, dtype="fp8_e4m3")

    def sparse8(**kw):
        args = dict(shape=s8, q=FAKE, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE,
                    codes=FAKE, scales=FAKE, bt=None, lens=FAKE, delta=4.0,
                    S=4, ws=FAKE, ws_bytes=1 << 30, out=FAKE, lse=None,
                    kept=None)
        args.update(kw)
        return lib.fd_decode_attn_sparse_fp8(
            ctypes.byref(args["shape"]), args["q"], args["k"], args["v"],
            args["ks"], args["vs"], args["codes"], args["scales"], args["bt"],
            args["lens"], F(args["delta"]), args["S"], args["ws"],
            args["ws_bytes"], args["out"], args["lse"], args["kept"], None)

    def summary8(**kw):
        args = dict(shape=s8, k=FAKE, ks=FAKE, bt=None, lens=FAKE,
                    codes=FAKE, scales=FAKE)
        args.update(kw)
        return lib.fd_build_key_summary_fp8(
            ctypes.byref(args["shape"]), args["k"], args["ks"], args["bt"],
            args["lens"], args["codes"], args["scales"], None)

    assert sparse8(ks=None) == fb.FD_ERR_INVALID_ARG
    assert sparse8(vs=None) == fb.FD_ERR_INVALID_ARG
    assert sparse8(ks=FAKE + 2) == fb.FD_ERR_INVALID_ARG
    assert sparse8(shape=s) == fb.FD_ERR_INVALID_ARG          # bf16 shape
    assert sparse8(shape=shp(max_seq_len=8192, dtype="int8")
                   ) == fb.FD_ERR_INVALID_ARG
    assert sparse8(codes=None) == fb.FD_ERR_INVALID_ARG
    assert sparse8(delta=float("nan")) == fb.FD_ERR_INVALID_ARG
    assert sparse8(ws_bytes=10) == fb.FD_ERR_WORKSPACE
    assert sparse8(shape=shp(max_seq_len=16384, dtype="fp8_e4m3"), S=1
                   ) == fb.FD_ERR_UNSUPPORTED
    # int8: per-position scales, 16-byte aligned for the sparse call
    si = shp(max_seq_len=8192, dtype="int8")

    def sparse_i8(**kw):
        args = dict(shape=si, ks=FAKE, vs=FAKE)
        args.update(kw)
        return lib.fd_decode_attn_sparse_int8(
            ctypes.byref(args["shape"]), FAKE, FAKE, FAKE, args["ks"],
            args["vs"], FAKE, FAKE, None, FAKE, F(4.0), 4, FAKE, 1 << 30,
            FAKE, None, None, None)

    assert sparse_i8(ks=None) == fb.FD_ERR_INVALID_ARG
    assert sparse_i8(vs=FAKE + 4) == fb.FD_ERR_INVALID_ARG    # not 16-aligned
    assert sparse_i8(shape=s8) == fb.FD_ERR_INVALID_ARG       # E4M3 shape
    assert sparse_i8(shape=s) == fb.FD_ERR_INVALID_ARG        # bf16 shape
    assert lib.fd_build_key_summary_int8(
        ctypes.byref(si), FAKE, None, None, FAKE, FAKE, FAKE,
        None) == fb.FD_ERR_INVALID_ARG
    assert lib.fd_build_key_summary_int8(
        ctypes.byref(s8), FAKE, FAKE, None, FAKE, FAKE, FAKE,
        None) == fb.FD_ERR_INVALID_ARG
    assert sparse(shape=si) == fb.FD_ERR_UNSUPPORTED          # bf16 call
    assert summary8(ks=None) == fb.FD_ERR_INVALID_ARG
    assert summary8(ks=FAKE + 1) == fb.FD_ERR_INVALID_ARG
    assert summary8(shape=s) == fb.FD_ERR_INVALID_ARG         # bf16 shape
    assert summary8(codes=FAKE + 8) == fb.FD_ERR_INVALID_ARG

    def summary(**kw):
        args = dict(shape=s, k=FAKE, bt=None, lens=FAKE, codes=FAKE,
                    scales=FAKE)
        args.update(kw)
        return lib.fd_build_key_summary(
            ctypes.byref(args["shape"]), args["k"], args["bt"], args["lens"],
            args["codes"], args["scales"], None)

    assert summary(codes=None) == fb.FD_ERR_INVALID_ARG
    assert summary(scales=FAKE + 2) == fb.FD_ERR_INVALID_ARG
    assert summary(k=FAKE + 4) == fb.FD_ERR_INVALID_ARG
    assert summary(shape=shp(dtype="f32")) == fb.FD_ERR_UNSUPPORTED
    assert summary(bt=FAKE) == fb.FD_ERR_INVALID_ARG


def test_32bit_index_limits_are_enforced():
    lib = fb.load()
    # batch * kv heads beyond 32-bit row indices
    s = shp(batch=65535, num_q_heads=65536, num_kv_heads=65536, max_seq_len=16)
    out = ctypes.c_int(-99)
    assert lib.fd_plan_splits(ctypes.byref(s), 256, -1,
                              ctypes.byref(out)) == fb.FD_ERR_UNSUPPORTED
    # S * P beyond 32 bits: the history bound near INT32_MAX, P rounded up
    s = shp(max_seq_len=2 ** 31 - 1)
    size = ctypes.c_size_t(0)
    assert lib.fd_workspace_size(ctypes.byref(s), 1,
                                 ctypes.byref(size)) == fb.FD_ERR_UNSUPPORTED
    assert call(shape=s, S=1) == fb.FD_ERR_UNSUPPORTED
    # a bound whose splits fit is fine for sizing
    assert fb.fd_workspace_size(shp(max_seq_len=2 ** 31 - 16), 1) == 0
    assert fb.fd_workspace_size(shp(max_seq_len=2 ** 30), 3) > 0


def call_int8(partials=False, **kw):
    lib = fb.load()
    args = dict(shape=shp(dtype="int8"), q=FAKE, k=FAKE, v=FAKE,
                ks=FAKE, vs=FAKE, bt=None, lens=FAKE, S=4, ws=FAKE,
                ws_bytes=1 << 30, out=FAKE, lse=None)
    args.update(kw)
    if partials:
        return lib.fd_decode_partials_int8(
            ctypes.byref(args["shape"]), args["q"], args["k"], args["v"],
            args["ks"], args["vs"], args["bt"], args["lens"], args["S"],
            args["out"], FAKE, None)
    return lib.fd_decode_attn_int8(ctypes.byref(args["shape"]), args["q"],
                                   args["k"], args["v"], args["ks"],
                                   args["vs"], args["bt"], args["lens"],
                                   args["S"], args["ws"], args["ws_bytes"],
                                   args["out"], args["lse"], None)


@pytest.mark.parametrize("partials", [False, True])
@pytest.mark.parametrize("kw,status", [
    (dict(ks=None), fb.FD_ERR_INVALID_ARG),
    (dict(vs=None), fb.FD_ERR_INVALID_ARG),
    (dict(vs=FAKE + 2), fb.FD_ERR_INVALID_ARG),
    (dict(ks=FAKE + 8), fb.FD_ERR_INVALID_ARG),       # scales: 16-byte
    (dict(shape=shp()), fb.FD_ERR_INVALID_ARG),           # bf16 shape
    (dict(shape=shp(dtype="fp8_e4m3")), fb.FD_ERR_INVALID_ARG),
    (dict(v=FAKE + 4), fb.FD_ERR_INVALID_ARG),
    (dict(shape=shp(dtype="int8", head_dim=96)), fb.FD_ERR_UNSUPPORTED),
    (dict(S=0), fb.FD_ERR_INVALID_ARG),
])
def test_int8_calls_are_rejected_on_the_host(kw, status, partials):
    assert call_int8(partials, **kw) == status


def test_int8_shape_needs_the_int8_entry_points():
    lib = fb.load()
    s = shp(dtype="int8")
    assert call(shape=s) == fb.FD_ERR_INVALID_ARG
    assert call_fp8(shape=s) == fb.FD_ERR_INVALID_ARG
    assert lib.fd_decode_partials(ctypes.byref(s), FAKE, FAKE, FAKE, None,
                                  FAKE, 4, FAKE, FAKE, None) == fb.FD_ERR_INVALID_ARG
    assert call_int8(ws_bytes=100) == fb.FD_ERR_WORKSPACE
    assert fb.fd_plan_splits(s, 256, -1) >= 1
    assert fb.fd_workspace_size(s, 8) == fb.fd_workspace_size(shp(), 8)
    # the sparse path takes bf16 keys only
    assert lib.fd_build_key_summary(ctypes.byref(s), FAKE, None, FAKE, FAKE,
                                    FAKE, None) == fb.FD_ERR_UNSUPPORTED


def test_wrapper_rejects_mismatched_dtypes():
    import torch
    import split_kv_long_amd as fd
    q = torch.zeros(1, 2, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 1, 8, 64, dtype=torch.float32)
    with pytest.raises(ValueError):
        fd.shape_for(q, k, torch.zeros(1, dtype=torch.int32))
    k8 = torch.zeros(1, 1, 8, 64).to(torch.float8_e4m3fn)
    s = fd.shape_for(q, k8, torch.zeros(1, dtype=torch.int32))
    assert s.dtype == fb.FD_DTYPE_FP8_E4M3
    with pytest.raises(ValueError):
        fd.shape_for(q.float(), k8, torch.zeros(1, dtype=torch.int32))
    ki = torch.zeros(1, 1, 8, 64, dtype=torch.int8)
    assert fd.shape_for(q, ki, torch.zeros(1, dtype=torch.int32)).dtype == \
        fb.FD_DTYPE_INT8
    with pytest.raises(ValueError):
        fd.shape_for(q.float(), ki, torch.zeros(1, dtype=torch.int32))


# --------------------------------------------- the header from plain C / C++

def test_header_is_strict_c99_and_cxx(tmp_path):
    import subprocess
    inc = os.path.join(ROOT, "include")
    src = tmp_path / "h.c"
    src.write_text('#include "fd_decode.h"\n#include "fd_probe.h"\n'
                   'int main(void) { fd_shape s;\n'
                   '  (void)s; return FD_OK; }\n')
    subprocess.run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra",
                    "-Werror", "-fsyntax-only", "-I", inc, str(src)],
                   check=True)
    cxx = tmp_path / "h.cpp"
    cxx.write_text(src.read_text())
    subprocess.run(["g++", "-std=c++11", "-pedantic", "-Wall", "-Wextra",
                    "-Werror", "-fsyntax-only", "-I", inc, str(cxx)],
                   check=True)


def test_c_caller_links_and_runs_host_calls(tmp_path):
    """A C program linked against the library plans, sizes and reports
    status strings without a GPU."""
    import subprocess
    import __graft_entry__ as ge
    exe = str(tmp_path / "decode_demo")
    subprocess.run(ge.c_demo_command(ge.C_DEMO_SRC, exe), check=True)
    r = subprocess.run([exe, "host"], capture_output=True, text=True,
                       timeout=60)
    assert r.returncode == 0, r.stderr
    lines = r.stdout.splitlines()
    assert lines[0].startswith("splits 128 workspace ")
    ws = fb.fd_workspace_size(shp(), 128)
    assert lines[0] == f"splits 128 workspace {ws} version {fb.fd_version()}"
    assert lines[1] == "status ok | " + fb.fd_status_str(fb.FD_ERR_WORKSPACE)
    assert lines[2] == f"head_dim 96 -> {fb.FD_ERR_UNSUPPORTED}"


def test_noalloc_entry_point_refuses_oversized_calls():
    """The allocation-free call serves workspaces up to 4 MiB; a larger one
    is refused on the host (FD_ERR_WORKSPACE) before any device access."""
    s = fb.make_shape(64, 32, 8, 128, 1024)
    assert fb.fd_workspace_size(s, 8) > 4 << 20
    with pytest.raises(fb.FdError) as e:
        fb.fd_decode_attn_noalloc(s, 16, 16, 16, None, 16, 8, 16, None,
                                  stream=0)
    assert e.value.status == fb.FD_ERR_WORKSPACE
    # bad shapes and split counts keep their own codes
    with pytest.raises(fb.FdError) as e:
        fb.fd_decode_attn_noalloc(fb.make_shape(1, 3, 2, 128, 64), 16, 16,
                                  16, None, 16, 2, 16, None, stream=0)
    assert e.value.status == fb.FD_ERR_INVALID_ARG
    with pytest.raises(fb.FdError) as e:
        fb.fd_decode_attn_noalloc(fb.make_shape(1, 2, 2, 128, 64), 16, 16,
                                  16, None, 16, 0, 16, None, stream=0)
    assert e.value.status == fb.FD_ERR_INVALID_ARG


@pytest.mark.parametrize("args", [
    # (bytes, workgroups, waves, loads_per_lane)
    (1 << 24, 256, 3, 8),            # waves not 4, 8 or 16
    (1 << 24, 256, 4, 3),            # loads per lane not 2, 4, 8 or 16
    (1 << 26, 256, 16, 16),          # 16 loads per lane need <= 8 waves
    (1 << 24, 0, 4, 8),              # no workgroups
    (1 << 24, 65536, 4, 8),          # grid past 65535
    ((1 << 24) + 16, 256, 4, 8),     # bytes not a multiple of a step
    (0, 256, 4, 8),                  # nothing to read
])
def test_read_probe_rejects_bad_args_on_the_host(args):
    """fd_read_probe validates before it launches anything (a fake aligned
    device address is never dereferenced)."""
    lib = fb.load()
    nbytes, wg, nw, lpl = args
    sink = ctypes.c_void_p(0x10000)
    st = lib.fd_read_probe(ctypes.c_void_p(0x100000), ctypes.c_size_t(nbytes),
                           wg, nw, lpl, sink, None)
    assert st == fb.FD_ERR_INVALID_ARG
    assert lib.fd_read_probe(ctypes.c_void_p(0x100008), ctypes.c_size_t(1 << 24),
                             256, 4, 8, sink, None) == fb.FD_ERR_INVALID_ARG
