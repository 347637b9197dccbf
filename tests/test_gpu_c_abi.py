"""The C ABI from a plain C caller on the GPU (needs a gfx950 GPU).

``tests/c_abi/decode_demo`` (built by ``__graft_entry__.build()`` from
``decode_demo.c``) allocates device memory with HIP, plans the splits and
calls ``fd_decode_attn`` with raw pointers; no Python or torch sits between
it and the library. Its output is compared with the float64 oracle at the
bf16 bar (2e-3 on out, 1e-4 on lse).
"""

import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEMO = os.path.join(ROOT, "tests", "c_abi", "decode_demo")


@pytest.mark.parametrize("lens", [[1000, 1, 517], [65536]])
def test_c_caller_matches_oracle(tmp_path, lens):
    assert os.path.exists(DEMO), "run __graft_entry__.build() first"
    L = max(lens)
    w = workloads.make("c_abi", seed=77, batch=len(lens), num_q_heads=16,
                       num_kv_heads=2, head_dim=128, max_seq_len=L,
                       seq_lens=lens)
    a = w.numpy_view()
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(np.array([w.batch, w.num_q_heads, w.num_kv_heads,
                          w.head_dim, L], dtype="<i4").tobytes())
        for x in (a["q"], a["k"], a["v"]):
            f.write(np.ascontiguousarray(x, dtype="<u2").tobytes())
        f.write(np.asarray(lens, dtype="<i4").tobytes())
    print(f"[gpu] C caller lens={lens}", flush=True)
    r = subprocess.run([DEMO, "run", str(src), str(dst)], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = dst.read_bytes()
    S = int(np.frombuffer(raw[:4], dtype="<i4")[0])
    n_out = w.batch * w.num_q_heads * w.head_dim
    out = np.frombuffer(raw[4:4 + 4 * n_out], dtype="<f4").reshape(
        w.batch, w.num_q_heads, w.head_dim).astype(np.float64)
    lse = np.frombuffer(raw[4 + 4 * n_out:], dtype="<f4").reshape(
        w.batch, w.num_q_heads).astype(np.float64)
    ref, ref_lse = oracle.decode_attention(a["q"], a["k"], a["v"],
                                           a["seq_lens"], dtype="bf16")
    assert S >= 1
    assert np.abs(out - ref).max() <= 2e-3
    assert np.abs(lse - ref_lse).max() <= 1e-4
