"""Host-side checks of the seeded input generators (no GPU, no oracle)."""

import torch

import workloads


def test_recipes_are_seeded_and_deterministic():
    a = workloads.make("tiny_mha")
    b = workloads.make("tiny_mha")
    assert torch.equal(a.q, b.q) and torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
    c = workloads.make("tiny_mha", seed=99)
    assert not torch.equal(a.q, c.q)
    assert a.dtype == "f32" and a.k.shape == (1, 8, 512, 64) and a.scale == 0.125


def test_bf16_values_are_rounded_once():
    w = workloads.make("long_gqa_64k", max_seq_len=256)
    assert w.k.dtype == torch.bfloat16
    g = torch.Generator().manual_seed(2)
    q32 = torch.randn(1, 16, 128, generator=g)
    assert torch.equal(w.q, q32.to(torch.bfloat16))


def test_hot_keys_fraction_and_gain():
    w = workloads.make("ultra_long_256k", max_seq_len=4096)
    n_hot = round(0.001 * 4096)
    assert w.hot_positions.shape == (1, 8, n_hot)
    for h in range(8):
        pos = w.hot_positions[0, h]
        assert len(set(pos.tolist())) == n_hot
        norms = w.k[0, h].float().norm(dim=-1)
        others = torch.ones(4096, dtype=torch.bool)
        others[pos] = False
        assert norms[pos].min() > 5 * norms[others].median()


def test_ragged_paged_table_is_a_permutation():
    w = workloads.make("ragged_paged", max_seq_len=2048, min_seq_len=100)
    lens = w.seq_lens
    assert lens.min() >= 100 and lens.max() <= 2048
    nblk = [(int(n) + 15) // 16 for n in lens]
    used = []
    for b in range(w.batch):
        row = w.block_table[b]
        used += row[:nblk[b]].tolist()
        assert torch.all(row[nblk[b]:] == -1)
    assert sorted(used) == list(range(sum(nblk)))
    assert w.k.shape == (sum(nblk), 8, 16, 128)


def test_poison_only_touches_unattended_slots():
    w = workloads.make("ragged_paged", max_seq_len=200, min_seq_len=1,
                       batch=4, poison_tail=True)
    c = workloads.to_contiguous(w)
    for b in range(4):
        n = int(w.seq_lens[b])
        assert torch.isfinite(c.k[b, :, :n].float()).all()
    # spare block and page tails are NaN
    assert torch.isnan(w.k[-1].float()).all()
    wc = workloads.make("long_gqa_64k", max_seq_len=64, seq_lens=[40],
                        poison_tail=True)
    assert torch.isnan(wc.k[0, :, 40:].float()).all()
    assert torch.isfinite(wc.k[0, :, :40].float()).all()


def test_needles_dominate_their_head():
    w = workloads.make("long_gqa_64k", max_seq_len=512, needles=[0, 300, 511])
    G = 8
    for h in range(2):
        qv = w.q[0, h * G].float()
        logits = (w.k[0, h].float() @ qv) * w.effective_scale
        top = torch.topk(logits, 4).indices.tolist()
        assert set(top[:3]) == {0, 300, 511}
        assert logits[[0, 300, 511]].min() > logits.sort().values[-4] + 25


def test_int8_recipe():
    """int8 caches: codes in [-127, 127], every non-zero row reaching 127
    (scale = amax / 127), fp32 scales laid out like the rows, contiguous
    rows padded with NaN to whole 16-position groups."""
    import math
    import torch
    w = workloads.make("custom", seed=5, batch=2, num_q_heads=8,
                       num_kv_heads=2, head_dim=64, max_seq_len=37,
                       kv_dtype="int8")
    assert w.k.dtype == torch.int8 and w.cache_dtype == "int8"
    assert w.k_scale.shape == (2, 2, 48) and w.k_scale.dtype == torch.float32
    assert torch.isnan(w.k_scale[..., 37:]).all()
    assert torch.isfinite(w.k_scale[..., :37]).all()
    for codes in (w.k, w.v):
        c = codes.to(torch.int32)
        assert int(c.abs().max()) <= 127
        assert (c.abs().amax(dim=-1) == 127).all()
    assert w.kv_bytes() == 2 * 37 * 2 * (2 * 64 + 8)
    p = workloads.make("custom", seed=5, batch=2, num_q_heads=8,
                       num_kv_heads=2, head_dim=64, max_seq_len=37,
                       kv_dtype="int8", paged=True, block_size=16)
    assert p.k_scale.shape == (p.k.shape[0], 2, 16)
    assert not math.isnan(float(p.k_scale[0, 0, 0]))
