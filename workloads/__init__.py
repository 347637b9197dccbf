"""Seeded synthetic decode-attention workloads.

This module only draws random inputs and lays them out in memory. It holds
none of the attention arithmetic, so both the float64 oracle (via the numpy
views) and the HIP library (via the torch tensors) can be fed from it without
sharing any code of the method.

Five named workloads follow the shapes of the long-context decode settings the
Flash-Decoding pages discuss (batch-one long history, a GQA model share, a
ragged paged batch, and the short-history / large-batch regime where the pages
say splitting stops paying). Every value is drawn on the CPU from
``torch.Generator().manual_seed(seed)`` as float32 N(0, 1) and, for bf16
workloads, rounded once to bfloat16 (round-to-nearest-even by torch). The
rounded values are the ground truth that both sides read.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

F32 = "f32"
BF16 = "bf16"
FP8 = "fp8_e4m3"
FP8_MAX = 448.0   # largest finite E4M3 magnitude
INT8 = "int8"
INT8_MAX = 127.0

# name -> recipe. seed = workload id.
SPECS = {
    "tiny_mha": dict(
        wid=1, batch=1, num_q_heads=8, num_kv_heads=8, head_dim=64,
        max_seq_len=512, dtype=F32, scale=1.0 / 8.0, paged=False,
        compare_splits=[1, 4]),
    "long_gqa_64k": dict(
        wid=2, batch=1, num_q_heads=16, num_kv_heads=2, head_dim=128,
        max_seq_len=65536, dtype=BF16, scale=None, paged=False),
    "ultra_long_256k": dict(
        wid=3, batch=1, num_q_heads=64, num_kv_heads=8, head_dim=128,
        max_seq_len=262144, dtype=BF16, scale=None, paged=False,
        hot_key_fraction=0.001, hot_key_gain=20.0),
    "ragged_paged": dict(
        wid=4, batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128,
        max_seq_len=32768, min_seq_len=512, dtype=BF16, scale=None,
        paged=True, block_size=16),
    # The 64K history in an 8-bit E4M3 cache: the same draws as long_gqa_64k,
    # each kv head's K and V divided by amax/448 and rounded to E4M3.
    "long_gqa_64k_fp8": dict(
        wid=2, batch=1, num_q_heads=16, num_kv_heads=2, head_dim=128,
        max_seq_len=65536, dtype=BF16, kv_dtype=FP8, scale=None,
        paged=False),
    # The same history in an 8-bit integer cache with one scale per
    # (position, kv head): each row of K and V divided by amax/127 and
    # rounded to the nearest integer.
    "long_gqa_64k_int8": dict(
        wid=2, batch=1, num_q_heads=16, num_kv_heads=2, head_dim=128,
        max_seq_len=65536, dtype=BF16, kv_dtype=INT8, scale=None,
        paged=False),
    # Needle-in-a-haystack structure (the retrieval-style long-context
    # evaluations the "Faster Than Flash" page cites): haystack keys scaled
    # so logits have std ~0.3, and in every 512-token chunk one 16-token
    # block of keys every head of a kv group scores at logit ~6.
    "needle_haystack_64k": dict(
        wid=7, batch=1, num_q_heads=16, num_kv_heads=2, head_dim=128,
        max_seq_len=65536, dtype=BF16, scale=None, paged=False,
        haystack_gain=0.3, needle_block_every=512, needle_block_logit=6.0),
    "short_batch": dict(
        wid=5, batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128,
        max_seq_len=1024, dtype=BF16, scale=None, paged=False,
        compare_splits=[1, 2, 8]),
    # The ragged batch's lengths in a contiguous [B, Hkv, L, D] cache, to
    # separate paging cost from ragged-length imbalance when measuring.
    "ragged_contig": dict(
        wid=4, batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128,
        max_seq_len=32768, min_seq_len=512, dtype=BF16, scale=None,
        paged=False),
}

ORDER = ["tiny_mha", "long_gqa_64k", "ultra_long_256k", "ragged_paged",
         "short_batch"]
# Further measured workloads (variants of the above).
EXTRA = ["long_gqa_64k_fp8", "long_gqa_64k_int8"]


@dataclasses.dataclass
class Workload:
    """One decode-attention call's inputs, resident on the CPU.

    Layouts (row-major):
      q            [B, Hq, D]
      k, v         contiguous: [B, Hkv, L, D]; paged: [NB, Hkv, bs, D]
      block_table  int32 [B, max_blocks] (paged only; unused entries = -1)
      seq_lens     int32 [B]
    """
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    max_seq_len: int
    dtype: str
    scale: Optional[float]
    block_size: int
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    seq_lens: torch.Tensor
    block_table: Optional[torch.Tensor]
    hot_positions: Optional[torch.Tensor] = None   # [B, Hkv, n_hot]
    kv_dtype: Optional[str] = None                 # None: same as dtype
    # Quantized caches: fp32 [Hkv] (E4M3), or one per (position, kv head)
    # (int8): contiguous [B, Hkv, Lp] with rows padded to Lp =
    # ceil(L / 16) * 16 (padding NaN), paged [NB, Hkv, bs].
    k_scale: Optional[torch.Tensor] = None
    v_scale: Optional[torch.Tensor] = None

    @property
    def cache_dtype(self) -> str:
        return self.kv_dtype or self.dtype

    @property
    def paged(self) -> bool:
        return self.block_size > 0

    @property
    def num_blocks(self) -> int:
        return int(self.k.shape[0]) if self.paged else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1]) if self.paged else 0

    @property
    def effective_scale(self) -> float:
        return self.scale if self.scale else 1.0 / math.sqrt(self.head_dim)

    def sum_seq_len(self) -> int:
        return int(self.seq_lens.to(torch.int64).sum())

    def kv_bytes(self) -> int:
        """K+V bytes the call must read: every attended row, once (with its
        two fp32 scales for an int8 cache)."""
        esz = {F32: 4, BF16: 2, FP8: 1, INT8: 1}[self.cache_dtype]
        row = 2 * self.head_dim * esz + (8 if self.cache_dtype == INT8 else 0)
        return self.sum_seq_len() * self.num_kv_heads * row

    def numpy_view(self) -> dict:
        """Raw arrays for the oracle: bf16 as uint16 bit patterns, E4M3 as
        uint8 codes, int8 and f32 as they are."""
        def raw(t):
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16)
            if t.dtype == torch.float8_e4m3fn:
                return t.view(torch.uint8).numpy()
            return t.numpy()
        return dict(
            q=raw(self.q), k=raw(self.k), v=raw(self.v),
            seq_lens=self.seq_lens.numpy().astype(np.int64),
            block_table=(None if self.block_table is None
                         else self.block_table.numpy().astype(np.int64)),
            block_size=self.block_size, dtype=self.dtype,
            scale=self.effective_scale, kv_dtype=self.cache_dtype,
            k_scale=(None if self.k_scale is None
                     else self.k_scale.numpy().astype(np.float64)),
            v_scale=(None if self.v_scale is None
                     else self.v_scale.numpy().astype(np.float64)))

    def shape_dict(self) -> dict:
        return dict(batch=self.batch, num_q_heads=self.num_q_heads,
                    num_kv_heads=self.num_kv_heads, head_dim=self.head_dim,
                    max_seq_len=self.max_seq_len, block_size=self.block_size,
                    max_blocks_per_seq=self.max_blocks_per_seq,
                    num_blocks=self.num_blocks, dtype=self.cache_dtype,
                    scale=self.scale or 0.0)


def _cast(x: torch.Tensor, dtype: str) -> torch.Tensor:
    return x.to(torch.bfloat16) if dtype == BF16 else x.contiguous()


def make(name: str = "custom", *, seed: Optional[int] = None,
         batch: Optional[int] = None, num_q_heads: Optional[int] = None,
         num_kv_heads: Optional[int] = None, head_dim: Optional[int] = None,
         max_seq_len: Optional[int] = None, dtype: Optional[str] = None,
         scale: Optional[float] = "spec", paged: Optional[bool] = None,
         block_size: Optional[int] = None,
         seq_lens: Optional[Sequence[int]] = None,
         min_seq_len: Optional[int] = None,
         hot_key_fraction: float = None, hot_key_gain: float = None,
         poison_tail: bool = False,
         needles: Optional[Sequence[int]] = None,
         needle_logit: float = 40.0,
         kv_dtype: Optional[str] = None,
         haystack_gain: Optional[float] = None,
         needle_block_every: Optional[int] = None,
         needle_block_logit: Optional[float] = None) -> Workload:
    """Build a workload from a named recipe, with optional overrides.

    Draw order on one CPU generator: seq_lens (ragged recipes only), q, k, v,
    then the hot-key positions, then the block-table permutation.

    poison_tail: fill every cache slot that is NOT attended (positions at or
      beyond seq_lens[b] in the contiguous layout; slots past the end of the
      last page, and every unreferenced pool block, in the paged layout) with
      NaN, so any read of an unattended slot shows up in the output.
    needles: token positions p; for every (b, kv head) the key at p is set to
      c * q[b, first head of the group] with c chosen so that head's logit is
      ``needle_logit``, far above the N(0, 1)-scale logits of the other keys.
    haystack_gain / needle_block_every / needle_block_logit: multiply every
      key by haystack_gain, then in each chunk of needle_block_every
      positions set one 16-aligned block (offset drawn after the block
      table) of each (b, kv head) to the minimum-norm key on which every
      query head of the group scores exactly needle_block_logit (before
      bf16 rounding).
    kv_dtype: "fp8_e4m3" stores K and V as 8-bit E4M3 codes: per kv head,
      scale = amax / 448 over that head's whole pool (fp32), codes =
      E4M3(x / scale) rounded by torch; q stays bf16. "int8" stores them as
      8-bit integers with one fp32 scale per (position, kv head): scale =
      amax / 127 over the row's head_dim values (1 for an all-zero row),
      codes = round(x / scale) (torch, ties to even), q bf16; contiguous
      scale rows are padded with NaN to whole 16-position groups. With
      poison_tail an int8 cache's unattended slots get code 127 and scale
      NaN.
    """
    spec = dict(SPECS.get(name, {}))
    wid = spec.get("wid", 0)
    seed = wid if seed is None else seed
    B = batch or spec.get("batch", 1)
    Hq = num_q_heads or spec.get("num_q_heads", 8)
    Hkv = num_kv_heads or spec.get("num_kv_heads", Hq)
    D = head_dim or spec.get("head_dim", 128)
    L = max_seq_len if max_seq_len is not None else spec.get("max_seq_len", 512)
    dt = dtype or spec.get("dtype", BF16)
    kvd = kv_dtype or spec.get("kv_dtype")
    assert kvd in (None, FP8, INT8) and (kvd is None or dt == BF16)
    sc = spec.get("scale") if scale == "spec" else scale
    pg = spec.get("paged", False) if paged is None else paged
    # An explicit page size overrides the recipe's (16 when neither says).
    bs = ((block_size if block_size is not None
           else spec.get("block_size", 16)) if pg else 0)
    hk_frac = (spec.get("hot_key_fraction", 0.0) if hot_key_fraction is None
               else hot_key_fraction)
    hk_gain = (spec.get("hot_key_gain", 1.0) if hot_key_gain is None
               else hot_key_gain)
    assert Hq % Hkv == 0
    g = torch.Generator().manual_seed(int(seed))

    if seq_lens is not None:
        lens = torch.tensor(list(seq_lens), dtype=torch.int32)
        assert lens.numel() == B
    elif "min_seq_len" in spec or min_seq_len is not None:
        lo = min_seq_len if min_seq_len is not None else spec["min_seq_len"]
        lens = torch.randint(lo, L + 1, (B,), generator=g, dtype=torch.int64)
        lens = lens.to(torch.int32)
    else:
        lens = torch.full((B,), L, dtype=torch.int32)
    if lens.numel():
        assert int(lens.max()) <= L and int(lens.min()) >= 0

    q32 = torch.randn(B, Hq, D, generator=g)
    if pg:
        nblk = [(int(n) + bs - 1) // bs for n in lens]
        NB = sum(nblk)
        NBalloc = max(NB, 1) + (1 if poison_tail else 0)  # one spare block
        k32 = torch.randn(NBalloc, Hkv, bs, D, generator=g)
        v32 = torch.randn(NBalloc, Hkv, bs, D, generator=g)
    else:
        k32 = torch.randn(B, Hkv, L, D, generator=g)
        v32 = torch.randn(B, Hkv, L, D, generator=g)

    hot = None
    if hk_frac and hk_frac > 0:
        assert not pg
        n_hot = int(round(hk_frac * L))
        hot = torch.empty(B, Hkv, n_hot, dtype=torch.int64)
        for b in range(B):
            for h in range(Hkv):
                hot[b, h] = torch.randperm(L, generator=g)[:n_hot]
                k32[b, h, hot[b, h]] *= hk_gain

    bt = None
    if pg:
        perm = torch.randperm(NB, generator=g).to(torch.int32)
        maxb = max((L + bs - 1) // bs, 1)
        bt = torch.full((B, maxb), -1, dtype=torch.int32)
        off = 0
        for b in range(B):
            bt[b, :nblk[b]] = perm[off:off + nblk[b]]
            off += nblk[b]

    q = _cast(q32, dt)
    hg = haystack_gain if haystack_gain is not None else spec.get(
        "haystack_gain")
    nbe = needle_block_every or spec.get("needle_block_every")
    nbl = needle_block_logit if needle_block_logit is not None else spec.get(
        "needle_block_logit", 6.0)
    if hg is not None:
        k32 *= hg
    if nbe:
        assert not pg and nbe % 16 == 0
        scl = sc if sc else 1.0 / math.sqrt(D)
        G = Hq // Hkv
        qd = q.to(torch.float32)
        offs = torch.randint(0, nbe // 16, (-(-L // nbe),), generator=g)
        for b in range(B):
            for h in range(Hkv):
                qs = qd[b, h * G:(h + 1) * G].to(torch.float64)
                # minimum-norm key with scl * <q_h, key> = nbl for every h
                tgt = torch.full((G,), nbl / scl, dtype=torch.float64)
                key = (qs.T @ torch.linalg.solve(qs @ qs.T, tgt)).float()
                for c in range(-(-L // nbe)):
                    p0 = c * nbe + 16 * int(offs[c])
                    k32[b, h, p0:min(p0 + 16, L)] = key
    if needles:
        scl = sc if sc else 1.0 / math.sqrt(D)
        G = Hq // Hkv
        qd = q.to(torch.float32)
        for b in range(B):
            for h in range(Hkv):
                qv = qd[b, h * G]
                c = needle_logit / (scl * float(qv @ qv))
                for p in needles:
                    if p >= int(lens[b]):
                        continue
                    if pg:
                        blk = int(bt[b, p // bs])
                        k32[blk, h, p % bs] = c * qv
                    else:
                        k32[b, h, p] = c * qv
    ks = vs = None
    if kvd == FP8:
        def quant(x):
            amax = x.abs().amax(dim=(0, 2, 3))
            sc = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
            sc = sc.to(torch.float32)
            return (x / sc[None, :, None, None]).to(torch.float8_e4m3fn), sc
        k, ks = quant(k32)
        v, vs = quant(v32)
    elif kvd == INT8:
        def quant(x):
            amax = x.abs().amax(dim=-1)
            sc = torch.where(amax > 0, amax / INT8_MAX, torch.ones_like(amax))
            sc = sc.to(torch.float32)
            c = torch.round(x / sc[..., None]).clamp(-INT8_MAX, INT8_MAX)
            if not pg:      # scale rows padded to whole 16-position groups
                pad = torch.full(sc.shape[:-1] + (-(-L // 16) * 16,),
                                 float("nan"))
                pad[..., :L] = sc
                sc = pad
            return c.to(torch.int8), sc
        k, ks = quant(k32)
        v, vs = quant(v32)
    else:
        k = _cast(k32, dt)
        v = _cast(v32, dt)

    if poison_tail and kvd == INT8:
        # No NaN code: the codes get 127 and the scales NaN instead.
        nan = float("nan")
        if pg:
            used = torch.zeros(k.shape[0], dtype=torch.bool)
            for b in range(B):
                n = int(lens[b])
                nb = (n + bs - 1) // bs
                for j in range(nb):
                    used[int(bt[b, j])] = True
                if n % bs:
                    last = int(bt[b, nb - 1])
                    for t, st in ((k, ks), (v, vs)):
                        t[last, :, n % bs:] = 127
                        st[last, :, n % bs:] = nan
            for t, st in ((k, ks), (v, vs)):
                t[~used] = 127
                st[~used] = nan
        else:
            for b in range(B):
                n = int(lens[b])
                for t, st in ((k, ks), (v, vs)):
                    t[b, :, n:] = 127
                    st[b, :, n:] = nan
    elif poison_tail:
        nan = float("nan")
        if kvd == FP8:     # poison through the byte view (0x7F is NaN)
            k = k.view(torch.uint8).to(torch.float32)
            v = v.view(torch.uint8).to(torch.float32)
        if pg:
            used = torch.zeros(k.shape[0], dtype=torch.bool)
            for b in range(B):
                n = int(lens[b])
                nb = (n + bs - 1) // bs
                for j in range(nb):
                    used[int(bt[b, j])] = True
                if n % bs:
                    last = int(bt[b, nb - 1])
                    k[last, :, n % bs:] = nan
                    v[last, :, n % bs:] = nan
            k[~used] = nan
            v[~used] = nan
        else:
            for b in range(B):
                n = int(lens[b])
                k[b, :, n:] = nan
                v[b, :, n:] = nan
        if kvd == FP8:
            k = torch.where(torch.isnan(k), 0x7F, k).to(torch.uint8).view(
                torch.float8_e4m3fn)
            v = torch.where(torch.isnan(v), 0x7F, v).to(torch.uint8).view(
                torch.float8_e4m3fn)

    return Workload(name=name, batch=B, num_q_heads=Hq, num_kv_heads=Hkv,
                    head_dim=D, max_seq_len=L, dtype=dt, scale=sc,
                    block_size=bs, q=q.contiguous(), k=k.contiguous(),
                    v=v.contiguous(), seq_lens=lens, block_table=bt,
                    hot_positions=hot, kv_dtype=kvd,
                    k_scale=None if ks is None else ks.contiguous(),
                    v_scale=None if vs is None else vs.contiguous())


def to_contiguous(w: Workload) -> Workload:
    """Re-lay a paged workload as [B, Hkv, L, D] (same values, no arithmetic)."""
    assert w.paged
    B, Hkv, D, L, bs = (w.batch, w.num_kv_heads, w.head_dim, w.max_seq_len,
                        w.block_size)
    k = torch.zeros(B, Hkv, L, D, dtype=w.k.dtype)
    v = torch.zeros(B, Hkv, L, D, dtype=w.v.dtype)
    rows = w.k_scale is not None and w.k_scale.dim() == 3
    Lp = -(-L // 16) * 16
    ks = torch.full((B, Hkv, Lp), float("nan")) if rows else w.k_scale
    vs = torch.full((B, Hkv, Lp), float("nan")) if rows else w.v_scale
    for b in range(B):
        n = int(w.seq_lens[b])
        for j in range((n + bs - 1) // bs):
            blk = int(w.block_table[b, j])
            t0, t1 = j * bs, min((j + 1) * bs, n)
            k[b, :, t0:t1] = w.k[blk, :, :t1 - t0]
            v[b, :, t0:t1] = w.v[blk, :, :t1 - t0]
            if rows:
                ks[b, :, t0:t1] = w.k_scale[blk, :, :t1 - t0]
                vs[b, :, t0:t1] = w.v_scale[blk, :, :t1 - t0]
    return dataclasses.replace(w, name=w.name + "/contig", k=k, v=v,
                               block_size=0, block_table=None, k_scale=ks,
                               v_scale=vs)
