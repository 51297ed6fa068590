"""Seeded synthetic ragged batches.

The one module shared by the GPU tests, the oracle tests and the bench.  It
only draws inputs and lays out paged-cache metadata; it computes nothing of
the attention itself.

Recipe (one CPU torch.Generator per batch, drawn in this order):
  1. random context lengths (uniform integers, inclusive bounds), then, for
     shuffled batches, the request order;
  2. a random permutation of the physical page pool, handed out to the
     requests consecutively in request order;
  3. q, k_new, v_new from N(0, 1) in fp32, rounded once to bf16 (RNE);
  4. the cache rows of every prior-context position from N(0, 1) bf16;
  5. every other cache row (free pages, the tail of a last page, and the
     slots the new tokens will be written to) holds the bf16 NaN 0x7FC0, so
     that reading a slot the method must not read shows up as NaN.

Page-table entries past a request's last page are 0 (a valid page): they are
never read, but no stray index can leave the cache.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

NAN_BF16_BITS = 0x7FC0


@dataclass
class Batch:
    q: torch.Tensor  # [T, Hq, D] bf16
    k_new: torch.Tensor  # [T, Hkv, D] bf16
    v_new: torch.Tensor  # [T, Hkv, D] bf16
    k_cache: torch.Tensor  # [P, S, Hkv, D] bf16
    v_cache: torch.Tensor  # [P, S, Hkv, D] bf16
    page_table: torch.Tensor  # [R, max_pages] int32
    cu_q_lens: torch.Tensor  # [R+1] int32
    context_lens: torch.Tensor  # [R] int32
    slot_mapping: torch.Tensor  # [T] int32
    causal: bool = True
    scale: float = 0.0  # 0 means 1/sqrt(D)
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def num_reqs(self):
        return int(self.context_lens.shape[0])

    @property
    def total_tokens(self):
        return int(self.q.shape[0])

    @property
    def num_q_heads(self):
        return int(self.q.shape[1])

    @property
    def num_kv_heads(self):
        return int(self.k_new.shape[1])

    @property
    def head_dim(self):
        return int(self.q.shape[2])

    @property
    def page_size(self):
        return int(self.k_cache.shape[1])

    @property
    def num_pages(self):
        return int(self.k_cache.shape[0])

    @property
    def q_lens(self):
        cu = self.cu_q_lens
        return (cu[1:] - cu[:-1]).tolist()

    def effective_scale(self) -> float:
        return self.scale if self.scale else 1.0 / float(np.sqrt(self.head_dim))


def u16(t: torch.Tensor) -> np.ndarray:
    """Raw bit pattern of a bf16 tensor as a numpy uint16 array (no copy if possible)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _bf16_normal(shape, g) -> torch.Tensor:
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def build_batch(q_lens, ctx_lens, *, num_q_heads, num_kv_heads, head_dim, page_size=16,
                num_pages=None, causal=True, scale=0.0, seed=0, generator=None,
                max_pages_per_req=None, name="") -> Batch:
    """Build a ragged batch with the given per-request new-token and context lengths.

    Draw steps 2-5 of the module recipe happen here; the caller has already
    drawn the lengths (step 1) from the same generator when they are random.
    """
    g = generator if generator is not None else torch.Generator().manual_seed(seed)
    q_lens = [int(x) for x in q_lens]
    ctx_lens = [int(x) for x in ctx_lens]
    R = len(q_lens)
    assert len(ctx_lens) == R
    S, Hq, Hkv, D = page_size, num_q_heads, num_kv_heads, head_dim
    lens = [c + q for c, q in zip(ctx_lens, q_lens)]
    npages = [(L + S - 1) // S for L in lens]
    used = sum(npages)
    P = used if num_pages is None else int(num_pages)
    assert P >= used, f"page pool too small: {P} < {used}"
    maxp = max([1] + npages) if max_pages_per_req is None else int(max_pages_per_req)

    perm = torch.randperm(P, generator=g).to(torch.int32)
    page_table = torch.zeros((R, maxp), dtype=torch.int32)
    off = 0
    for r in range(R):
        page_table[r, : npages[r]] = perm[off : off + npages[r]]
        off += npages[r]

    T = sum(q_lens)
    cu = torch.zeros(R + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(q_lens, dtype=torch.int64), 0).to(torch.int32)
    slot = torch.empty(T, dtype=torch.int64)
    for r in range(R):
        if q_lens[r] == 0:
            continue
        pos = torch.arange(ctx_lens[r], lens[r], dtype=torch.int64)
        pages = page_table[r].to(torch.int64)[pos // S]
        slot[cu[r] : cu[r + 1]] = pages * S + pos % S

    q = _bf16_normal((T, Hq, D), g)
    k_new = _bf16_normal((T, Hkv, D), g)
    v_new = _bf16_normal((T, Hkv, D), g)

    k_cache = torch.full((P, S, Hkv, D), NAN_BF16_BITS, dtype=torch.int16).view(torch.bfloat16)
    v_cache = torch.full((P, S, Hkv, D), NAN_BF16_BITS, dtype=torch.int16).view(torch.bfloat16)
    # Prior-context rows: positions 0..c_r-1 of each request, in request order.
    n_prior = sum(ctx_lens)
    if n_prior:
        rows = torch.empty(n_prior, dtype=torch.int64)
        o = 0
        for r in range(R):
            c = ctx_lens[r]
            if c == 0:
                continue
            pos = torch.arange(0, c, dtype=torch.int64)
            rows[o : o + c] = page_table[r].to(torch.int64)[pos // S] * S + pos % S
            o += c
        kc = k_cache.view(P * S, Hkv, D)
        vc = v_cache.view(P * S, Hkv, D)
        kc[rows] = _bf16_normal((n_prior, Hkv, D), g)
        vc[rows] = _bf16_normal((n_prior, Hkv, D), g)

    return Batch(q=q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache,
                 page_table=page_table, cu_q_lens=cu, context_lens=torch.tensor(ctx_lens, dtype=torch.int32),
                 slot_mapping=slot.to(torch.int32), causal=causal, scale=scale, name=name)


def _uniform(g, lo, hi, n):
    return torch.randint(lo, hi + 1, (n,), generator=g).tolist()


# The workloads: Llama-3-8B attention shapes (Hq=32, Hkv=8, D=128) and a
# head_dim-256 variant, page_size 16, q/k/v from N(0, 1).
CONFIGS = ("tiny", "decode", "prefill", "prefill_noncausal", "mixed", "decode_d256", "prefill_d256")


def config(name: str) -> Batch:
    """One of the named workloads, seeded with 1000 + its index."""
    if name == "tiny":
        # 4 requests: decode with context 37, decode with context 100, a
        # 20-token prefill with no context, a 33-token chunk after 50 tokens.
        # Hq=4, Hkv=2, D=64, 64 physical pages.
        return build_batch([1, 1, 20, 33], [37, 100, 0, 50], num_q_heads=4, num_kv_heads=2,
                           head_dim=64, num_pages=64, seed=1000, name=name)
    if name == "decode":
        g = torch.Generator().manual_seed(1001)
        ctx = _uniform(g, 1024, 8192, 128)
        return build_batch([1] * 128, ctx, num_q_heads=32, num_kv_heads=8, head_dim=128,
                           generator=g, name=name)
    if name in ("prefill", "prefill_noncausal"):
        g = torch.Generator().manual_seed(1002)
        return build_batch([2048] * 4, [0] * 4, num_q_heads=32, num_kv_heads=8, head_dim=128,
                           generator=g, causal=(name == "prefill"), name=name)
    if name == "mixed":
        g = torch.Generator().manual_seed(1003)
        dec_ctx = _uniform(g, 512, 8192, 96)
        pre_ctx = _uniform(g, 0, 4096, 8)
        q_lens = [1] * 96 + [512] * 8
        ctx = dec_ctx + pre_ctx
        order = torch.randperm(104, generator=g).tolist()
        return build_batch([q_lens[i] for i in order], [ctx[i] for i in order], num_q_heads=32,
                           num_kv_heads=8, head_dim=128, generator=g, name=name)
    if name == "decode_d256":
        g = torch.Generator().manual_seed(1004)
        ctx = _uniform(g, 1024, 4096, 128)
        return build_batch([1] * 128, ctx, num_q_heads=16, num_kv_heads=8, head_dim=256,
                           generator=g, name=name)
    if name == "prefill_d256":
        g = torch.Generator().manual_seed(1005)
        return build_batch([2048] * 4, [0] * 4, num_q_heads=16, num_kv_heads=8, head_dim=256,
                           generator=g, name=name)
    raise KeyError(name)


def random_batch(seed, *, num_reqs, max_q, max_ctx, num_q_heads, num_kv_heads, head_dim,
                 page_size=16, causal=True, decode_frac=0.5, extra_pages=3) -> Batch:
    """A small random ragged batch for parity sweeps (decode/prefill mix, empty rows allowed)."""
    g = torch.Generator().manual_seed(seed)
    kinds = torch.rand(num_reqs, generator=g).tolist()
    q_lens, ctx = [], []
    for k in kinds:
        if k < decode_frac:
            q_lens.append(1)
        else:
            q_lens.append(int(torch.randint(0, max_q + 1, (1,), generator=g)))
        ctx.append(int(torch.randint(0, max_ctx + 1, (1,), generator=g)))
    npages = sum((c + q + page_size - 1) // page_size for c, q in zip(ctx, q_lens))
    return build_batch(q_lens, ctx, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                       head_dim=head_dim, page_size=page_size, num_pages=npages + extra_pages,
                       causal=causal, generator=g, name=f"random{seed}")
