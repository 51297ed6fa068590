"""The bench's algorithmic bytes and FLOPs (the numerators of every roofline
figure) against hand-derived values: closed forms for the uniform prefill
workloads, a one-request decode batch counted term by term, and brute-force
pair counts over the tiny workload's requests."""
from __future__ import annotations

import importlib.util
import os
from types import SimpleNamespace

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def lengths(q_lens, ctx, *, hq, hkv, d, s=16, causal=True):
    """Just the metadata the counts read (no tensors of the batch itself)."""
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    return SimpleNamespace(cu_q_lens=torch.from_numpy(cu), context_lens=torch.tensor(ctx, dtype=torch.int32),
                           num_reqs=len(q_lens), num_q_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=s,
                           causal=causal)


def test_prefill_flops_closed_form(bench):
    # 4 x 2048 new tokens, no context, Hq=32, D=128: causal rows see 1..2048 keys.
    b = lengths([2048] * 4, [0] * 4, hq=32, hkv=8, d=128)
    assert bench.algorithmic_flops(b) == 4 * (2048 * 2049 // 2) * 32 * 4 * 128 == 137_506_062_336
    b.causal = False
    assert bench.algorithmic_flops(b) == 4 * 2048 * 2048 * 32 * 4 * 128


def test_flops_brute_force_pairs(bench):
    # The tiny workload's shape: decodes after 37 and 100, a fresh 20-token
    # prefill, a 33-token chunk after 50; count visible (query, key) pairs by
    # enumeration.
    q_lens, ctx = [1, 1, 20, 33], [37, 100, 0, 50]
    for causal in (True, False):
        pairs = 0
        for q, c in zip(q_lens, ctx):
            for i in range(q):
                for j in range(c + q):
                    if not causal or j <= c + i:
                        pairs += 1
        b = lengths(q_lens, ctx, hq=4, hkv=2, d=64, causal=causal)
        assert bench.algorithmic_flops(b) == pairs * 4 * 4 * 64


def test_decode_bytes_term_by_term(bench):
    # One decode request after 100 tokens, Hq=4, Hkv=2, D=64, 16-token pages.
    b = lengths([1], [100], hq=4, hkv=2, d=64)
    prior = 100 * 2 * 64 * 2 * 2        # K and V of the context, bf16
    new_kv = 1 * 2 * 64 * 2 * 2 * 2     # the new K/V row read and written
    q_out = 1 * 4 * 64 * 2 * 2          # q read, out written
    page_ids = 4 * 7                    # ceil(101 / 16) page-table entries
    meta = 4 * (2 + 1) + 4              # cu_q_lens (R + 1), context_lens, slot_mapping
    assert bench.algorithmic_bytes(b) == prior + new_kv + q_out + page_ids + meta == 53_292


def test_bytes_split_by_request_kind(bench):
    # The per-kernel numerators split the batch's bytes by request kind; the
    # parts add up to the whole but for the one shared cu_q_lens entry.
    q_lens, ctx = [1, 512, 1, 1, 300], [4000, 1000, 12, 8191, 0]
    b = lengths(q_lens, ctx, hq=32, hkv=8, d=128)
    dec = [r for r, q in enumerate(q_lens) if q == 1]
    pre = [r for r, q in enumerate(q_lens) if q > 1]
    whole = bench.algorithmic_bytes(b)
    assert bench.algorithmic_bytes(b, dec) + bench.algorithmic_bytes(b, pre) == whole + 4
    # Per context token: 4096 bytes of K and V at Hkv=8, D=128.
    one = lengths([1], [1024], hq=32, hkv=8, d=128)
    two = lengths([1], [2048], hq=32, hkv=8, d=128)
    assert bench.algorithmic_bytes(two) - bench.algorithmic_bytes(one) == 1024 * 4096 + 4 * 64
