"""Pins of the fp64 CPU oracle against things other than itself.

* dense gathered numpy formulation and torch SDPA (fp64, CPU) on seeded batches;
* hand-derived closed forms (tests/golden/closed_forms.json) and brute-force
  special cases (one key, all-equal keys, zero query, one dominant logit);
* invariants: physical-page permutation, request order, V shift, V linearity,
  equal q heads within a group;
* the scatter, bit for bit, including the untouched rows;
* the precondition checker, rule by rule;
* planted mistakes: mutated copies of oracle.c must fail at least one pin.
"""
from __future__ import annotations

import json
import math
import os
import re
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
from ragged_paged_attention_amd.inputs import (Batch, build_batch, config, random_batch, u16)
from tests.dense_ref import dense_numpy, sdpa_torch, widen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def run_oracle(b: Batch, lib=None):
    return oracle.forward(u16(b.q), u16(b.k_new), u16(b.v_new), u16(b.k_cache), u16(b.v_cache),
                          b.page_table.numpy(), b.cu_q_lens.numpy(), b.context_lens.numpy(),
                          b.slot_mapping.numpy(), scale=b.effective_scale(), causal=b.causal,
                          lib=lib)


def small_batches():
    out = [config("tiny")]
    for s in range(6):
        out.append(random_batch(100 + s, num_reqs=5, max_q=40, max_ctx=70, num_q_heads=4,
                                num_kv_heads=2, head_dim=16, page_size=8,
                                causal=(s % 3 != 2)))
    out.append(random_batch(200, num_reqs=3, max_q=9, max_ctx=20, num_q_heads=3,
                            num_kv_heads=1, head_dim=8, page_size=4))
    out.append(random_batch(201, num_reqs=4, max_q=12, max_ctx=30, num_q_heads=2,
                            num_kv_heads=2, head_dim=8, page_size=16))
    return out


# --------------------------------------------------------------------------
# Independent formulations
# --------------------------------------------------------------------------
@pytest.mark.parametrize("idx", range(9))
def test_matches_dense_numpy(idx):
    b = small_batches()[idx]
    out, _, _ = run_oracle(b)
    ref = dense_numpy(b)
    assert np.max(np.abs(out - ref), initial=0.0) < 1e-12


@pytest.mark.parametrize("idx", [0, 1, 3, 7])
def test_matches_torch_sdpa(idx):
    b = small_batches()[idx]
    out, _, _ = run_oracle(b)
    ref = sdpa_torch(b)
    assert np.max(np.abs(out - ref), initial=0.0) < 1e-10


# --------------------------------------------------------------------------
# Closed forms
# --------------------------------------------------------------------------
def _golden_batch(case) -> Batch:
    def bf(x):
        a = np.array(x, dtype=object)
        f = np.vectorize(lambda v: np.nan if v == "NaN" else float(v))(a).astype(np.float32)
        t = torch.from_numpy(f).to(torch.bfloat16)
        back = t.to(torch.float32).numpy()
        ok = np.isnan(f) | (back == f)
        assert ok.all(), "golden value not exact in bf16"
        return t

    scale = case["scale"]
    scale = {"ln3": math.log(3.0), "ln2": math.log(2.0)}.get(scale, scale)
    return Batch(q=bf(case["q"]), k_new=bf(case["k_new"]), v_new=bf(case["v_new"]),
                 k_cache=bf(case["k_cache"]), v_cache=bf(case["v_cache"]),
                 page_table=torch.tensor(case["page_table"], dtype=torch.int32),
                 cu_q_lens=torch.tensor(case["cu_q_lens"], dtype=torch.int32),
                 context_lens=torch.tensor(case["context_lens"], dtype=torch.int32),
                 slot_mapping=torch.tensor(case["slot_mapping"], dtype=torch.int32),
                 causal=bool(case["causal"]), scale=float(scale), name=case["name"])


def golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", golden_cases(), ids=lambda c: c["name"])
def test_golden_closed_forms(case):
    b = _golden_batch(case)
    out, kc, vc = run_oracle(b)
    np.testing.assert_allclose(out, np.array(case["expected_out"], dtype=np.float64),
                               rtol=0, atol=1e-12)
    # the new rows landed where slot_mapping says, bit for bit
    S = b.page_size
    for t, slot in enumerate(b.slot_mapping.tolist()):
        assert (kc[slot // S, slot % S] == u16(b.k_new)[t]).all()
        assert (vc[slot // S, slot % S] == u16(b.v_new)[t]).all()


def test_single_key_returns_its_value():
    # context 0 and one new token: softmax over one key is 1, out = v exactly.
    b = build_batch([1, 1], [0, 0], num_q_heads=4, num_kv_heads=2, head_dim=32, seed=7)
    out, _, _ = run_oracle(b)
    v = widen(u16(b.v_new))
    for h in range(4):
        assert np.array_equal(out[:, h, :], v[:, h // 2, :])


def test_first_row_of_fresh_prefill_is_exact():
    # causal prefill from context 0: query 0 sees only key 0.
    b = build_batch([9], [0], num_q_heads=2, num_kv_heads=1, head_dim=16, seed=8)
    out, _, _ = run_oracle(b)
    assert np.array_equal(out[0, 0], widen(u16(b.v_new))[0, 0])


def _set_all(t: torch.Tensor, value: float):
    t.view(torch.int16)[...] = torch.tensor(value, dtype=torch.bfloat16).view(torch.int16)


def test_equal_keys_give_mean_of_visible_values():
    b = build_batch([5, 1], [11, 6], num_q_heads=2, num_kv_heads=1, head_dim=8, seed=9)
    # every key identical -> every logit equal -> uniform weights
    _set_all(b.k_new, 0.5)
    kc = b.k_cache.view(torch.int16)
    nan = torch.tensor(0x7FC0, dtype=torch.int16)
    prior = kc != nan
    kc[prior] = torch.tensor(0.5, dtype=torch.bfloat16).view(torch.int16)
    out, _, _ = run_oracle(b)
    for r in range(b.num_reqs):
        from tests.dense_ref import request_sequences
        _, V = request_sequences(b, r)
        c = int(b.context_lens[r])
        for i, t in enumerate(range(int(b.cu_q_lens[r]), int(b.cu_q_lens[r + 1]))):
            want = V[: c + i + 1, 0, :].mean(axis=0)
            np.testing.assert_allclose(out[t, 0], want, rtol=0, atol=1e-13)
            np.testing.assert_allclose(out[t, 1], want, rtol=0, atol=1e-13)


def test_zero_query_gives_mean_of_visible_values():
    b = build_batch([4], [13], num_q_heads=2, num_kv_heads=2, head_dim=8, seed=10)
    _set_all(b.q, 0.0)
    out, _, _ = run_oracle(b)
    from tests.dense_ref import request_sequences
    _, V = request_sequences(b, 0)
    for i in range(4):
        for h in range(2):
            np.testing.assert_allclose(out[i, h], V[: 13 + i + 1, h].mean(axis=0), atol=1e-13)


def test_dominant_logit_selects_its_value():
    # q = 8 e0, key of position 5 = 8 e0, all others 0, scale 1: logit 64 vs 0.
    b = build_batch([1], [9], num_q_heads=1, num_kv_heads=1, head_dim=8, seed=11, page_size=4)
    _set_all(b.q, 0.0)
    _set_all(b.k_new, 0.0)
    kc = b.k_cache.view(torch.int16)
    prior = kc != torch.tensor(0x7FC0, dtype=torch.int16)
    kc[prior] = 0
    b.q.view(torch.int16)[0, 0, 0] = torch.tensor(8.0, dtype=torch.bfloat16).view(torch.int16)
    row = int(b.page_table[0, 5 // 4]) * 4 + 5 % 4
    b.k_cache.view(-1, 1, 8)[row, 0, 0] = 8.0
    b.scale = 1.0
    out, _, _ = run_oracle(b)
    from tests.dense_ref import request_sequences
    _, V = request_sequences(b, 0)
    np.testing.assert_allclose(out[0, 0], V[5, 0], rtol=0, atol=1e-20 + 40 * math.exp(-64))


@pytest.mark.parametrize("idx", [0, 1, 3, 7])
def test_attention_rows_matches_dense_and_full(idx):
    """oracle_attention_rows (the per-(token, head) entry the long-chunk GPU
    test samples with) against the independent dense numpy formulation, and
    bit for bit against the whole-batch oracle_attention: random (token, head)
    pairs in random order, repeats included, every first and last token of a
    request and every q head."""
    b = small_batches()[idx]
    out, kc, vc = run_oracle(b)
    dense = dense_numpy(b)
    rng = np.random.default_rng(40 + idx)
    T, Hq = b.total_tokens, b.num_q_heads
    cu = b.cu_q_lens.tolist()
    edge = [t for r in range(b.num_reqs) if cu[r + 1] > cu[r] for t in (cu[r], cu[r + 1] - 1)]
    tokens = np.concatenate([rng.integers(0, T, 3 * T), np.repeat(edge, Hq)]).astype(np.int32)
    heads = np.concatenate([rng.integers(0, Hq, 3 * T), np.tile(np.arange(Hq), len(edge))]).astype(np.int32)
    perm = rng.permutation(len(tokens))
    tokens, heads = tokens[perm], heads[perm]
    rows = oracle.attention_rows(u16(b.q), kc, vc, b.page_table.numpy(), b.cu_q_lens.numpy(),
                                 b.context_lens.numpy(), tokens, heads, scale=b.effective_scale(),
                                 causal=b.causal)
    np.testing.assert_allclose(rows, dense[tokens, heads], rtol=0, atol=1e-12)
    assert np.array_equal(rows, out[tokens, heads])


# --------------------------------------------------------------------------
# Invariants
# --------------------------------------------------------------------------
def permute_pages(b: Batch, perm: np.ndarray) -> Batch:
    """Move physical page p to perm[p]; remap page_table and slot_mapping."""
    P, S = b.num_pages, b.page_size
    inv = np.argsort(perm)
    kc = b.k_cache[torch.from_numpy(inv)].clone()
    vc = b.v_cache[torch.from_numpy(inv)].clone()
    pt = torch.from_numpy(perm[b.page_table.numpy()].astype(np.int32))
    sm = b.slot_mapping.numpy().astype(np.int64)
    sm = torch.from_numpy((perm[sm // S] * S + sm % S).astype(np.int32))
    return Batch(q=b.q, k_new=b.k_new, v_new=b.v_new, k_cache=kc, v_cache=vc, page_table=pt,
                 cu_q_lens=b.cu_q_lens, context_lens=b.context_lens, slot_mapping=sm,
                 causal=b.causal, scale=b.scale)


@pytest.mark.parametrize("idx", [0, 2, 5])
def test_page_permutation_invariance(idx):
    b = small_batches()[idx]
    perm = np.random.default_rng(idx).permutation(b.num_pages)
    out, kc, _ = run_oracle(b)
    bp = permute_pages(b, perm)
    out2, kc2, _ = run_oracle(bp)
    assert np.array_equal(out, out2)
    # the caches agree after undoing the permutation
    assert np.array_equal(kc, kc2[perm])


def reorder_requests(b: Batch, order) -> tuple[Batch, np.ndarray]:
    """Requests in a new order; returns the batch and the new->old token map."""
    cu = b.cu_q_lens.tolist()
    tok = np.concatenate([np.arange(cu[r], cu[r + 1]) for r in order]).astype(np.int64)
    q_lens = [cu[r + 1] - cu[r] for r in order]
    ncu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    idx = torch.from_numpy(tok)
    nb = Batch(q=b.q[idx], k_new=b.k_new[idx], v_new=b.v_new[idx], k_cache=b.k_cache,
               v_cache=b.v_cache, page_table=b.page_table[list(order)],
               cu_q_lens=torch.from_numpy(ncu), context_lens=b.context_lens[list(order)],
               slot_mapping=b.slot_mapping[idx], causal=b.causal, scale=b.scale)
    return nb, tok


@pytest.mark.parametrize("idx", [0, 1, 4])
def test_request_order_invariance(idx):
    b = small_batches()[idx]
    order = np.random.default_rng(idx + 50).permutation(b.num_reqs)
    out, kc, vc = run_oracle(b)
    nb, tok = reorder_requests(b, order)
    out2, kc2, vc2 = run_oracle(nb)
    assert np.array_equal(out[tok], out2)
    assert np.array_equal(kc, kc2) and np.array_equal(vc, vc2)


def _grid_values(b: Batch, seed, lo=-4, hi=4):
    """Overwrite V (cache rows in use and v_new) with small integers: sums stay exact."""
    g = torch.Generator().manual_seed(seed)
    vn = torch.randint(lo, hi + 1, b.v_new.shape, generator=g).to(torch.bfloat16)
    vc = b.v_cache.clone()
    used = vc.view(torch.int16) != torch.tensor(0x7FC0, dtype=torch.int16)
    vc[used] = torch.randint(lo, hi + 1, (int(used.sum()),), generator=g).to(torch.bfloat16)
    return vn, vc


def _with_v(b: Batch, v_new, v_cache) -> Batch:
    return Batch(q=b.q, k_new=b.k_new, v_new=v_new, k_cache=b.k_cache, v_cache=v_cache,
                 page_table=b.page_table, cu_q_lens=b.cu_q_lens, context_lens=b.context_lens,
                 slot_mapping=b.slot_mapping, causal=b.causal, scale=b.scale)


@pytest.mark.parametrize("idx", [0, 3])
def test_value_shift(idx):
    b = small_batches()[idx]
    vn, vc = _grid_values(b, idx)
    out, _, _ = run_oracle(_with_v(b, vn, vc))
    shift = 3.0
    used = vc.view(torch.int16) != torch.tensor(0x7FC0, dtype=torch.int16)
    vc2 = vc.clone()
    vc2[used] = vc[used] + shift
    out2, _, _ = run_oracle(_with_v(b, vn + shift, vc2))
    np.testing.assert_allclose(out2, out + shift, rtol=0, atol=1e-12)


@pytest.mark.parametrize("idx", [0, 6])
def test_value_linearity(idx):
    b = small_batches()[idx]
    vn1, vc1 = _grid_values(b, 10 + idx)
    vn2, vc2 = _grid_values(b, 20 + idx)
    used = vc1.view(torch.int16) != torch.tensor(0x7FC0, dtype=torch.int16)
    vc3 = vc1.clone()
    vc3[used] = vc1[used] + 2 * vc2[used]
    o1, _, _ = run_oracle(_with_v(b, vn1, vc1))
    o2, _, _ = run_oracle(_with_v(b, vn2, vc2))
    o3, _, _ = run_oracle(_with_v(b, vn1 + 2 * vn2, vc3))
    np.testing.assert_allclose(o3, o1 + 2 * o2, rtol=0, atol=1e-11)


def test_equal_query_heads_in_group_agree():
    b = config("tiny")
    b.q[:, 1] = b.q[:, 0]  # heads 0 and 1 share kv head 0
    b.q[:, 3] = b.q[:, 0]  # head 3 reads kv head 1
    out, _, _ = run_oracle(b)
    assert np.array_equal(out[:, 0], out[:, 1])
    assert not np.allclose(out[:, 0], out[:, 3])


# --------------------------------------------------------------------------
# Scatter
# --------------------------------------------------------------------------
@pytest.mark.parametrize("idx", [0, 1, 2])
def test_scatter_exact(idx):
    b = small_batches()[idx]
    _, kc, vc = run_oracle(b)
    k0, v0 = u16(b.k_cache), u16(b.v_cache)
    S = b.page_size
    written = np.zeros(b.num_pages * S, dtype=bool)
    for t, slot in enumerate(b.slot_mapping.tolist()):
        written[slot] = True
        assert (kc[slot // S, slot % S] == u16(b.k_new)[t]).all()
        assert (vc[slot // S, slot % S] == u16(b.v_new)[t]).all()
    flat_k, flat_v = kc.reshape(-1, *kc.shape[2:]), vc.reshape(-1, *vc.shape[2:])
    assert np.array_equal(flat_k[~written], k0.reshape(flat_k.shape)[~written])
    assert np.array_equal(flat_v[~written], v0.reshape(flat_v.shape)[~written])
    assert written.sum() == b.total_tokens


# --------------------------------------------------------------------------
# Preconditions
# --------------------------------------------------------------------------
def _check(b: Batch, **over):
    args = dict(page_table=b.page_table.numpy(), cu_q_lens=b.cu_q_lens.numpy(),
                context_lens=b.context_lens.numpy(), slot_mapping=b.slot_mapping.numpy())
    args.update(over)
    return oracle.check(**args, num_q_heads=b.num_q_heads, num_kv_heads=b.num_kv_heads,
                        head_dim=b.head_dim, page_size=b.page_size, num_pages=b.num_pages)


def test_check_accepts_valid_batches():
    for b in small_batches():
        assert _check(b) == oracle.OK


def test_check_rejects_each_rule():
    b = config("tiny")
    cu = b.cu_q_lens.numpy().copy()
    cu[0] = 1
    assert _check(b, cu_q_lens=cu) == oracle.BAD_CU_Q_LENS
    cu = b.cu_q_lens.numpy().copy()
    cu[2], cu[1] = cu[1], cu[2] + 1
    assert _check(b, cu_q_lens=cu) == oracle.BAD_CU_Q_LENS
    ctx = b.context_lens.numpy().copy()
    ctx[1] = -1
    assert _check(b, context_lens=ctx) == oracle.BAD_CONTEXT
    ctx = b.context_lens.numpy().copy()
    ctx[0] = 10_000
    assert _check(b, context_lens=ctx) == oracle.TOO_LONG
    pt = b.page_table.numpy().copy()
    pt[2, 0] = b.num_pages
    assert _check(b, page_table=pt) == oracle.BAD_PAGE
    pt[2, 0] = -3
    assert _check(b, page_table=pt) == oracle.BAD_PAGE
    sm = b.slot_mapping.numpy().copy()
    sm[5] += 1
    assert _check(b, slot_mapping=sm) == oracle.BAD_SLOT
    # two requests sharing the page that both write into
    pt = b.page_table.numpy().copy()
    pt[1, 100 // 16] = pt[0, 37 // 16]
    ctx = b.context_lens.numpy().copy()
    ctx[1] = 37  # request 1 now writes position 37 of the same page as request 0
    sm = b.slot_mapping.numpy().copy()
    sm[1] = sm[0]
    pt[1, 37 // 16] = pt[0, 37 // 16]
    assert _check(b, page_table=pt, context_lens=ctx, slot_mapping=sm) == oracle.DUP_SLOT
    assert oracle.check(b.page_table.numpy(), b.cu_q_lens.numpy(), b.context_lens.numpy(),
                        b.slot_mapping.numpy(), num_q_heads=3, num_kv_heads=2, head_dim=64,
                        page_size=16, num_pages=64) == oracle.BAD_SHAPE


# --------------------------------------------------------------------------
# Planted mistakes: each mutant of oracle.c must fail at least one pin.
# --------------------------------------------------------------------------
MUTANTS = {
    "causal_off_by_one": ("p->causal ? pos + 1 : L", "p->causal ? pos : L"),
    "gqa_modulo_map": ("const int hk = h / G;", "const int hk = h % p->Hkv;"),
    "dropped_scale": ("scores[j] = p->scale * dot;", "scores[j] = dot;"),
    "top_left_alignment": ("const long long pos = c + (t - p->cu_q_lens[r]);",
                           "const long long pos = (t - p->cu_q_lens[r]);"),
    "in_page_index_lost": ("return page * p->S + j % p->S;", "return page * p->S;"),
    "k_gets_v": ("k_cache[dst + d] = k_new[src + d];", "k_cache[dst + d] = v_new[src + d];"),
    "no_normalisation": ("out[d] /= denom;", "out[d] /= 1.0;"),
    "wrong_page_row": ("long long page = p->page_table[(long long)r * p->max_pages + j / p->S];",
                       "long long page = p->page_table[(long long)r * p->max_pages + j % p->S];"),
    "q_head_stride": ("p->q + ((long long)t * p->Hq + h) * D",
                      "p->q + ((long long)t * p->Hq + h / G) * D"),
    "rows_request_of_pair": ("attend_one(&p, req[tokens[i]], tokens[i], heads[i]",
                             "attend_one(&p, req[i % T], tokens[i], heads[i]"),
    "rows_head_of_pair": ("tokens[i], heads[i], scores", "tokens[i], heads[i] / 2, scores"),
}


def _pins_pass(lib) -> bool:
    for b in small_batches()[:4] + [_golden_batch(c) for c in golden_cases()]:
        try:
            out, kc, vc = run_oracle(b, lib=lib)
        except ValueError:
            return False
        ref = dense_numpy(b)
        if not (np.max(np.abs(out - ref), initial=0.0) < 1e-12):
            return False
        S = b.page_size
        for t, slot in enumerate(b.slot_mapping.tolist()):
            if not (kc[slot // S, slot % S] == u16(b.k_new)[t]).all():
                return False
        # the per-(token, head) entry, on every pair in reverse order
        T, Hq = b.total_tokens, b.num_q_heads
        tokens = np.repeat(np.arange(T), Hq)[::-1].astype(np.int32)
        heads = np.tile(np.arange(Hq), T)[::-1].astype(np.int32)
        rows = oracle.attention_rows(u16(b.q), kc, vc, b.page_table.numpy(), b.cu_q_lens.numpy(),
                                     b.context_lens.numpy(), tokens, heads,
                                     scale=b.effective_scale(), causal=b.causal, lib=lib)
        if not (np.max(np.abs(rows - ref[tokens, heads]), initial=0.0) < 1e-12):
            return False
    return True


def test_unmutated_oracle_passes_pins():
    assert _pins_pass(oracle.load())


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    """A mutant either fails a pin or crashes; it runs in a child process."""
    src = open(oracle._SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    path = tmp_path / f"oracle_{name}.c"
    path.write_text(src.replace(old, new))
    so = str(tmp_path / f"liboracle_{name}.so")
    oracle.build(str(path), so)
    code = ("import sys; sys.path.insert(0, %r); import oracle; "
            "from tests.test_oracle import _pins_pass; "
            "sys.exit(0 if _pins_pass(oracle.load(%r)) else 3)" % (ROOT, so))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    rc = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env,
                        capture_output=True, timeout=300).returncode
    assert rc != 0, f"mutant {name} survived every pin"
