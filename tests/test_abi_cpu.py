"""The C ABI without a GPU: the library loads, exports every symbol its header
declares, and its host-side checks (shape, metadata, workspace) behave."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
import torch

import oracle
from ragged_paged_attention_amd import binding
from ragged_paged_attention_amd.inputs import build_batch, config, random_batch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ragged_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("ra_forward", "ra_forward_variant", "ra_forward_profiled", "ra_workspace_bytes",
                 "ra_validate_metadata", "ra_status_str", "ra_last_error"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(\w+)", out))
    for name in declared_functions():
        assert name in exported, f"{name} declared in ragged_attn.h but not exported"
        assert hasattr(lib, name)


def test_status_strings(lib):
    for code in range(7):
        s = lib.ra_status_str(code).decode()
        assert s.startswith(binding.STATUS[code])


def shape_for(b, **over):
    kw = dict(num_reqs=b.num_reqs, total_tokens=b.total_tokens, num_q_heads=b.num_q_heads,
              num_kv_heads=b.num_kv_heads, head_dim=b.head_dim, page_size=b.page_size,
              num_pages=b.num_pages, max_pages_per_req=b.page_table.shape[1], causal=b.causal)
    kw.update(over)
    return binding.make_shape(**kw)


def validate(b, shape=None, **over):
    args = dict(page_table=b.page_table, cu_q_lens=b.cu_q_lens, context_lens=b.context_lens,
                slot_mapping=b.slot_mapping)
    args.update(over)
    try:
        binding.validate_metadata(shape or shape_for(b), **args)
        return "RA_OK"
    except binding.RaError as e:
        return e.name


def test_validate_accepts_generated_batches():
    for b in [config("tiny")] + [random_batch(s, num_reqs=6, max_q=30, max_ctx=90, num_q_heads=8,
                                              num_kv_heads=2, head_dim=64) for s in range(5)]:
        assert validate(b) == "RA_OK"


def test_validate_rejects_like_the_oracle():
    """Each broken rule is rejected by the library and by the oracle's checker."""
    b = config("tiny")
    cases = []
    cu = b.cu_q_lens.clone(); cu[0] = 1; cases.append(dict(cu_q_lens=cu))
    ctx = b.context_lens.clone(); ctx[1] = -1; cases.append(dict(context_lens=ctx))
    ctx = b.context_lens.clone(); ctx[0] = 5000; cases.append(dict(context_lens=ctx))
    pt = b.page_table.clone(); pt[2, 0] = b.num_pages; cases.append(dict(page_table=pt))
    pt = b.page_table.clone(); pt[3, 1] = -1; cases.append(dict(page_table=pt))
    sm = b.slot_mapping.clone(); sm[4] += 1; cases.append(dict(slot_mapping=sm))
    for over in cases:
        got = validate(b, **over)
        assert got == "RA_E_METADATA", over
        args = dict(page_table=b.page_table, cu_q_lens=b.cu_q_lens, context_lens=b.context_lens,
                    slot_mapping=b.slot_mapping)
        args.update(over)
        rc = oracle.check(*(args[k].numpy() for k in ("page_table", "cu_q_lens", "context_lens",
                                                      "slot_mapping")),
                          num_q_heads=b.num_q_heads, num_kv_heads=b.num_kv_heads,
                          head_dim=b.head_dim, page_size=b.page_size, num_pages=b.num_pages)
        assert rc != oracle.OK


def test_validate_rejects_duplicate_slot():
    # two decode requests whose new tokens land in the same slot
    b = random_batch(3, num_reqs=2, max_q=1, max_ctx=20, num_q_heads=2, num_kv_heads=1,
                     head_dim=64, decode_frac=1.0)
    pt = b.page_table.clone()
    ctx = b.context_lens.clone()
    ctx[1] = ctx[0]
    pt[1] = pt[0]
    sm = b.slot_mapping.clone()
    sm[1] = sm[0]
    assert validate(b, page_table=pt, context_lens=ctx, slot_mapping=sm) == "RA_E_METADATA"
    assert "twice" in binding.last_error()


def test_shape_errors(lib):
    b = config("tiny")
    assert validate(b, shape=shape_for(b, num_q_heads=3)) == "RA_E_SHAPE"
    assert validate(b, shape=shape_for(b, total_tokens=54)) == "RA_E_METADATA"
    assert lib.ra_workspace_bytes(None, None, None) == 0


def _forward_status(lib, shape, cu, ctx, ws_bytes=1 << 30, ptr=0x1000, ws_ptr=0x100000,
                    variant=0):
    """Call ra_forward_variant with fake device pointers (only host checks run)."""
    P = ctypes.c_void_p
    fake = P(ptr)
    return lib.ra_forward_variant(ctypes.byref(shape), fake, fake, fake, fake, fake, fake, fake,
                                  fake, fake, cu.data_ptr() and P(cu.data_ptr()),
                                  P(ctx.data_ptr()), fake, P(ws_ptr), ctypes.c_size_t(ws_bytes),
                                  None, variant)


def test_forward_rejects_before_touching_the_gpu(lib):
    b = config("tiny")
    cu, ctx = b.cu_q_lens.clone(), b.context_lens.clone()
    assert _forward_status(lib, shape_for(b, head_dim=96), cu, ctx) == 3  # unsupported
    assert _forward_status(lib, shape_for(b, page_size=24), cu, ctx) == 3  # not a multiple of 16
    assert _forward_status(lib, shape_for(b, page_size=2048), cu, ctx) == 3  # page above 1024
    assert _forward_status(lib, shape_for(b, num_kv_heads=3), cu, ctx) == 2
    assert _forward_status(lib, shape_for(b), cu, ctx, ws_bytes=16) == 5  # workspace too small
    assert _forward_status(lib, shape_for(b), cu, ctx, ws_ptr=0x100010) == 5  # misaligned
    assert _forward_status(lib, shape_for(b), cu, ctx, variant=7) == 2
    bad = cu.clone(); bad[2] = 0
    assert _forward_status(lib, shape_for(b), bad, ctx) == 4
    assert _forward_status(lib, shape_for(b, scale=-1.0), cu, ctx) == 2
    assert _forward_status(lib, shape_for(b, scale=float("inf")), cu, ctx) == 2
    huge = ctx.clone(); huge[0] = 1 << 30  # key positions are 32-bit inside the kernels
    assert _forward_status(lib, shape_for(b, max_pages_per_req=1 << 27), cu, huge) == 3


@pytest.mark.parametrize("hq,hkv", [(32, 1), (64, 2), (300, 1), (48, 3)])
def test_any_group_size_is_accepted(lib, hq, hkv):
    """Any G = Hq / Hkv >= 1 passes the host checks and gets a workspace
    (decode heads go in blocks of 16, prefill rows up to G = 256, the
    generic kernel beyond that)."""
    b = random_batch(9, num_reqs=5, max_q=40, max_ctx=200, num_q_heads=hq, num_kv_heads=hkv,
                     head_dim=64, decode_frac=0.5)
    assert validate(b) == "RA_OK"
    assert binding.workspace_bytes(shape_for(b), b.cu_q_lens, b.context_lens) > 0


def test_workspace_bound_covers_every_batch_of_the_same_size(lib, monkeypatch):
    """Planning on the device sizes the workspace from R and T alone (host
    copies NULL): that bound is at least the workspace the same kernels need
    for any batch with R requests and T new tokens, whatever its
    decode/prefill mix (planning on the device sends short chunks to the
    prefill kernel, as RA_SHORT_CHUNKS=0 does for host planning)."""
    monkeypatch.setenv("RA_SHORT_CHUNKS", "0")
    rng = np.random.default_rng(12)
    for Hq, Hkv, D in ((32, 8, 128), (16, 8, 256), (8, 1, 64), (64, 2, 128)):
        R, T = 9, 300
        for _ in range(20):
            cuts = np.sort(rng.integers(0, T + 1, R - 1))
            q = np.diff(np.concatenate([[0], cuts, [T]])).tolist()
            c = rng.integers(0, 5000, R).tolist()
            b = build_batch(q, c, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, seed=1)
            shape = shape_for(b)
            exact = binding.workspace_bytes(shape, b.cu_q_lens, b.context_lens)
            bound = binding.workspace_bytes(shape, None, None)
            assert bound >= exact > 0
    shape = shape_for(b)
    cu = b.cu_q_lens.clone()
    # one host copy without the other is refused
    assert lib.ra_workspace_bytes(ctypes.byref(shape), ctypes.c_void_p(cu.data_ptr()), None) == 0


def test_empty_batch_is_a_no_op(lib):
    shape = binding.make_shape(num_reqs=0, total_tokens=0, num_q_heads=8, num_kv_heads=2,
                               head_dim=128, page_size=16, num_pages=0, max_pages_per_req=0)
    cu = torch.zeros(1, dtype=torch.int32)
    ctx = torch.zeros(0, dtype=torch.int32)
    st = lib.ra_forward_variant(ctypes.byref(shape), *([None] * 9), ctypes.c_void_p(cu.data_ptr()),
                                ctypes.c_void_p(ctx.data_ptr() or 8), None, None,
                                ctypes.c_size_t(0), None, 0)
    assert st == 0, binding.last_error()


def test_decode_workspace_does_not_grow_with_context(lib):
    """Decode partials live in fixed per-workgroup slots: the workspace depends on
    the number of requests, not on how long their contexts are."""
    short = random_batch(5, num_reqs=4, max_q=1, max_ctx=100, num_q_heads=32, num_kv_heads=8,
                         head_dim=128, decode_frac=1.0)
    n_short = binding.workspace_bytes(shape_for(short), short.cu_q_lens, short.context_lens)
    long_ = random_batch(5, num_reqs=4, max_q=1, max_ctx=50000, num_q_heads=32, num_kv_heads=8,
                         head_dim=128, decode_frac=1.0)
    n_long = binding.workspace_bytes(shape_for(long_), long_.cu_q_lens, long_.context_lens)
    assert n_short > 0 and n_long == n_short
    assert n_short % 256 == 0
    # bounded by the partial slots (2 per workgroup, at most 512 workgroups)
    # plus the small per-request tables
    assert n_short <= 2 * 512 * 32 * (128 + 2) * 4 + 64 * 1024


def test_profiled_call_checks_its_events(lib):
    """ra_forward_profiled takes a start and a stop event per stage (eight);
    a wrong count or a NULL entry is refused before anything else runs."""
    b = config("tiny")
    cu, ctx = b.cu_q_lens.clone(), b.context_lens.clone()
    P = ctypes.c_void_p
    fake = P(0x1000)

    def call(events, n):
        return lib.ra_forward_profiled(ctypes.byref(shape_for(b)), fake, fake, fake, fake, fake, fake, fake,
                                       fake, fake, P(cu.data_ptr()), P(ctx.data_ptr()), fake, P(0x100000),
                                       ctypes.c_size_t(1 << 30), None, 0, events, n)

    assert binding.StageTimer.N_EVENTS == 8
    five = (ctypes.c_void_p * 5)(*([0x2000] * 5))
    assert call(five, 5) == 2  # RA_E_SHAPE: n_events must be 8
    eight = (ctypes.c_void_p * 8)(*([0x2000] * 7 + [None]))
    assert call(eight, 8) == 1  # RA_E_NULL: an event is NULL
