"""ra_forward_noalloc (the entry point that allocates nothing; its workspace is
the library's static scratch array) against ra_forward, through the C ABI.

Two calls in a row on one device, the second with a smaller batch, so the
second reads a scratch array that still holds the first call's work lists
and partials.  Mixed batches run sequentially in ra_forward_noalloc, so the
ra_forward reference runs with RA_MIXED_OVERLAP=0 (the same plan): outputs and
caches must then be bitwise equal, and both within the oracle's bound.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from ragged_paged_attention_amd import binding
from ragged_paged_attention_amd.inputs import build_batch, u16
from tests.test_gpu_parity import assert_close, oracle_full, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()
    yield


def _run(b, fn):
    dev = torch.device("cuda:0")
    kc, vc = b.k_cache.to(dev), b.v_cache.to(dev)
    out = fn(b.q.to(dev), b.k_new.to(dev), b.v_new.to(dev), kc, vc, b.page_table.to(dev),
             b.cu_q_lens.to(dev), b.context_lens.to(dev), b.slot_mapping.to(dev), causal=b.causal,
             cu_q_lens_host=b.cu_q_lens, context_lens_host=b.context_lens)
    torch.cuda.synchronize()
    return out.cpu(), kc.cpu(), vc.cpu()


def test_noalloc_matches_forward_on_two_calls(monkeypatch):
    monkeypatch.setenv("RA_MIXED_OVERLAP", "0")
    big = build_batch([1] * 90 + [300, 77, 512], [(211 * i) % 6000 for i in range(90)] + [0, 900, 2000],
                      num_q_heads=32, num_kv_heads=8, head_dim=128, seed=501, name="noalloc_big")
    small = build_batch([1, 1, 40, 1, 9], [3000, 17, 100, 1200, 0], num_q_heads=32, num_kv_heads=8,
                        head_dim=128, seed=502, name="noalloc_small")
    results = []
    for b in (big, small):
        say(f"[noalloc] {b.name}: R={b.num_reqs} T={b.total_tokens}")
        results.append((b, _run(b, binding.forward_noalloc)))
    for b, (out_na, kc_na, vc_na) in results:
        out, kc, vc = _run(b, binding.forward)
        assert torch.equal(out_na.view(torch.int16), out.view(torch.int16)), f"{b.name}: outputs differ"
        assert torch.equal(kc_na.view(torch.int16), kc.view(torch.int16)), f"{b.name}: k caches differ"
        assert torch.equal(vc_na.view(torch.int16), vc.view(torch.int16)), f"{b.name}: v caches differ"
        ref, rkc, rvc = oracle_full(b)
        assert np.array_equal(u16(kc_na), rkc) and np.array_equal(u16(vc_na), rvc)
        worst = assert_close(out_na, ref, b.name)
        say(f"[noalloc] {b.name}: bitwise equal to ra_forward, max abs error {worst:.3g}")


def test_noalloc_refuses_a_batch_beyond_the_scratch():
    """A batch whose workspace exceeds the 64 MiB scratch is refused before
    anything runs (G = 64 at head_dim 256 needs about 258 MiB of decode partials)."""
    b = build_batch([1, 1], [10, 20], num_q_heads=512, num_kv_heads=8, head_dim=256, seed=503)
    dev = torch.device("cuda:0")
    sentinel = torch.full(b.q.shape, 3.0, dtype=torch.bfloat16, device=dev)
    with pytest.raises(binding.RaError) as e:
        binding.forward_noalloc(b.q.to(dev), b.k_new.to(dev), b.v_new.to(dev), b.k_cache.to(dev),
                                b.v_cache.to(dev), b.page_table.to(dev), b.cu_q_lens.to(dev),
                                b.context_lens.to(dev), b.slot_mapping.to(dev), out=sentinel,
                                cu_q_lens_host=b.cu_q_lens, context_lens_host=b.context_lens)
    assert e.value.name == "RA_E_WORKSPACE"
    torch.cuda.synchronize()
    assert bool((sentinel == 3.0).all())


def test_noalloc_short_chunks_beyond_the_slot_limit():
    """Short chunks at Llama-3-8B shapes would widen the decode partial slots
    past the 64 MiB scratch; the call then runs them in the prefill kernel and
    still matches the oracle."""
    b = build_batch([4, 1, 3, 2] * 8, [(97 * i) % 3000 for i in range(32)], num_q_heads=32,
                    num_kv_heads=8, head_dim=128, seed=504, name="noalloc_short")
    out, kc, vc = _run(b, binding.forward_noalloc)
    ref, rkc, rvc = oracle_full(b)
    assert np.array_equal(u16(kc), rkc) and np.array_equal(u16(vc), rvc)
    assert_close(out, ref, b.name)
