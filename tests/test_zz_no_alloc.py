"""The allocation-free decode (nkv_paged_attn_decode_noalloc) against the decode with a
workspace (nkv_paged_attn_decode) and against the oracle.

Both entry points share the plan and the kernels; the only difference is where the
partial results of split sequences live (the library's static device scratch instead of
the caller's workspace), so the outputs must agree bit for bit.  Two calls in a row, the
second with fewer and shorter sequences, check that the scratch keeps no state that a
later call depends on.
"""

import numpy as np
import pytest
import torch

from oracle import ref
from paged_kv_cache_258_amd import (nkv_paged_attn_decode, nkv_paged_attn_decode_noalloc,
                                    nkv_store_kvcache)
from paged_kv_cache_258_amd import workloads as wl

from _gpu_helpers import assert_close, dev_i32, elem, host_bits, log, require_gpu, to_f64

pytestmark = pytest.mark.gpu


def make_case(seed, lens, shape):
    """Pool with NaN everywhere except the cached history; one new token per sequence,
    stored before the decode (oracle and GPU alike)."""
    dev = require_gpu()
    rng = np.random.default_rng(seed)
    gen = torch.Generator(device=dev).manual_seed(seed)
    bs = shape.block_size
    lens = np.asarray(lens, dtype=np.int32)
    nblk = [wl.blocks_needed(int(l), bs) for l in lens]
    nb = sum(nblk) + 2
    table = wl.assign_blocks(rng, nblk, nb, max(nblk) + 1)
    kc = wl.nan_pool(nb, bs, shape.num_kv_heads, shape.head_dim, shape.dtype, dev)
    vc = wl.nan_pool(nb, bs, shape.num_kv_heads, shape.head_dim, shape.dtype, dev)
    hist = np.concatenate([wl.slots_for_positions(table[b], np.arange(l - 1), bs)
                           for b, l in enumerate(lens)] + [np.zeros(0, np.int32)])
    if len(hist):
        wl._fill_cached(kc, gen, hist)
        wl._fill_cached(vc, gen, hist)
    b = len(lens)
    q = wl.randn((b, shape.num_q_heads, shape.head_dim), gen, dev, shape.dtype)
    k = wl.randn((b, shape.num_kv_heads, shape.head_dim), gen, dev, shape.dtype)
    v = wl.randn((b, shape.num_kv_heads, shape.head_dim), gen, dev, shape.dtype)
    slots = np.array([wl.slots_for_positions(table[i], [lens[i] - 1], bs)[0] for i in range(b)],
                     dtype=np.int32)
    want_k, want_v = ref.store_ref(host_bits(k), host_bits(v), host_bits(kc), host_bits(vc), slots)
    nkv_store_kvcache(k, v, kc, vc, dev_i32(slots, dev))
    want = ref.decode_ref(host_bits(q), want_k, want_v, lens, table, shape.scale, elem=elem(q))
    return q, kc, vc, dev_i32(lens, dev), dev_i32(table, dev), want


@pytest.mark.parametrize("shape", [wl.QWEN3_8B, wl.Shape(16, 4, 64, 16, "bf16"),
                                   wl.Shape(32, 8, 128, 256, "f32")],
                         ids=["qwen3-8b-bf16", "small-bf16", "qwen3-8b-f32"])
def test_noalloc_decode_matches_workspace_decode(shape):
    big = make_case(1300, [4096, 1, 3001, 17, 40960, 512, 2048, 777, 65, 1500], shape)
    small = make_case(1301, [300, 5, 1025], shape)
    for tag, (q, kc, vc, lens, table, want) in (("first call", big), ("second, smaller call", small)):
        log(f"[decode noalloc] {tag}: B={q.shape[0]} shape={shape}")
        ref_out = nkv_paged_attn_decode(q, kc, vc, lens, table, shape.scale)
        out = torch.full_like(q, float("nan"))
        nkv_paged_attn_decode_noalloc(q, kc, vc, lens, table, shape.scale, out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out.view(torch.int32),
                           ref_out.view(torch.int16) if ref_out.dtype == torch.bfloat16
                           else ref_out.view(torch.int32)), f"{tag}: differs from the workspace decode"
        assert_close(to_f64(out), want, f"noalloc {tag}")
