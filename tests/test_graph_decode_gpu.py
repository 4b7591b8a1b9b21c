"""Decode steps captured once in a HIP graph and replayed (the capture/replay of the decode
step that 「同一个 Qwen3，两种写法」 §3 mentions for nano-vLLM).

The library's store and decode calls allocate nothing, set no memory with memset, and
never synchronise, so they can be captured as they are; the decode work split is
computed on the device from context_lens, so a graph stays valid while the lengths grow.
The test captures one step (store of the new token, then decode) on static buffers, and
for several steps writes new q/k/v, slots and lengths eagerly, synchronises, replays the
graph, and runs the same two calls eagerly on a second copy of the pools.  Every replay
must give the eager result bit for bit (the kernels are deterministic), the pools must
match, and the last step is checked against the oracle on sampled sequences.
"""

import numpy as np
import pytest
import torch

from oracle import ref
from paged_kv_cache_258_amd import nkv_paged_attn_decode, nkv_paged_attn_decode_workspace_size, nkv_store_kvcache
from paged_kv_cache_258_amd import workloads as wl

from _gpu_helpers import assert_close, dev_i32, host_bits, log, require_gpu, to_f64

pytestmark = pytest.mark.gpu

STEPS = 4


def test_decode_step_graph_replays_match_eager():
    dev = require_gpu()
    sh = wl.QWEN3_8B
    bs, hq, hkv, d = sh.block_size, sh.num_q_heads, sh.num_kv_heads, sh.head_dim
    rng = np.random.default_rng(1300)
    gen = torch.Generator(device=dev).manual_seed(1300)
    b = 24
    lens0 = rng.integers(200, 3000, size=b).astype(np.int32)     # includes the first new token
    nblk = [wl.blocks_needed(int(l) + STEPS, bs) for l in lens0]
    nb = sum(nblk) + 1
    maxb = max(nblk)
    table = wl.assign_blocks(rng, nblk, nb, maxb)
    kc_g = wl.nan_pool(nb, bs, hkv, d, "bf16", dev)
    vc_g = wl.nan_pool(nb, bs, hkv, d, "bf16", dev)
    hist = np.concatenate([wl.slots_for_positions(table[i], np.arange(lens0[i] - 1), bs) for i in range(b)])
    wl._fill_cached(kc_g, gen, hist)
    wl._fill_cached(vc_g, gen, hist)
    kc_e, vc_e = kc_g.clone(), vc_g.clone()
    log(f"[graph decode] B={b} lens {int(lens0.min())}..{int(lens0.max())} steps={STEPS}")

    # static buffers the graph reads and writes
    q = torch.empty((b, hq, d), dtype=torch.bfloat16, device=dev)
    k = torch.empty((b, hkv, d), dtype=torch.bfloat16, device=dev)
    v = torch.empty((b, hkv, d), dtype=torch.bfloat16, device=dev)
    slots = torch.empty(b, dtype=torch.int32, device=dev)
    ctx = torch.empty(b, dtype=torch.int32, device=dev)
    table_d = dev_i32(table, dev)
    out_g = torch.empty((b, hq, d), dtype=torch.bfloat16, device=dev)
    out_e = torch.empty_like(out_g)
    ws = torch.empty(nkv_paged_attn_decode_workspace_size(b, hq, hkv, d, maxb, bs), dtype=torch.uint8,
                     device=dev)

    def set_step(s):
        lens = lens0 + s
        q.copy_(wl.randn((b, hq, d), gen, dev, "bf16"))
        k.copy_(wl.randn((b, hkv, d), gen, dev, "bf16"))
        v.copy_(wl.randn((b, hkv, d), gen, dev, "bf16"))
        sl = np.array([wl.slots_for_positions(table[i], [lens[i] - 1], bs)[0] for i in range(b)], np.int32)
        slots.copy_(dev_i32(sl, dev))
        ctx.copy_(dev_i32(lens, dev))
        torch.cuda.synchronize()
        return lens

    def step(kc, vc, out):
        nkv_store_kvcache(k, v, kc, vc, slots)
        nkv_paged_attn_decode(q, kc, vc, ctx, table_d, sh.scale, out=out, workspace=ws)

    # warm up on a side stream, then capture on it (torch's recipe)
    set_step(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(kc_e.clone(), vc_e.clone(), torch.empty_like(out_g))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(kc_g, vc_g, out_g)
    torch.cuda.synchronize()

    for s in range(STEPS):
        lens = set_step(s)
        graph.replay()
        torch.cuda.synchronize()
        step(kc_e, vc_e, out_e)                 # eager, same inputs, its own pools
        torch.cuda.synchronize()
        same = torch.equal(out_g.view(torch.int16), out_e.view(torch.int16))
        log(f"  step {s}: replay == eager: {same}")
        assert same, f"step {s}: graph replay differs from the eager call"
    assert torch.equal(kc_g.view(torch.int16), kc_e.view(torch.int16))
    assert torch.equal(vc_g.view(torch.int16), vc_e.view(torch.int16))

    seqs = [0, 5, b - 1]
    want = ref.decode_ref(host_bits(q), host_bits(kc_g), host_bits(vc_g), lens, table, sh.scale,
                          elem="bf16", seqs=seqs)
    got = to_f64(out_g)
    assert_close(got[seqs], want[seqs], "last replay vs oracle")
