"""Parity of nkv_qk_norm_rope_store (q/k RMSNorm + rotary + KV store, bf16) with the
oracle oracle/rope_norm.py on the same seeded inputs.

Both sides take the same rounding points (the listings' casts back to bf16 after the
normalisation, after the weight product and after the rotation, float32 in between); what
can still differ is the summation order of a head's mean square and the last bit of its
reciprocal root, which moves a normalised element across a bf16 rounding boundary now and
then.  The bar, per output element: at most one q/k element in a thousand (and
never fewer than one) differing from the oracle's bits, and every
difference within 2^-6 of the largest |normed * weight| value of its head (two bf16 units
at that scale).  v rows must be stored bit-exactly; pool rows that no slot names must stay
untouched (NaN).

Inputs: projection outputs N(0, 1) with a per-head scale drawn log-uniformly in
[1e-2, 30] (RMSNorm must take any scale), weights 1 + 0.1 N(0, 1), positions uniform in
[0, 40960) (Qwen3's maximum position), a rotary table of base 1e6 built by the oracle (a
model constant, so an input), slots a random permutation of pool rows with every 7th
token skipped (-1).
"""

import numpy as np
import pytest
import torch

from oracle import rope_norm as rn
from paged_kv_cache_258_amd import nkv_qk_norm_rope_store
from paged_kv_cache_258_amd import workloads as wl

from _gpu_helpers import dev_i32, host_bits, log, require_gpu

pytestmark = pytest.mark.gpu

MAX_POS = 40960
BASE = 1.0e6
EPS = 1e-6
_TABLES = {}


def table(d):
    if d not in _TABLES:
        _TABLES[d] = rn.rope_cos_sin_table(MAX_POS, d, BASE)
    return _TABLES[d]


def make_case(seed, t, hq, hkv, d, nb=None, bs=16, extra_cols=0):
    dev = require_gpu()
    rng = np.random.default_rng(seed)
    gen = torch.Generator(device=dev).manual_seed(seed)
    width = (hq + 2 * hkv) * d
    qkv_full = wl.randn((t, width + extra_cols), gen, dev, "bf16")
    scales = np.exp(rng.uniform(np.log(1e-2), np.log(30.0), size=(1, hq + 2 * hkv, 1))).astype(np.float32)
    sc = torch.as_tensor(scales, device=dev)
    body = (qkv_full[:, :width].contiguous().float().view(t, hq + 2 * hkv, d) * sc).to(torch.bfloat16)
    qkv_full[:, :width] = body.view(t, width)
    qkv = qkv_full[:, :width]                       # rows strided when extra_cols > 0
    wq = (1.0 + 0.1 * wl.randn((d,), gen, dev, "f32")).to(torch.bfloat16)
    wk = (1.0 + 0.1 * wl.randn((d,), gen, dev, "f32")).to(torch.bfloat16)
    pos = rng.integers(0, MAX_POS, size=t).astype(np.int32)
    if nb is None:
        nb = max(2, -(-2 * t // bs))
    slots = rng.permutation(nb * bs)[:t].astype(np.int32)
    slots[::7] = -1
    kc = wl.nan_pool(nb, bs, hkv, d, "bf16", dev)
    vc = wl.nan_pool(nb, bs, hkv, d, "bf16", dev)
    return dict(qkv=qkv, wq=wq, wk=wk, pos=pos, slots=slots, kc=kc, vc=vc, hq=hq, hkv=hkv, d=d, t=t)


def run_and_check(c, what):
    dev = c["qkv"].device
    log(f"[rope_store] {what}: T={c['t']} Hq={c['hq']} Hkv={c['hkv']} D={c['d']} "
        f"row_stride={c['qkv'].stride(0)}")
    tab = table(c["d"])
    kc0, vc0 = host_bits(c["kc"]), host_bits(c["vc"])
    q_out = nkv_qk_norm_rope_store(c["qkv"], dev_i32(c["pos"], dev), c["wq"], c["wk"],
                                   torch.as_tensor(tab, device=dev), dev_i32(c["slots"], dev),
                                   c["kc"], c["vc"], c["hq"], EPS)
    torch.cuda.synchronize()
    qkv_bits = host_bits(c["qkv"].contiguous())
    want_q, want_k, want_v = rn.qk_norm_rope_store_ref(qkv_bits, c["pos"], host_bits(c["wq"]),
                                                        host_bits(c["wk"]), tab, c["slots"], kc0,
                                                        vc0, c["hq"], c["hkv"], EPS)
    got_q, got_k, got_v = host_bits(q_out), host_bits(c["kc"]), host_bits(c["vc"])
    assert np.array_equal(got_v, want_v), "v rows or untouched pool rows differ"
    # scale of each head: the largest |normed * weight| value (before the rotation)
    x = rn.bf16_bits_to_f32(qkv_bits.reshape(c["t"], c["hq"] + 2 * c["hkv"], c["d"]))
    yq = rn.rms_norm_ref(x[:, :c["hq"]], rn.bf16_bits_to_f32(host_bits(c["wq"])), EPS)
    yk = rn.rms_norm_ref(x[:, c["hq"]:c["hq"] + c["hkv"]], rn.bf16_bits_to_f32(host_bits(c["wk"])), EPS)
    sq = np.abs(yq).max(axis=-1, keepdims=True)
    sk = np.abs(yk).max(axis=-1, keepdims=True)
    compare(got_q, want_q, sq, f"{what} q")
    # k rows: compare the stored rows of the tokens that have a slot
    rows_got = got_k.reshape(-1, c["hkv"], c["d"])
    rows_want = want_k.reshape(-1, c["hkv"], c["d"])
    keep = c["slots"] >= 0
    sl = c["slots"][keep]
    compare(rows_got[sl], rows_want[sl], sk[keep], f"{what} k")
    untouched = np.setdiff1d(np.arange(rows_got.shape[0]), sl)
    assert np.array_equal(rows_got[untouched], rows_want[untouched]), "untouched k rows changed"


def compare(got_bits, want_bits, scale, what):
    if got_bits.size == 0:
        return
    g, w = rn.bf16_bits_to_f32(got_bits), rn.bf16_bits_to_f32(want_bits)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    same = float(np.mean(got_bits == want_bits))
    err = np.abs(g.astype(np.float64) - w.astype(np.float64))
    bound = (2.0 ** -6) * np.broadcast_to(scale, err.shape)
    worst = float((err / np.maximum(bound, 1e-30)).max())
    log(f"  {what}: bit-identical {same:.5f}, worst error / bound {worst:.3f}")
    flips = int(np.count_nonzero(got_bits != want_bits))
    # at most one element in a thousand (and never fewer than one) may differ
    assert flips <= max(1, got_bits.size // 1000), f"{what}: {flips} of {got_bits.size} elements differ"
    assert np.all(err <= bound), f"{what}: error beyond two bf16 units of the head scale"


@pytest.mark.parametrize("t,hq,hkv,d", [(300, 32, 8, 128), (37, 4, 1, 64), (1, 2, 2, 128),
                                        (129, 16, 2, 128), (64, 8, 8, 64)])
def test_rope_store_matches_oracle(t, hq, hkv, d):
    run_and_check(make_case(900 + t + hq + d, t, hq, hkv, d), "shapes")


def test_rope_store_strided_qkv_rows():
    run_and_check(make_case(950, 200, 32, 8, 128, extra_cols=64), "strided rows")


def test_rope_store_prefill_sized_batch():
    # 16384 tokens: the 8 x 2048-token prefill's projection output, block_size 256
    run_and_check(make_case(960, 16384, 32, 8, 128, nb=160, bs=256), "16384 tokens")


def test_rope_store_zero_heads_and_position_zero():
    # an all-zero head normalises to zero (eps keeps it finite); position 0 leaves the
    # normalised head unrotated
    c = make_case(970, 50, 8, 2, 128)
    c["qkv"][:5] = 0
    c["pos"][5:10] = 0
    run_and_check(c, "zero heads, position 0")
    dev = c["qkv"].device
    q_out = nkv_qk_norm_rope_store(c["qkv"], dev_i32(c["pos"], dev), c["wq"], c["wk"],
                                   torch.as_tensor(table(128), device=dev), dev_i32(c["slots"], dev),
                                   c["kc"], c["vc"], 8, EPS)
    torch.cuda.synchronize()
    assert bool((q_out[:5] == 0).all())
