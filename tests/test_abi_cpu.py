"""CPU checks of the C ABI: the library loads, exports what include/nkv.h declares, and
rejects bad host-checkable arguments before launching anything (no GPU needed: every
call here returns before a kernel would be enqueued)."""

import ctypes
import os
import re

import pytest

from paged_kv_cache_258_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nkv.h")

FAKE = 0x10000          # aligned, never dereferenced: these calls fail validation first
MISALIGNED = 0x10008


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nkv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = header_functions()
    for n in ("nkv_store_kvcache", "nkv_paged_attn_prefill", "nkv_paged_attn_decode"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    names = header_functions()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    nm = os.popen(f"nm -D --defined-only {_lib.LIB_PATH}").read()
    exported = set(re.findall(r"\bT (nkv_[a-z0-9_]+)", nm))
    assert exported == set(names), exported ^ set(names)


def test_version_and_status_strings(lib):
    assert lib.nkv_abi_version() == 1
    assert lib.nkv_status_string(0) == b"NKV_OK"
    assert lib.nkv_status_string(3) == b"NKV_ERR_WORKSPACE"
    assert lib.nkv_status_string(99) == b"NKV_UNKNOWN_STATUS"


def store(lib, **kw):
    a = dict(key=FAKE, ks=1024, value=FAKE, vs=1024, kc=FAKE, vc=FAKE, slots=FAKE, n=4,
             hkv=8, d=128, nb=4, bs=256, dtype=1, stream=None)
    a.update(kw)
    return lib.nkv_store_kvcache(a["key"], a["ks"], a["value"], a["vs"], a["kc"], a["vc"],
                                 a["slots"], a["n"], a["hkv"], a["d"], a["nb"], a["bs"],
                                 a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(ks=1000), _lib.NKV_ERR_INVALID_ARG),         # stride below Hkv*D
    (dict(vs=1028), _lib.NKV_ERR_INVALID_ARG),         # stride not 16-byte multiple
    (dict(key=None), _lib.NKV_ERR_INVALID_ARG),
    (dict(slots=None), _lib.NKV_ERR_INVALID_ARG),
    (dict(kc=MISALIGNED), _lib.NKV_ERR_INVALID_ARG),
    (dict(dtype=7), _lib.NKV_ERR_INVALID_ARG),
    (dict(n=-1), _lib.NKV_ERR_INVALID_ARG),
    (dict(hkv=1, d=2, ks=2, vs=2), _lib.NKV_ERR_UNSUPPORTED),   # 4-byte rows
    (dict(nb=1 << 24, bs=1 << 10), _lib.NKV_ERR_UNSUPPORTED),  # > 2^31 rows
])
def test_store_rejects(lib, kw, status):
    assert store(lib, **kw) == status
    assert lib.nkv_last_error() != b""


def test_store_zero_tokens_is_noop(lib):
    assert store(lib, n=0, key=None, value=None, kc=None, vc=None, slots=None) == _lib.NKV_OK


def decode(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, lens=FAKE, table=FAKE, maxb=16, b=64, hq=32, hkv=8,
             d=128, nb=600, bs=256, scale=0.088, dtype=1, out=FAKE, ws=FAKE, wsb=1 << 40,
             stream=None)
    a.update(kw)
    return lib.nkv_paged_attn_decode(a["q"], a["kc"], a["vc"], a["lens"], a["table"], a["maxb"],
                                     a["b"], a["hq"], a["hkv"], a["d"], a["nb"], a["bs"],
                                     a["scale"], a["dtype"], a["out"], a["ws"], a["wsb"],
                                     a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(hq=30), _lib.NKV_ERR_INVALID_ARG),           # Hq % Hkv != 0
    (dict(hq=24), _lib.NKV_ERR_UNSUPPORTED),           # group of 3
    (dict(d=96), _lib.NKV_ERR_UNSUPPORTED),
    (dict(bs=48), _lib.NKV_ERR_UNSUPPORTED),
    (dict(bs=8), _lib.NKV_ERR_UNSUPPORTED),
    (dict(dtype=2), _lib.NKV_ERR_INVALID_ARG),
    (dict(q=None), _lib.NKV_ERR_INVALID_ARG),
    (dict(table=None), _lib.NKV_ERR_INVALID_ARG),
    (dict(out=MISALIGNED), _lib.NKV_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _lib.NKV_ERR_INVALID_ARG),
    (dict(maxb=0), _lib.NKV_ERR_INVALID_ARG),
    (dict(b=-2), _lib.NKV_ERR_INVALID_ARG),
    (dict(ws=None), _lib.NKV_ERR_WORKSPACE),
    (dict(wsb=16), _lib.NKV_ERR_WORKSPACE),
])
def test_decode_rejects(lib, kw, status):
    assert decode(lib, **kw) == status


def test_decode_workspace_size(lib):
    f = lib.nkv_paged_attn_decode_workspace_size
    big = f(64, 32, 8, 128, 16, 256)
    assert big > 0 and big % 16 == 0
    # at least the split-K partials of a 4096-token context: (B, Hq, splits >= 2, D+2) floats
    assert big >= 64 * 32 * 2 * (128 + 2) * 4
    assert f(0, 32, 8, 128, 16, 256) == 0
    # longer contexts never need less
    assert f(64, 32, 8, 128, 32, 256) >= big


def decode_noalloc(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, lens=FAKE, table=FAKE, maxb=16, b=64, hq=32, hkv=8,
             d=128, nb=600, bs=256, scale=0.088, dtype=1, out=FAKE, stream=None)
    a.update(kw)
    return lib.nkv_paged_attn_decode_noalloc(a["q"], a["kc"], a["vc"], a["lens"], a["table"],
                                             a["maxb"], a["b"], a["hq"], a["hkv"], a["d"], a["nb"],
                                             a["bs"], a["scale"], a["dtype"], a["out"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(hq=30), _lib.NKV_ERR_INVALID_ARG),
    (dict(q=None), _lib.NKV_ERR_INVALID_ARG),
    (dict(out=MISALIGNED), _lib.NKV_ERR_INVALID_ARG),
    (dict(d=96), _lib.NKV_ERR_UNSUPPORTED),
    # beyond the static scratch: 4096 fp32 sequences of up to 65536 tokens need far more
    # than NKV_DECODE_SCRATCH_BYTES of partials
    (dict(b=4096, maxb=256, dtype=0), _lib.NKV_ERR_WORKSPACE),
])
def test_decode_noalloc_rejects_before_launch(lib, kw, status):
    assert lib.nkv_paged_attn_decode_workspace_size(4096, 32, 8, 128, 256, 256) > 64 << 20
    assert decode_noalloc(lib, **kw) == status
    assert lib.nkv_last_error() != b""
    if status == _lib.NKV_ERR_WORKSPACE:
        assert b"scratch" in lib.nkv_last_error()


def test_decode_noalloc_zero_sequences_is_noop(lib):
    assert decode_noalloc(lib, b=0, q=None, lens=None, out=None) == _lib.NKV_OK


def test_decode_scratch_size_in_header():
    text = open(HEADER).read()
    m = re.search(r"#define NKV_DECODE_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == 64 << 20


def prefill(lib, **kw):
    a = dict(q=FAKE, qs=4096, kc=FAKE, vc=FAKE, cuq=FAKE, cuk=FAKE, table=FAKE, maxb=8, b=8,
             tq=16384, mq=2048, mk=2048, hq=32, hkv=8, d=128, nb=64, bs=256, scale=0.088,
             dtype=1, out=FAKE, stream=None)
    a.update(kw)
    return lib.nkv_paged_attn_prefill(a["q"], a["qs"], a["kc"], a["vc"], a["cuq"], a["cuk"],
                                      a["table"], a["maxb"], a["b"], a["tq"], a["mq"], a["mk"],
                                      a["hq"], a["hkv"], a["d"], a["nb"], a["bs"], a["scale"],
                                      a["dtype"], a["out"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(qs=4000), _lib.NKV_ERR_INVALID_ARG),          # q row stride below Hq*D
    (dict(qs=4100), _lib.NKV_ERR_INVALID_ARG),          # not a 16-byte multiple
    (dict(mq=4096), _lib.NKV_ERR_INVALID_ARG),          # max_seqlen_q > max_seqlen_k
    (dict(mk=4096), _lib.NKV_ERR_INVALID_ARG),          # exceeds max_blocks * block_size
    (dict(hkv=3, hq=9), _lib.NKV_ERR_UNSUPPORTED),           # group of 3
    (dict(cuq=None), _lib.NKV_ERR_INVALID_ARG),
    (dict(out=None), _lib.NKV_ERR_INVALID_ARG),
    (dict(kc=MISALIGNED), _lib.NKV_ERR_INVALID_ARG),
    (dict(tq=-1), _lib.NKV_ERR_INVALID_ARG),
])
def test_prefill_rejects(lib, kw, status):
    assert prefill(lib, **kw) == status


def test_prefill_empty_is_noop(lib):
    assert prefill(lib, tq=0, mq=0, q=None, out=None) == _lib.NKV_OK
    assert prefill(lib, b=0, table=FAKE) == _lib.NKV_OK


def rope_store(lib, **kw):
    a = dict(qkv=FAKE, rs=6144, pos=FAKE, wq=FAKE, wk=FAKE, cs=FAKE, maxpos=40960, eps=1e-6,
             slots=FAKE, n=64, hq=32, hkv=8, d=128, qout=FAKE, kc=FAKE, vc=FAKE, nb=600, bs=256,
             dtype=1, stream=None)
    a.update(kw)
    return lib.nkv_qk_norm_rope_store(a["qkv"], a["rs"], a["pos"], a["wq"], a["wk"], a["cs"],
                                      a["maxpos"], a["eps"], a["slots"], a["n"], a["hq"],
                                      a["hkv"], a["d"], a["qout"], a["kc"], a["vc"], a["nb"],
                                      a["bs"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=0), _lib.NKV_ERR_UNSUPPORTED),          # fp32: bf16 only
    (dict(dtype=5), _lib.NKV_ERR_INVALID_ARG),
    (dict(d=96), _lib.NKV_ERR_UNSUPPORTED),
    (dict(rs=6000), _lib.NKV_ERR_INVALID_ARG),          # below (Hq + 2 Hkv) * D
    (dict(rs=6148), _lib.NKV_ERR_INVALID_ARG),          # not a multiple of 8 elements
    (dict(maxpos=0), _lib.NKV_ERR_INVALID_ARG),
    (dict(eps=-1.0), _lib.NKV_ERR_INVALID_ARG),
    (dict(eps=float("nan")), _lib.NKV_ERR_INVALID_ARG),
    (dict(hkv=0), _lib.NKV_ERR_INVALID_ARG),
    (dict(n=-3), _lib.NKV_ERR_INVALID_ARG),
    (dict(pos=None), _lib.NKV_ERR_INVALID_ARG),
    (dict(qout=None), _lib.NKV_ERR_INVALID_ARG),
    (dict(cs=FAKE + 8), _lib.NKV_ERR_INVALID_ARG),     # table needs 16-byte alignment
    (dict(qkv=FAKE + 8), _lib.NKV_ERR_INVALID_ARG),    # 16-byte alignment
    (dict(wq=FAKE + 8), _lib.NKV_ERR_INVALID_ARG),
    (dict(nb=1 << 24, bs=1 << 10), _lib.NKV_ERR_UNSUPPORTED),
])
def test_rope_store_rejects(lib, kw, status):
    assert rope_store(lib, **kw) == status
    assert lib.nkv_last_error() != b""


def test_rope_store_zero_tokens_is_noop(lib):
    assert rope_store(lib, n=0, qkv=None, pos=None, slots=None, qout=None, kc=None, vc=None) == _lib.NKV_OK


# distinct fake buffers 1 MiB apart: a [4, 4096] bf16 row block is 32 KiB
X_, R_, W_, O_, RO_ = (0x100000 * i for i in range(1, 6))


def add_rms(lib, **kw):
    a = dict(x=X_, r=R_, w=W_, eps=1e-6, n=4, h=4096, out=O_, ro=RO_, dtype=1, stream=None)
    a.update(kw)
    return lib.nkv_add_rms_norm(a["x"], a["r"], a["w"], a["eps"], a["n"], a["h"], a["out"],
                                a["ro"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=0), _lib.NKV_ERR_UNSUPPORTED),          # fp32: bf16 only
    (dict(dtype=7), _lib.NKV_ERR_INVALID_ARG),
    (dict(h=0), _lib.NKV_ERR_INVALID_ARG),
    (dict(h=4100), _lib.NKV_ERR_INVALID_ARG),           # not a multiple of 8
    (dict(h=16392), _lib.NKV_ERR_UNSUPPORTED),          # above the widest row
    (dict(n=-1), _lib.NKV_ERR_INVALID_ARG),
    (dict(eps=2.0), _lib.NKV_ERR_INVALID_ARG),
    (dict(eps=float("nan")), _lib.NKV_ERR_INVALID_ARG),
    (dict(x=None), _lib.NKV_ERR_INVALID_ARG),
    (dict(w=None), _lib.NKV_ERR_INVALID_ARG),
    (dict(out=None), _lib.NKV_ERR_INVALID_ARG),
    (dict(x=X_ + 8), _lib.NKV_ERR_INVALID_ARG),         # 16-byte alignment
    (dict(ro=RO_ + 8), _lib.NKV_ERR_INVALID_ARG),
    (dict(out=RO_), _lib.NKV_ERR_INVALID_ARG),          # out is residual_out
    (dict(out=RO_ + 4096), _lib.NKV_ERR_INVALID_ARG),   # out overlaps residual_out
    (dict(out=X_ + 16), _lib.NKV_ERR_INVALID_ARG),      # shifted onto x: not in place
    (dict(ro=R_ - 16), _lib.NKV_ERR_INVALID_ARG),       # shifted onto residual
    (dict(out=R_ + 64), _lib.NKV_ERR_INVALID_ARG),
    (dict(ro=W_), _lib.NKV_ERR_INVALID_ARG),            # output on top of the weight
])
def test_add_rms_norm_rejects(lib, kw, status):
    assert add_rms(lib, **kw) == status
    assert lib.nkv_last_error() != b""


def test_add_rms_norm_zero_tokens_is_noop(lib):
    assert add_rms(lib, n=0, x=None, r=None, w=None, out=None, ro=None) == _lib.NKV_OK


def varlen(lib, **kw):
    a = dict(q=FAKE, qs=4096, k=FAKE, ks=1024, v=FAKE, vs=1024, cuq=FAKE, cuk=FAKE, b=2, tq=64,
             tk=64, mq=32, mk=32, hq=32, hkv=8, d=128, scale=0.088, dtype=1, out=FAKE, stream=None)
    a.update(kw)
    return lib.nkv_attn_varlen_prefill(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["cuq"],
                                       a["cuk"], a["b"], a["tq"], a["tk"], a["mq"], a["mk"], a["hq"],
                                       a["hkv"], a["d"], a["scale"], a["dtype"], a["out"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), _lib.NKV_ERR_INVALID_ARG),
    (dict(hq=12), _lib.NKV_ERR_INVALID_ARG),             # 12 heads over 8 KV heads
    (dict(hq=24, hkv=2), _lib.NKV_ERR_UNSUPPORTED),      # group 12
    (dict(d=80), _lib.NKV_ERR_UNSUPPORTED),
    (dict(scale=-1.0), _lib.NKV_ERR_INVALID_ARG),
    (dict(mq=64, mk=32), _lib.NKV_ERR_INVALID_ARG),      # max_seqlen_q > max_seqlen_k
    (dict(mk=65), _lib.NKV_ERR_INVALID_ARG),             # max_seqlen_k > total_k
    (dict(qs=4000), _lib.NKV_ERR_INVALID_ARG),           # below Hq * D
    (dict(ks=1000), _lib.NKV_ERR_INVALID_ARG),           # below Hkv * D
    (dict(vs=1028), _lib.NKV_ERR_INVALID_ARG),           # not a multiple of 16 bytes
    (dict(k=None), _lib.NKV_ERR_INVALID_ARG),
    (dict(cuk=None), _lib.NKV_ERR_INVALID_ARG),
    (dict(v=FAKE + 8), _lib.NKV_ERR_INVALID_ARG),
    (dict(tk=-1), _lib.NKV_ERR_INVALID_ARG),
])
def test_varlen_prefill_rejects(lib, kw, status):
    assert varlen(lib, **kw) == status
    assert lib.nkv_last_error() != b""


def test_varlen_prefill_empty_is_noop(lib):
    assert varlen(lib, b=0, q=None, k=None, v=None, out=None) == _lib.NKV_OK
    assert varlen(lib, tq=0, mq=0, q=None) == _lib.NKV_OK


def header_prototypes():
    """name -> list of parameter declarations, from include/nkv.h."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"\b(nkv_[a-z0-9_]+)\s*\(([^()]*)\)\s*;", text):
        out[m.group(1)] = [" ".join(p.split()) for p in m.group(2).split(",")]
    return out


def test_stream_arguments_are_hip_streams():
    # every call that launches work takes the stream last, as a hipStream_t
    protos = header_prototypes()
    launching = [n for n, ps in protos.items() if any("stream" in p for p in ps)]
    assert set(launching) >= {"nkv_store_kvcache", "nkv_paged_attn_prefill", "nkv_paged_attn_decode",
                              "nkv_attn_varlen_prefill", "nkv_qk_norm_rope_store", "nkv_add_rms_norm"}
    for n in launching:
        assert protos[n][-1] == "hipStream_t stream", (n, protos[n][-1])
    assert "typedef struct ihipStream_t* hipStream_t;" in open(HEADER).read()


def test_decode_workspace_query_signature():
    # the query takes num_kv_heads beside the five call sizes (the stream-K plan
    # counts rounds per KV head and sizes partial slots per GQA group)
    assert header_prototypes()["nkv_paged_attn_decode_workspace_size"] == [
        "int32_t num_seqs", "int32_t num_q_heads", "int32_t num_kv_heads", "int32_t head_dim",
        "int32_t max_blocks_per_seq", "int32_t block_size"]
