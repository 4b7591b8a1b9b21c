"""CPU oracle for the paged KV-cache store and paged causal GQA attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The product path (``paged_kv_cache_258_amd``) never imports it and the oracle
never imports the product: they share no code.

Sources (pages, cited by title and section):
  * 「Nano-vLLM深度解读（下）」 (devpress.csdn.net), §4 "与 KV Cache 数据面结合":
    the ``attention.py`` listing (``store_kvcache`` and ``Attention.forward``).
  * 「同一个 Qwen3，两种写法：从 transformers 到 nano-vllm 的推理改造」
    (violet-quartz.github.io), §3.2 (flat varlen layout and ``cu_seqlens``),
    §3.3 (paged pool, ``block_table``, ``slot_mapping``), §3.4 (GQA, ``repeat_kv``,
    the two FlashAttention entries).

Modules:
  ref    -- store, gather, prefill and decode in numpy float64 (the definition).
  brute  -- contiguous, mask-materialising brute force used only to pin ``ref``.

Parity status: every function here is pinned by ``tests/test_oracle_cpu.py``
(worked examples from the pages, closed forms, invariants and the brute force).
No function is "parity unpinned".
"""

from . import ref, brute  # noqa: F401
