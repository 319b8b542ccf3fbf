"""fp64 CPU oracle for the Infini-attention forward pass (test infrastructure).

This package is the *checker*, never the product: only the test suite, the
smoke check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may
import it. It shares no code with the HIP library and imports nothing from it.

Pages cited (by title and section):

* [HF-repro]  "Hugging Face Infini-Attention 再現分析" (agentlenshq.com),
  section "Infini-Attention メカニズム": the six steps Segmentation, Local
  Attention, Memory Retrieval, Integration, Memory Update, State Transfer.
* [LNCB-review] the abeam-guide review of "Leave No Context Behind: Efficient
  Infinite Context Transformers with Infini-attention", section "技術の仕組み"
  and its sub-sections "基本アイデア", "メモリ構造", "メモリの読み出し",
  "メモリの更新", "長期情報と短期情報の統合", "実装上の流れ".
* [aivaro-QA] "Как работает Infini-attention (Google, 2024) для бесконечного
  контекста?", section 4 (memory update by an outer-product sum of
  sigma(K)^T V).  Its sections 3 and 5 and its pseudocode describe a different
  slot-memory mechanism and are not followed.
"""

from .infini_ref import (  # noqa: F401
    elu_plus_one,
    gate_value,
    kv_head_of,
    segment_bounds,
    local_causal_attention,
    local_causal_attention_rows,
    memory_retrieval,
    memory_update,
    infini_attention,
    memory_chain,
    streaming_decode,
    infini_block,
    infini_attention_backward,
)
