"""Plain fp64 CPU oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the library path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run it.  It shares no code, table or constant with
the HIP kernels under ``paged_kv_cache_map_amd/``.

What it computes is the plain definition of the method: new K/V rows are
scattered into a block-paged cache through a slot map, K/V are gathered back
through a block table, and textbook softmax attention is applied in float64.
A FlashAttention-style kernel reaches exactly this result up to rounding
order, so the definition is the oracle.

Page citations used in this package (titles as the pages give them):

* [KV-mgmt]   itan.pw, "効率的な KV キャッシュ管理と Attention 計算"
              (Triton KV write kernel, its launcher, the attention module).
* [paged-doc] transformers documentation, "ページド・アテンション"
              (Varlen path and decode path, each with a worked example).
* [ch15]      1s.xyz, "KV cache / batching / paged attention"
              (KV-size closed form, GQA/MQA/MLA, PagedAttention, FlashAttention).
* [glossary]  rra.reload.co.jp, "KVキャッシュとは" (KV-cache lifecycle).

Parity status per function (pins live in ``tests/test_oracle*.py``):

* ``e4m3.decode_table`` / ``e4m3.encode``: pinned (format spot values, round
  trip, tie-to-even midpoints, torch's float8_e4m3fn conversion in range).
  The saturation branch (|x| >= 448 -> +-448) is a reading of the pages, not
  something they print; it is pinned only by that reading.
* ``paged.cu_seqlens`` / ``paged.request_index``: pinned by the varlen worked
  example of [paged-doc].
* ``paged.slot_of`` / ``paged.blocks_needed``: pinned by the decode worked
  example of [paged-doc].
* ``paged.kv_cache_write``: pinned by the same example's slots, by whole-cache
  untouched-slot checks and by the fp8 codec pins.
* ``paged.gather`` / ``paged.attention`` / ``paged.paged_decode`` /
  ``paged.varlen_prefill``: pinned by dense equivalence with torch's
  ``scaled_dot_product_attention`` in float64, by the exact special cases
  (single visible key, equal keys, empty rows) and by paging invariants.
* ``kvsize.*``: pinned by the figures [ch15] prints.
* ``int8.encode`` / ``int8.decode``: pinned by the definition's spot values
  (ties to even, saturation at +-127, NaN -> 0) and by torch's
  round-half-to-even on the same fp32 quotients; the encoding itself is a
  reading (the pages only say an INT8 cache halves the memory).
* ``paged.paged_decode_append``: pinned by the decode worked example (the
  new rows land at the derived slots and nowhere else; outputs equal float64
  SDPA over the keys walked through the printed table) and by the empty
  history case (the output is the new V row).
* ``blocks.BlockModel`` / ``blocks.copy_blocks``: pinned by the copy-on-write
  behaviour [ch15] describes (a fork shares every block; the first write to a
  shared block copies exactly that block and leaves the other holder's
  bytes as they were) on hand-made scenarios checked by other code.
"""

from . import blocks, e4m3, int8, kvsize, paged  # noqa: F401
