"""Block management of a paged cache, as plain Python: the reference the
library's host-side block manager and its block-copy kernel are checked
against.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

[ch15] "KV cache / batching / paged attention", section "PagedAttention：メモ
リを「ページ」で貸し出す": the cache is split into blocks of a fixed number of
tokens handed out when a sequence needs one; answers generated from one prompt
share the prompt's blocks, and a shared block is copied only when one of them
must write into it (copy-on-write).  Section "プレフィックスキャッシュと
chunked prefill": requests whose prompts begin alike reuse the cache of that
prefix, found by a hash of the block's tokens.

The model keeps, per block, the set of its holders' count and an optional
prefix hash; a block nobody holds is free.  Which free block is handed out
next is a policy, not part of the method: the model tracks the pool as sets
and the tests compare what is unique (counts, sharing, which positions were
copied, the bytes) and check that the library's choices are valid ones.
"""

import numpy as np


class BlockModel:
    def __init__(self, num_blocks: int, block_size: int):
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.ref = [0] * num_blocks
        self.hash = {}  # block -> registered prefix hash

    # ---- queries ---------------------------------------------------------
    def free_blocks(self):
        return {b for b in range(self.num_blocks) if self.ref[b] == 0}

    def num_free(self) -> int:
        return len(self.free_blocks())

    # ---- transitions: each takes the library's choice of block and checks it
    def take(self, b: int):
        """A free block becomes held once (any free block is a valid choice)."""
        assert 0 <= b < self.num_blocks and self.ref[b] == 0, f"block {b} is not free"
        self.ref[b] = 1
        self.hash.pop(b, None)

    def share(self, b: int):
        assert self.ref[b] > 0
        self.ref[b] += 1

    def release(self, b: int):
        assert self.ref[b] > 0
        self.ref[b] -= 1

    def append(self, row, num_tokens: int, chosen_row, copy):
        """The next token at position ``num_tokens`` of a sequence with
        block-table row ``row``.  ``chosen_row``/``copy`` are the library's
        answer; returns the slot the token must go to."""
        bs = self.block_size
        lb = num_tokens // bs
        old = row[lb]
        if num_tokens % bs == 0 or old < 0:
            # a new logical block: the sequence needs a block of its own
            if old >= 0 and self.ref[old] == 1 and old not in self.hash:
                assert chosen_row[lb] == old and copy is None
            else:
                new = chosen_row[lb]
                self.take(new)
                if old >= 0 and self.ref[old] > 0:
                    self.release(old)
                assert copy is None
        elif self.ref[old] > 1 or old in self.hash:
            # shared: copy on write into a fresh block
            new = chosen_row[lb]
            assert copy == (old, new) and new != old
            self.take(new)
            self.release(old)
        else:
            assert chosen_row[lb] == old and copy is None
        assert [x for j, x in enumerate(chosen_row) if j != lb] == [x for j, x in enumerate(row) if j != lb]
        return chosen_row[lb] * bs + num_tokens % bs


def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, pairs):
    """Copies of the caches after block src is copied to block dst for every
    (src, dst) pair (targets distinct and never a source, so the order of the
    pairs does not matter)."""
    k_out, v_out = k_cache.copy(), v_cache.copy()
    pairs = [(int(s), int(d)) for s, d in np.asarray(pairs).reshape(-1, 2)]
    dsts = [d for _, d in pairs]
    assert len(set(dsts)) == len(dsts) and not set(dsts) & {s for s, _ in pairs}
    for s, d in pairs:
        k_out[d] = k_cache[s]
        v_out[d] = v_cache[s]
    return k_out, v_out
