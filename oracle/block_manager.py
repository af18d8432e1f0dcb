"""Plain Python model of the KV block manager -- TEST INFRASTRUCTURE ONLY.

Only tests/ (and bench.py's cpu leg, if ever) may import this module; the
product library never does, and it shares no code with the C++ manager in
paged_kv_cache_275_amd/csrc/pa_blocks.cpp.

What it models, from the pages:
  * the KV cache is a pool of fixed-size blocks (16 tokens); a sequence asks
    for a new block only when the blocks it holds are full, and gives all of
    them back when it finishes -- page "轻量级的vLLM", section
    核心机制一：分页 KV Cache;
  * sequences join and leave the running batch between steps -- same page,
    section 核心机制二：连续批处理;
  * requests can share the KV blocks of a common prompt prefix -- page
    "vllm-v0 版本介绍", section 为什么需要推理框架？ (PagedAttention item).  The
    sharing is modelled as a fork that shares every block, with reference
    counts, and a sequence about to write into a shared, partly filled last
    block first gets its own copy (copy on write).
The allocation order is a policy the pages leave open; the one modelled is the
library's documented one: free blocks form a stack with block 0 on top at the
start, allocation takes the top, a finished sequence returns its blocks from
its last to its first, and a request that cannot be met changes nothing.
"""
from __future__ import annotations

BLOCK = 16
OK, EINVAL, ENOMEM = 0, -1, -5


class OracleBlockManager:
    def __init__(self, num_blocks: int):
        self.free_stack = list(range(num_blocks - 1, -1, -1))   # last element = top
        self.refs = [0] * num_blocks
        self.seqs = {}                                          # id -> [blocks, tokens]

    # -- helpers -------------------------------------------------------------
    def _take(self):
        b = self.free_stack.pop()
        self.refs[b] = 1
        return b

    def _drop(self, b):
        self.refs[b] -= 1
        if self.refs[b] == 0:
            self.free_stack.append(b)

    # -- operations ----------------------------------------------------------
    def add_sequence(self, sid, tokens):
        if tokens < 0 or sid in self.seqs:
            return EINVAL
        need = -(-tokens // BLOCK)
        if need > len(self.free_stack):
            return ENOMEM
        self.seqs[sid] = [[self._take() for _ in range(need)], tokens]
        return OK

    def fork(self, parent, child):
        if parent == child or parent not in self.seqs or child in self.seqs:
            return EINVAL
        blocks, tokens = self.seqs[parent]
        for b in blocks:
            self.refs[b] += 1
        self.seqs[child] = [list(blocks), tokens]
        return OK

    def free(self, sid):
        if sid not in self.seqs:
            return EINVAL
        blocks, _ = self.seqs.pop(sid)
        for b in reversed(blocks):
            self._drop(b)
        return OK

    def append_batch(self, sids):
        """-> (status, slots, copies); on failure nothing changes."""
        if len(set(sids)) != len(sids) or any(s not in self.seqs for s in sids):
            return EINVAL, None, None
        # dry run on a copy of the counts, in batch order
        refs = list(self.refs)
        need = 0
        for s in sids:
            blocks, tokens = self.seqs[s]
            if tokens % BLOCK == 0:
                need += 1
            elif refs[blocks[-1]] > 1:
                need += 1
                refs[blocks[-1]] -= 1
        if need > len(self.free_stack):
            return ENOMEM, None, None
        slots, copies = [], []
        for s in sids:
            entry = self.seqs[s]
            blocks, tokens = entry
            if tokens % BLOCK == 0:
                blocks.append(self._take())
            elif self.refs[blocks[-1]] > 1:
                old = blocks[-1]
                new = self._take()
                copies.append((old, new))
                self._drop(old)
                blocks[-1] = new
            slots.append(blocks[-1] * BLOCK + tokens % BLOCK)
            entry[1] = tokens + 1
        return OK, slots, copies

    def tables(self, sids, max_blocks):
        rows, lens = [], []
        for s in sids:
            blocks, tokens = self.seqs[s]
            rows.append(blocks + [-1] * (max_blocks - len(blocks)))
            lens.append(tokens)
        return rows, lens
