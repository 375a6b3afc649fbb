"""Seeded layouts of a paged cache (block tables, block counts, tail lengths).

Input structure only: which physical block holds which logical block of which
sequence, and how many tokens each sequence has.  Holds none of the method's
arithmetic; the tests and the benchmark use it for the oracle and the GPU
alike.
"""
import numpy as np


def paged_layout(seed, batch, max_blocks, pool_blocks=None, full=False):
    """Random block tables over a shuffled pool.

    Returns (block_table [batch][max_blocks] int32, n_blocks [batch] int32,
    tail_len [batch] int32, pool_blocks).  Every sequence gets distinct
    physical blocks; unused table entries are -1.  With full=True every
    sequence has max_blocks blocks and a non-empty tail.
    """
    rng = np.random.default_rng(seed)
    if full:
        n_blocks = np.full(batch, max_blocks, np.int32)
        tail = rng.integers(1, 128, size=batch).astype(np.int32)
    else:
        n_blocks = rng.integers(0, max_blocks + 1, size=batch).astype(np.int32)
        tail = rng.integers(0, 128, size=batch).astype(np.int32)
        # the edge cases: an empty sequence, a tail-only one, a full one
        if batch >= 3:
            n_blocks[0], tail[0] = 0, 0
            n_blocks[1], tail[1] = 0, 77
            n_blocks[2], tail[2] = max_blocks, 127
    need = int(n_blocks.sum())
    if pool_blocks is None:
        pool_blocks = need + 3
    assert pool_blocks >= need
    phys = rng.permutation(pool_blocks)[:need]
    table = np.full((batch, max_blocks), -1, np.int32)
    k = 0
    for b in range(batch):
        table[b, :n_blocks[b]] = phys[k:k + n_blocks[b]]
        k += n_blocks[b]
    return table, n_blocks, tail, pool_blocks


def gather_sequence_tiles(table, n_blocks, n_kv_heads):
    """Pool tile index of every (b, g, logical block) in sequence order:
    list over (b, g) of int64 arrays (physical block p holds tiles
    p * n_kv_heads + g)."""
    out = []
    for b in range(table.shape[0]):
        for g in range(n_kv_heads):
            out.append(table[b, :n_blocks[b]].astype(np.int64) * n_kv_heads + g)
    return out
