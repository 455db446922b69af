"""Token samples for full-size parity checks.

At full size the oracle evaluates a subset of tokens.  The subset is chosen
from the routing so that every output tile of the grouped GEMMs holds a checked
row: within each minibatch, the rows of one expert are that expert's tokens in
ascending order, cut into M tiles from the segment's first row.  The sample
covers every block of `block_rows` consecutive rows of every (minibatch,
expert) segment, and always the segment's first and last row.  With
block_rows = 128 it also covers every 256-row tile.  Each token contributes one
row to each of its k experts, so a greedy cover needs far fewer tokens than
blocks.  Only the routing indices are used here; no layer arithmetic.
"""
from __future__ import annotations

import numpy as np


def segment_rows(idx: np.ndarray, minibatch: int, shared: bool = False):
    """For every (minibatch b, expert e): the tokens of the segment in row order
    (ascending token), as {(b, e): array of absolute token ids}.  With `shared`,
    expert E (the shared expert, after the E routed ones) takes every token."""
    T = idx.shape[0]
    segs = {}
    for b, t0 in enumerate(range(0, T, minibatch)):
        t1 = min(T, t0 + minibatch)
        sub = idx[t0:t1]
        for e in np.unique(sub):
            toks = t0 + np.nonzero((sub == e).any(axis=1))[0]
            segs[(b, int(e))] = toks
        if shared:
            segs[(b, -1)] = np.arange(t0, t1)
    return segs


def covering_tokens(idx: np.ndarray, minibatch: int, block_rows: int = 128, shared: bool = False) -> np.ndarray:
    """Sorted token ids whose rows touch every block of `block_rows` rows of every
    (minibatch, expert) segment, including each segment's first and last row
    (and those of the shared expert's segment with `shared`)."""
    segs = segment_rows(idx, minibatch, shared)
    blocks_of_token = {}
    all_blocks = set()
    chosen = set()
    for (b, e), toks in segs.items():
        chosen.add(int(toks[0]))
        chosen.add(int(toks[-1]))
        for r, t in enumerate(toks):
            blk = (b, e, r // block_rows)
            all_blocks.add(blk)
            blocks_of_token.setdefault(int(t), []).append(blk)
    covered = set()
    for t in chosen:
        covered.update(blocks_of_token[t])
    # greedy: for each block still uncovered, take the token in it that covers
    # the most uncovered blocks
    by_block = {}
    for t, blks in blocks_of_token.items():
        for blk in blks:
            by_block.setdefault(blk, []).append(t)
    for blk in sorted(all_blocks):
        if blk in covered:
            continue
        best = max(by_block[blk], key=lambda t: (sum(x not in covered for x in blocks_of_token[t]), -t))
        chosen.add(best)
        covered.update(blocks_of_token[best])
    assert covered == all_blocks
    return np.array(sorted(chosen), dtype=np.int64)
