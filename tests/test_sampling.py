"""CPU checks of the full-size parity sampler: on random routings, the chosen
tokens touch every block of every (minibatch, expert) segment, found here by
brute force over the rows."""
import numpy as np
import pytest

from sampling import covering_tokens


@pytest.mark.parametrize("T,E,k,mb,blk,shared", [(1000, 8, 2, 256, 16, False), (3000, 32, 8, 700, 32, True),
                                                  (50, 4, 4, 64, 8, False)])
def test_covering_tokens_touch_every_block(T, E, k, mb, blk, shared):
    rng = np.random.default_rng(T + E)
    idx = np.stack([rng.choice(E, size=k, replace=False, p=np.arange(1, E + 1) / (E * (E + 1) / 2))
                    for _ in range(T)])
    S = set(covering_tokens(idx, mb, block_rows=blk, shared=shared).tolist())
    for t0 in range(0, T, mb):
        t1 = min(T, t0 + mb)
        segs = [[t for t in range(t0, t1) if e in idx[t]] for e in range(E)]
        if shared:
            segs.append(list(range(t0, t1)))
        for rows in segs:  # rows of one segment in layout order: ascending token
            if not rows:
                continue
            assert rows[0] in S and rows[-1] in S
            for r0 in range(0, len(rows), blk):
                assert any(t in S for t in rows[r0:r0 + blk])
    assert len(S) < T
