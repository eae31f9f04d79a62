"""Seeded random programs for the prefix-cache tests: prompts that share
prefixes (a few system prompts, then private turns), requests that attach,
extend, insert and end, and evictions.  Draws only; no cache logic."""

import numpy as np


def make_program(seed, n_ops=120, block_size=4, vocab=3, evictions=True):
    rng = np.random.default_rng(seed)
    bases = [list(rng.integers(0, vocab, size=int(rng.integers(2, 6)) * block_size + int(rng.integers(0, block_size))))
             for _ in range(3)]
    ops, live, next_id = [], [], 0
    for _ in range(n_ops):
        r = rng.random()
        if r < 0.35 or not live:
            base = bases[int(rng.integers(0, len(bases)))]
            cut = int(rng.integers(0, len(base) + 1))
            prompt = base[:cut] + list(rng.integers(0, vocab, size=int(rng.integers(0, 3 * block_size))))
            ops.append(("attach", next_id, prompt))
            live.append(next_id)
            next_id += 1
        elif r < 0.55:
            ops.append(("insert", live[int(rng.integers(0, len(live)))]))
        elif r < 0.7:
            s = live.pop(int(rng.integers(0, len(live))))
            ops.append(("release", s))
        elif r < 0.85:
            if evictions:
                ops.append(("evict", int(rng.integers(0, 40))))
        else:
            base = bases[int(rng.integers(0, len(bases)))]
            ops.append(("match", base[:int(rng.integers(0, len(base) + 1))] + [int(rng.integers(0, vocab))]))
    return ops
