"""Worker side of the full-length parity checks (tests only): the oracle's
float64 sampler on rows whose logits sit in a memory-mapped file.

Started with the "spawn" method, so the workers are fresh interpreters that
never touch the GPU; they import numpy and the oracle only.
"""
import sys

import numpy as np

_X = None  # bf16 bits of the checked logits rows, uint16 [n_rows, V]


def init(root, path):
    global _X
    if root not in sys.path:
        sys.path.insert(0, root)
    _X = np.load(path, mmap_mode="r")


def sample(task):
    """task: (row index in the file, mask words uint64, T, seed, step) ->
    (id, logprob, margin_chunk, margin_token) of the oracle's pick."""
    from oracle import oracle as O
    i, words, T, seed, step = task
    bits = np.asarray(_X[i], dtype=np.uint32) << np.uint32(16)
    x = bits.view(np.float32).astype(np.float64)
    pick, lp, info = O.sample_row(x, O.unpack_mask(words, x.shape[0]), T, seed, step)
    return pick, lp, info["margin_chunk"], info["margin_token"]
