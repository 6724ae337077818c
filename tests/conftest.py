import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")


def make_verified_batch(rng, L_list, a_list, K, vocab=512, block_size=16, ctx=None, H=8):
    """Small hand-shaped verified batch (ids, positions, block tables) for sweeps."""
    c = len(L_list)
    L = np.asarray(L_list, dtype=np.int32)
    a = np.asarray(a_list, dtype=np.int32)
    P = rng.integers(0, 40, size=c) if ctx is None else np.asarray(ctx)
    ids = rng.integers(0, vocab - 1, size=int(L.sum())).astype(np.int32)
    pos = np.concatenate([P[i] + np.arange(L[i]) for i in range(c)]).astype(np.int32)
    bonus = rng.integers(0, vocab - 1, size=c).astype(np.int32)
    need = [int(-(-(P[i] + L[i] + K - 1) // block_size)) for i in range(c)]
    perm = rng.permutation(sum(need)).astype(np.int32)
    bt = np.full((c, max(need)), sum(need), dtype=np.int32)
    o = 0
    for i in range(c):
        bt[i, :need[i]] = perm[o:o + need[i]]
        o += need[i]
    hidden = rng.standard_normal((int(L.sum()), H)).astype(np.float32)
    return dict(query_lens=L, target_ids=ids, target_pos=pos, num_accepted=a, bonus_ids=bonus,
                block_table=bt, context=P, target_hidden=hidden, num_blocks=sum(need) + 1)


@pytest.fixture(scope="session")
def tiny():
    import synth
    wl = synth.WORKLOADS["tiny-fp32-c2-k3"]
    return wl, synth.make_weights(wl.model, wl.seed), synth.make_batch(wl)
