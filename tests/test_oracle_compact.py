"""Pins for the compacted draft layout (rejected rows dropped, inert padding
after the live rows): it holds exactly the fixed layout's non-rejected rows,
in order, and the drafter pass over it yields the same tokens and logits.
"""

import itertools

import numpy as np

import oracle
import synth
from conftest import make_verified_batch


def _both(vb, K, mask_id=511):
    args = (vb["query_lens"], vb["target_ids"], vb["target_pos"], vb["num_accepted"], vb["bonus_ids"],
            vb["block_table"], K, mask_id, 16)
    return oracle.expand_batch(*args), oracle.expand_batch(*args, compact=True)


def test_compact_rows_are_the_fixed_layouts_live_rows():
    rng = np.random.default_rng(0)
    for L, K in itertools.product((1, 2, 5), (1, 2, 4)):
        for a_list in itertools.product(*[range(L)] * 3):
            vb = make_verified_batch(rng, [L, L, L], list(a_list), K)
            fx, cp = _both(vb, K)
            c, N = 3, 3 * L + 3 * (K - 1)
            live = int(sum(a_list)) + c * K
            assert len(cp["draft_ids"]) == N and int(cp["cu_draft"][c]) == live
            for i, a in enumerate(a_list):
                f0, c0 = int(fx["cu_draft"][i]), int(cp["cu_draft"][i])
                n = a + K
                for key in ("draft_ids", "draft_pos", "slot_mapping", "is_masked"):
                    np.testing.assert_array_equal(cp[key][c0:c0 + n], fx[key][f0:f0 + n])
                assert not cp["is_rejected"][c0:c0 + n].any()
                assert int(cp["cu_draft"][i + 1]) - c0 == n if i + 1 < c else live - c0 == n
                np.testing.assert_array_equal(cp["sample_idx"][i * K:(i + 1) * K], c0 + a + np.arange(K))
            # padding: everything past the live rows is inert
            assert cp["is_rejected"][live:].all() and (cp["slot_mapping"][live:] == -1).all()
            assert not cp["is_masked"][live:].any()
            np.testing.assert_array_equal(cp["kv_lens"], fx["kv_lens"])
            # hidden map: accepted prefix kept, the rest dropped
            s = 0
            for i, a in enumerate(a_list):
                for j in range(L):
                    want = int(cp["cu_draft"][i]) + j if j <= a else -1
                    assert int(cp["hidden_map"][s + j]) == want
                s += L


def test_compact_forward_equals_fixed_forward():
    spec = synth.ModelSpec(hidden=32, vocab=97, n_layers=2, n_q=4, n_kv=2, head_dim=8, inter=48, dtype="fp32")
    wl = synth.Workload("compact", spec, c=4, K=3, ctx_lo=3, ctx_hi=40, accept_hi=3, seed=81)
    w = synth.make_weights(spec, 81)
    b = synth.make_batch(wl)
    assert (b.num_accepted < wl.L - 1).any(), "need some rejected rows for the comparison"
    fx = oracle.parallel_draft_step(spec, w, b, precision="fp64")["forward"]
    cp_step = oracle.parallel_draft_step(spec, w, b, precision="fp64", compact=True)
    cp = cp_step["forward"]
    assert np.array_equal(fx["tokens"], cp["tokens"])
    np.testing.assert_allclose(cp["logits"], fx["logits"], rtol=1e-12, atol=1e-13)
    # fewer rows went through the drafter
    assert len(cp["rows"]) == int(b.num_accepted.sum()) + wl.c * wl.K < len(fx["rows"])
