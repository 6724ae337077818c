"""Pins of the oracle's batch expansion and hidden placement (CPU only).

The expansion is checked against properties the pages fix, over an exhaustive
grid of verified lengths L, accepted counts a and depths K:

* one pass yields exactly K sampled rows per sequence (Step 2: Parallel
  Drafting, t_1..t_K together);
* the first sampled row pairs the bonus (new) token with the hidden state of
  the last accepted verified row, the other K-1 carry the MASK id and the
  shared hidden state (Input_i equation);
* earlier rows pair each token with the hidden state one position before it
  (shift by one, Step 2: Parallel Drafting);
* rejected rows get the padding slot and never a cache slot (KV Cache and
  CUDA Graphs); all other slots are distinct and point at the row's own
  position through the block table;
* the hidden map and the MASK rows cover every draft row exactly once.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from conftest import make_verified_batch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")
FACTS = json.load(open(GOLDEN))
PAD = FACTS["padding_slot_id"]["value"]
MASK_ID = 511
BS = 16


def _expand(vb, K):
    return oracle.expand_batch(vb["query_lens"], vb["target_ids"], vb["target_pos"], vb["num_accepted"],
                               vb["bonus_ids"], vb["block_table"], K, MASK_ID, BS)


def _check_invariants(vb, m, K):
    L = vb["query_lens"].astype(int)
    a = vb["num_accepted"].astype(int)
    c = len(L)
    T = int(L.sum())
    N = T + c * (K - 1)
    assert len(m["draft_ids"]) == N and m["cu_draft"][-1] == N
    assert oracle.PADDING_SLOT_ID == PAD
    hid = vb["target_hidden"]
    hd = oracle.scatter_broadcast(hid, m["hidden_map"], m["is_masked"], np.full(hid.shape[1], 7.5, np.float32), N)
    # exact cover of draft rows by hidden map + masked rows
    hmap = m["hidden_map"]
    assert len(set(hmap.tolist())) == T
    masked_rows = set(np.nonzero(m["is_masked"])[0].tolist())
    assert masked_rows.isdisjoint(set(hmap.tolist()))
    assert masked_rows | set(hmap.tolist()) == set(range(N))
    # slot -1 exactly on rejected rows; others distinct
    rej = m["is_rejected"].astype(bool)
    assert np.all((m["slot_mapping"] == PAD) == rej)
    valid_slots = m["slot_mapping"][~rej]
    assert len(np.unique(valid_slots)) == len(valid_slots)
    assert not np.any(rej & m["is_masked"].astype(bool))
    s = 0
    for i in range(c):
        lo, hi = m["cu_draft"][i], m["cu_draft"][i + 1]
        assert hi - lo == L[i] + K - 1
        P = int(vb["target_pos"][s])
        rows = np.arange(lo, hi)
        # rejected count, masked count
        assert rej[rows].sum() == L[i] - 1 - a[i]
        assert m["is_masked"][rows].sum() == K - 1
        # valid positions: P .. P+a+K-1, each once
        vp = sorted(m["draft_pos"][rows][~rej[rows]].tolist())
        assert vp == list(range(P, P + a[i] + K))
        assert m["kv_lens"][i] == P + a[i] + K
        # slots resolve to the row's own position through the block table
        inv = {int(b): j for j, b in enumerate(vb["block_table"][i])}
        for r in rows[~rej[rows]]:
            sl = int(m["slot_mapping"][r])
            assert inv[sl // BS] * BS + sl % BS == m["draft_pos"][r]
        # exactly K sampled rows: NTP row then K-1 MASK rows
        samp = m["sample_idx"][i * K:(i + 1) * K]
        assert len(samp) == K and np.all(np.diff(samp) == 1)
        ntp = samp[0]
        assert m["draft_ids"][ntp] == vb["bonus_ids"][i] and not m["is_masked"][ntp]
        assert m["draft_pos"][ntp] == P + a[i]
        np.testing.assert_array_equal(hd[ntp], hid[s + a[i]])        # h_context
        for r in samp[1:]:
            assert m["is_masked"][r] and m["draft_ids"][r] == MASK_ID
            assert np.all(hd[r] == 7.5)                              # h_shared
        # shift by one on the accepted rows: token of position q+1 with hidden of q
        for r in rows:
            if m["is_masked"][r] or rej[r] or r == ntp:
                continue
            q = int(m["draft_pos"][r])
            assert m["draft_ids"][r] == vb["target_ids"][s + (q - P) + 1]
            np.testing.assert_array_equal(hd[r], hid[s + (q - P)])
        # rejected rows keep their own verified hidden state
        for r in rows[rej[rows]]:
            q = int(m["draft_pos"][r])
            np.testing.assert_array_equal(hd[r], hid[s + (q - P)])
        s += L[i]


@pytest.mark.parametrize("K", range(1, 9))
def test_expand_exhaustive_single_sequence(K):
    rng = np.random.default_rng(100 + K)
    for L in range(1, 9):
        for a in range(L):
            vb = make_verified_batch(rng, [L], [a], K)
            _check_invariants(vb, _expand(vb, K), K)


@pytest.mark.parametrize("K", [1, 3, 7])
def test_expand_exhaustive_three_sequences(K):
    rng = np.random.default_rng(200 + K)
    for L0 in range(1, 9):
        for a0 in range(L0):
            L = [L0, int(rng.integers(1, 9)), int(rng.integers(1, 9))]
            a = [a0, int(rng.integers(0, L[1])), int(rng.integers(0, L[2]))]
            vb = make_verified_batch(rng, L, a, K)
            _check_invariants(vb, _expand(vb, K), K)


def test_expand_rejects_bad_accepted_count():
    rng = np.random.default_rng(3)
    vb = make_verified_batch(rng, [4], [0], 3)
    vb["num_accepted"] = np.array([4], np.int32)
    with pytest.raises(ValueError):
        _expand(vb, 3)


def test_prefill_like_round_has_no_rejected_rows():
    # a = L-1: every verified row accepted (first round after prefill)
    rng = np.random.default_rng(4)
    vb = make_verified_batch(rng, [6, 1], [5, 0], 4)
    m = _expand(vb, 4)
    assert not m["is_rejected"].any()
    _check_invariants(vb, m, 4)


def test_scatter_broadcast_matches_one_hot_contraction():
    """Independent formulation of the placement: Hd = S^T Ht + m h_shared^T with
    S the one-hot hidden map and m the masked indicator (exact in float64)."""
    rng = np.random.default_rng(5)
    vb = make_verified_batch(rng, [8, 3, 5], [2, 0, 4], 7, H=32)
    m = _expand(vb, 7)
    N = len(m["draft_ids"])
    ht = torch.tensor(vb["target_hidden"], dtype=torch.float64)
    hs = torch.tensor(rng.standard_normal(32), dtype=torch.float64)
    S = torch.zeros(ht.shape[0], N, dtype=torch.float64)
    S[torch.arange(ht.shape[0]), torch.tensor(m["hidden_map"])] = 1.0
    msk = torch.tensor(m["is_masked"], dtype=torch.float64)
    ref = S.T @ ht + msk[:, None] * hs[None, :]
    got = oracle.scatter_broadcast(vb["target_hidden"].astype(np.float64), m["hidden_map"],
                                   m["is_masked"], hs.numpy(), N)
    assert np.array_equal(got, ref.numpy())


def test_scatter_broadcast_bf16_bits_exact():
    import synth
    wl = synth.WORKLOADS["prep-bf16-c64-k7-h2880"]
    b = synth.make_batch(wl, with_cache=False)
    w = synth.make_weights(wl.model, wl.seed, prep_only=True)
    m = oracle.expand_batch(b.query_lens, b.target_ids, b.target_pos, b.num_accepted, b.bonus_ids,
                            b.block_table, b.K, wl.model.mask_token_id)
    hd = oracle.scatter_broadcast(b.target_hidden, m["hidden_map"], m["is_masked"], w["h_shared"], b.N)
    assert hd.dtype == np.uint16 and hd.shape == (b.N, wl.model.hidden)
    assert np.array_equal(hd[m["hidden_map"]], b.target_hidden)
    assert np.all(hd[m["is_masked"].astype(bool)] == w["h_shared"][None, :])


def test_training_positions_closed_form():
    """The pages' long-sequence training example: N x K positions, attention
    matrix elements = positions^2 (at least 4e9)."""
    f = FACTS["training_positions_example"]["value"]
    assert f["N"] * f["K"] == f["positions"]
    assert f["positions"] ** 2 >= f["attention_elements_at_least"]
