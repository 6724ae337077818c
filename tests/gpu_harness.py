"""Shared pieces of the GPU parity tests: run one round through the C ABI and
compare it with the oracle on the same seeded inputs."""

from __future__ import annotations

import functools

import numpy as np
import torch

import oracle
import synth
from synth.device import from_torch, upload_batch, upload_weights

LOGIT_TOL = {"fp32": 1e-5, "bf16": 2e-2}
DEV = "cuda:0"


def _say(msg):
    """Progress line for the GPU logs (flushed: a fault must not swallow it)."""
    print(msg, flush=True)



@functools.lru_cache(maxsize=4)
def host_weights(spec, wseed, prep_only=False):
    return synth.make_weights(spec, wseed, prep_only=prep_only)


_dev_cache = {}


def device_model(spec, wseed, prep_only=False, pack=True):
    import drafting_draft_expand_amd as pe
    key = (spec, wseed, prep_only, pack)
    if key not in _dev_cache:
        if len(_dev_cache) >= 2:
            _dev_cache.clear()
            torch.cuda.empty_cache()
        w = host_weights(spec, wseed, prep_only)
        dw = upload_weights(w, DEV)
        if prep_only:
            m = pe.DraftModel(spec.hidden, spec.vocab, 0, 1, 1, 16, 8, spec.dtype, dw,
                              mask_token_id=spec.mask_token_id)
        else:
            m = pe.DraftModel.from_spec(spec, dw, pack=pack)
        _dev_cache[key] = (m, dw)
    return _dev_cache[key][0]


def gpu_round(model, db, K, want_logits=True):
    import drafting_draft_expand_amd as pe
    prep = pe.prepare_draft_batch(model, K, db["query_lens"], db["target_ids"], db["target_pos"],
                                  db["num_accepted"], db["bonus_ids"], db["target_hidden"], db["block_table"])
    c = prep["num_seqs"]
    logits = torch.empty((c * K, model.desc.vocab), dtype=torch.float32, device=DEV) if want_logits else None
    gap = torch.empty(c * K, dtype=torch.float32, device=DEV)
    tokens = pe.draft_forward(model, prep, db["block_table"], db["k_cache"], db["v_cache"], logits=logits,
                              top2_gap=gap)
    torch.cuda.synchronize()
    return prep, tokens, logits, gap


META_KEYS = ("draft_ids", "draft_pos", "slot_mapping", "is_rejected", "is_masked", "hidden_map", "cu_draft",
             "kv_lens", "sample_idx")


def check_prepare_exact(prep, meta, hd_oracle):
    for k in META_KEYS:
        got = from_torch(prep[k]).astype(np.int64)
        assert np.array_equal(got, np.asarray(meta[k]).astype(np.int64)), f"{k} differs"
    got_h = from_torch(prep["draft_hidden"])
    assert got_h.dtype == hd_oracle.dtype
    assert np.array_equal(got_h.view(np.uint8), np.ascontiguousarray(hd_oracle).view(np.uint8)), \
        "draft_hidden bits differ"


def check_tokens(tokens_gpu: np.ndarray, oracle_logits: np.ndarray, tol: float):
    """GPU token must be an oracle argmax up to the logit tolerance."""
    tok = tokens_gpu.reshape(-1)
    lg = oracle_logits.reshape(len(tok), -1)
    best = lg.max(axis=1)
    picked = lg[np.arange(len(tok)), tok]
    bad = np.nonzero(picked < best - tol)[0]
    assert len(bad) == 0, f"rows {bad[:8]}: gpu token logit {picked[bad[:8]]} vs best {best[bad[:8]]}"
    exact = np.mean(tok == lg.argmax(axis=1))
    return exact


def check_cache(spec, before_k, before_v, after_k, after_v, prep_slots, writes, dtype):
    """Unwritten slots keep their bits; slots written by the pass match the oracle."""
    written = np.unique(prep_slots[prep_slots >= 0])
    for li in range(spec.n_layers):
        for before, after, key in ((before_k[li], after_k[li], "k"), (before_v[li], after_v[li], "v")):
            # [blocks, n_kv, bs, d] -> one row per slot (block * bs + offset)
            b = before.transpose(0, 2, 1, 3).reshape(-1, spec.n_kv, spec.head_dim)
            a = after.transpose(0, 2, 1, 3).reshape(-1, spec.n_kv, spec.head_dim)
            keep = np.ones(len(b), bool)
            keep[written] = False
            assert np.array_equal(a[keep].view(np.uint8), b[keep].view(np.uint8)), f"layer {li} {key}: unwritten slot changed"
            w = writes[li]
            got = oracle.decode(a[w["slots"]], dtype)
            if dtype == "fp32":
                np.testing.assert_allclose(got, w[key], rtol=1e-5, atol=1e-5)
            else:
                np.testing.assert_allclose(got, w[key], rtol=2.0 ** -7, atol=1e-2)


def upload_round(wl, batch=None):
    batch = synth.make_batch(wl) if batch is None else batch
    return batch, upload_batch(batch, DEV)
