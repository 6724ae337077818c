"""GPU parity of the steps around one parallel-draft round.

* The autoregressive baseline (K one-token passes on the same kernels,
  "P-EAGLE: Parallel Speculative Decoding in vLLM", Solving the Autoregressive
  Drafting Bottleneck) against the oracle's, teacher-forced with the GPU's own
  tokens and fed-back hidden rows (so every pass sees identical inputs): every
  step's logits within the logit tolerance, every token an oracle argmax up to
  it, the fed-back rows close to the oracle's own (5% of the row rms in bf16),
  the cache entries the passes append match the oracle's.
* Several rounds in a row with the KV cache carried over: accept's outputs
  and the GPU-built next verified batch feed the next prepare; the oracle
  keeps its own cache state, committing each round's writes.  Checked per
  round: expansion bit-exact, logits within the tolerance, tokens oracle
  argmaxes, acceptance and next-batch metadata exact; at the end the cache.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.device import from_torch, to_torch, upload_batch

from gpu_harness import DEV, LOGIT_TOL, _say, check_prepare_exact, check_tokens, device_model, host_weights

pytestmark = pytest.mark.gpu


def _small_bf16(c, K, seed, ctx_hi=200):
    spec = synth.ModelSpec(hidden=256, vocab=1000, n_layers=1, n_q=8, n_kv=2, head_dim=64, inter=512)
    return synth.Workload(f"small-bf16-c{c}-k{K}", spec, c=c, K=K, ctx_lo=10, ctx_hi=ctx_hi, accept_hi=K,
                          seed=seed)


def _workload(name):
    if name == "small-bf16":
        return _small_bf16(3, 5, 71)
    if name == "two-layer-fp32":
        spec = synth.ModelSpec(hidden=96, vocab=300, n_layers=2, n_q=6, n_kv=2, head_dim=32, inter=160,
                               dtype="fp32")
        return synth.Workload("two-layer-ar", spec, c=3, K=4, ctx_lo=0, ctx_hi=70, accept_hi=4, seed=72)
    return synth.WORKLOADS[name]


def _cache_close(spec, got, want, where):
    """Same slots written (NaN canaries elsewhere), values within the cache
    tolerance."""
    g = oracle.decode(got, spec.dtype)
    w = oracle.decode(want, spec.dtype)
    both = np.isfinite(w)
    assert np.array_equal(np.isfinite(g), both), f"{where}: written slots differ"
    err = float(np.max(np.abs(g[both] - w[both]))) if both.any() else 0.0
    _say(f"  {where}: max|d| = {err:.3e}")
    if spec.dtype == "fp32":
        np.testing.assert_allclose(g[both], w[both], rtol=1e-5, atol=1e-5, err_msg=where)
    else:
        np.testing.assert_allclose(g[both], w[both], rtol=2.0 ** -7, atol=1e-2, err_msg=where)


@pytest.mark.parametrize("name", ["tiny-fp32-c2-k3", "two-layer-fp32", "small-bf16", "gptoss20b-bf16-c1-k7",
                                  "qwen3coder30b-bf16-c16-k3"])
def test_autoregressive_matches_oracle(name):
    import drafting_draft_expand_amd as pe
    wl = _workload(name)
    spec, K = wl.model, wl.K
    _say(f"autoregressive {wl.name} K={K}")
    w = host_weights(spec, wl.wseed)
    model = device_model(spec, wl.wseed)
    b = synth.make_batch(wl)
    db = upload_batch(b, DEV)
    logits = torch.empty((K, wl.c, spec.vocab), dtype=torch.float32, device=DEV)
    fed = torch.empty((K - 1, wl.c, spec.hidden), dtype=model.torch_dtype, device=DEV)
    toks = pe.draft_autoregressive(model, K, db["query_lens"], db["target_ids"], db["target_pos"],
                                   db["num_accepted"], db["bonus_ids"], db["target_hidden"], db["block_table"],
                                   db["k_cache"], db["v_cache"], logits=logits, fed_hidden=fed)
    torch.cuda.synchronize()
    g = from_torch(toks).astype(np.int64)
    g_logits = from_torch(logits)
    g_fed = from_torch(fed)
    _say("  gpu done, oracle")
    # teacher forcing: every pass of the oracle takes the GPU's token and fed-back
    # hidden row, so each pass is compared on identical inputs
    ref = oracle.autoregressive_draft(spec, w, b, K, precision="mirror", forced_tokens=g, forced_hidden=g_fed)
    tol = LOGIT_TOL[spec.dtype]
    # the fed-back rows themselves against the oracle's own rounding of the
    # residual it computes from the same inputs.  That residual carries the
    # pass's usual deviation from the oracle (in bf16 the attention
    # probabilities are a bf16 matrix operand on the GPU and float64 in the
    # oracle), so the bound is relative to the row's rms: 5% of it, where
    # feeding back a wrong row or quantity (another row's residual, the
    # normalised row) is off by the order of the rms itself.
    if K > 1:
        go, oo = oracle.decode(g_fed, spec.dtype), oracle.decode(ref["fed_hidden"], spec.dtype)
        rms = np.sqrt(np.mean(oo * oo, axis=-1, keepdims=True))
        rel = float(np.max(np.abs(go - oo) / rms))
        same = float(np.mean(g_fed == ref["fed_hidden"]))
        _say(f"  fed-back hidden rows: {same:.4f} bit-identical, max|d| = {rel:.3e} of the row rms")
        assert rel <= (0.05 if spec.dtype == "bf16" else 1e-5)
    assert np.isfinite(g_logits).all()
    for k in range(K):
        err = float(np.max(np.abs(g_logits[k] - ref["logits"][:, k])))
        exact = check_tokens(g[:, k], ref["logits"][:, k], tol)
        _say(f"  step {k}: max|dlogit| = {err:.3e} (tol {tol}), tokens identical to oracle argmax {exact:.3f}")
        assert err <= tol, f"step {k}"
        # the reported logits are the ones the token was taken from (lowest id on ties)
        assert np.array_equal(g_logits[k].argmax(axis=1), g[:, k])
    for li in range(spec.n_layers):
        _cache_close(spec, from_torch(db["k_cache"][li]), ref["k_cache"][li], f"k cache layer {li}")
        _cache_close(spec, from_torch(db["v_cache"][li]), ref["v_cache"][li], f"v cache layer {li}")


def _round_inputs_host(b):
    return dict(query_lens=np.asarray(b.query_lens), target_ids=np.asarray(b.target_ids),
                target_pos=np.asarray(b.target_pos), num_accepted=np.asarray(b.num_accepted),
                bonus_ids=np.asarray(b.bonus_ids), target_hidden=np.asarray(b.target_hidden))


@pytest.mark.parametrize("name,rounds,prefill", [("tiny-fp32-c2-k3", 4, False), ("small-bf16", 3, True),
                                                 ("qwen3coder30b-bf16-c16-k3", 2, False)])
def test_multi_round_kv_continuity(name, rounds, prefill):
    import drafting_draft_expand_amd as pe
    wl = _workload(name)
    spec, K, c = wl.model, wl.K, wl.c
    _say(f"multi-round {wl.name} rounds={rounds} prefill={prefill}")
    w = host_weights(spec, wl.wseed)
    model = device_model(spec, wl.wseed)
    acc0 = np.full(c, wl.L - 1) if prefill else None
    b = synth.make_batch(wl, accepted=acc0, extra_positions=rounds * (K + 1) + K)
    db = upload_batch(b, DEV)
    kc = [np.array(k, copy=True) for k in b.k_cache]
    vc = [np.array(v, copy=True) for v in b.v_cache]
    host = _round_inputs_host(b)
    dev = {k: db[k] for k in ("query_lens", "target_ids", "target_pos", "num_accepted", "bonus_ids",
                              "target_hidden")}
    tol = LOGIT_TOL[spec.dtype]
    rng = np.random.default_rng(wl.seed + 500)
    for r in range(rounds):
        prep = pe.prepare_draft_batch(model, K, dev["query_lens"], dev["target_ids"], dev["target_pos"],
                                      dev["num_accepted"], dev["bonus_ids"], dev["target_hidden"],
                                      db["block_table"])
        logits = torch.empty((c * K, spec.vocab), dtype=torch.float32, device=DEV)
        tokens = pe.draft_forward(model, prep, db["block_table"], db["k_cache"], db["v_cache"], logits=logits)
        # synthetic verifier: target tokens agree with the drafts with the
        # workload's per-depth probability; target hidden states for the
        # K+1 verified rows of the next round
        g = from_torch(tokens).astype(np.int64)
        u = rng.random((c, K))
        alt = rng.integers(0, spec.vocab - 1, size=(c, K + 1))
        tgt = synth.target_tokens_from_drafts(g, u, alt, wl.agree_probs(), spec.vocab)
        acc, bonus = pe.accept(tokens, to_torch(tgt.astype(np.int32), device=DEV))
        nxt = pe.next_verified_batch(K, prep["kv_lens"], dev["bonus_ids"], tokens, acc, bonus)
        torch.cuda.synchronize()
        # oracle round on the same verified batch, its own cache state
        meta = oracle.expand_batch(host["query_lens"], host["target_ids"], host["target_pos"],
                                   host["num_accepted"], host["bonus_ids"], b.block_table, K, spec.mask_token_id,
                                   spec.block_size)
        hd = oracle.scatter_broadcast(host["target_hidden"], meta["hidden_map"], meta["is_masked"], w["h_shared"],
                                      len(meta["draft_ids"]))
        check_prepare_exact(prep, meta, hd)
        fw = oracle.draft_forward(spec, w, meta, hd, b.block_table, kc, vc, K, precision="mirror")
        oracle.apply_cache_writes(spec, kc, vc, fw["cache_writes"])
        o_logits = fw["logits"].reshape(c * K, -1)
        err = float(np.max(np.abs(from_torch(logits) - o_logits)))
        assert err <= tol, f"round {r}: max|dlogit| = {err:.3e}"
        exact = check_tokens(g.reshape(-1), o_logits, tol)
        oa, ob = oracle.accept(g, tgt)
        assert np.array_equal(from_torch(acc), oa) and np.array_equal(from_torch(bonus), ob)
        on = oracle.next_verified_batch(meta["kv_lens"], host["bonus_ids"], g, oa, ob, K)
        for k in ("query_lens", "target_ids", "target_pos", "num_accepted", "bonus_ids"):
            assert np.array_equal(from_torch(nxt[k]), on[k]), f"round {r}: next-batch {k} differs"
        _say(f"  round {r}: max|dlogit| = {err:.3e} (tol {tol}), tokens identical to oracle argmax {exact:.3f}, "
             f"accepted {oa.tolist()}")
        hid = synth.store(rng.standard_normal((c * (K + 1), spec.hidden)).astype(np.float32), spec.dtype)
        host = dict(on, target_hidden=hid)
        dev = dict(nxt, target_hidden=to_torch(hid, device=DEV))
    for li in range(spec.n_layers):
        _cache_close(spec, from_torch(db["k_cache"][li]), kc[li], f"k cache layer {li} after {rounds} rounds")
        _cache_close(spec, from_torch(db["v_cache"][li]), vc[li], f"v cache layer {li} after {rounds} rounds")
