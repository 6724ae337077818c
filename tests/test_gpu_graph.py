"""HIP-graph capture of a whole parallel-draft round.

The round (prepare_draft_batch -> draft_forward -> accept) is captured once at
fixed shapes and replayed, the deployment form of the CUDA-graph capture the
pages describe ("P-EAGLE: Parallel Speculative Decoding in vLLM", KV Cache and
CUDA Graphs).  Every replay must reproduce the eager round exactly, also with
unrelated eager work and synchronisations between the replays, and the
replayed round is checked against the oracle: expansion and placed hidden
rows bit-exact, every token an oracle argmax up to the logit tolerance, every
KV entry the round writes equal to the oracle's (unwritten slots untouched),
acceptance equal to the oracle's on the replayed drafts.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.device import from_torch, to_torch, upload_batch

from gpu_harness import (DEV, LOGIT_TOL, _say, check_cache, check_prepare_exact, check_tokens, device_model,
                         host_weights)

pytestmark = pytest.mark.gpu


def _round(pe, model, db, K, prep, ws, tokens, tgt, acc, bonus):
    pe.prepare_draft_batch(model, K, db["query_lens"], db["target_ids"], db["target_pos"], db["num_accepted"],
                           db["bonus_ids"], db["target_hidden"], db["block_table"], out=prep)
    pe.draft_forward(model, prep, db["block_table"], db["k_cache"], db["v_cache"], workspace=ws, tokens=tokens)
    pe.accept(tokens, tgt, acc, bonus)


@pytest.mark.parametrize("name", ["tiny-fp32-c2-k3", "qwen3coder30b-bf16-c16-k5", "gptoss20b-bf16-c1-k7",
                                  "gptoss20b-bf16-c64-k7"])
def test_graph_replay_matches_eager(name):
    import drafting_draft_expand_amd as pe
    wl = synth.WORKLOADS[name]
    _say(f"graph replay {name}")
    model = device_model(wl.model, wl.wseed)
    b = synth.make_batch(wl)
    db = upload_batch(b, DEV)
    c, K, N = wl.c, wl.K, b.N
    rng = np.random.default_rng(7)
    tgt = to_torch(rng.integers(0, wl.model.vocab - 1, size=(c, K + 1)).astype(np.int32), device=DEV)
    prep = pe.prepare_draft_batch(model, K, db["query_lens"], db["target_ids"], db["target_pos"],
                                  db["num_accepted"], db["bonus_ids"], db["target_hidden"], db["block_table"])
    ws = torch.empty(model.workspace_bytes(c, K, N), dtype=torch.uint8, device=DEV)
    tokens = torch.empty((c, K), dtype=torch.int32, device=DEV)
    acc = torch.empty(c, dtype=torch.int32, device=DEV)
    bonus = torch.empty(c, dtype=torch.int32, device=DEV)
    # eager reference (twice: the KV writes of a round are idempotent)
    _round(pe, model, db, K, prep, ws, tokens, tgt, acc, bonus)
    _round(pe, model, db, K, prep, ws, tokens, tgt, acc, bonus)
    torch.cuda.synchronize()
    ref = {k: from_torch(v).copy() for k, v in (("tokens", tokens), ("acc", acc), ("bonus", bonus),
                                               ("hidden", prep["draft_hidden"]), ("slots", prep["slot_mapping"]))}
    ref_k = [from_torch(k).copy() for k in db["k_cache"]]

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            _round(pe, model, db, K, prep, ws, tokens, tgt, acc, bonus)
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device=DEV)
    for rep in range(4):
        # clobber the outputs, do unrelated eager work, then replay
        tokens.fill_(-1)
        acc.fill_(-1)
        bonus.fill_(-1)
        prep["draft_hidden"].zero_()
        scratch.mul_(1.0001)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in (("tokens", tokens), ("acc", acc), ("bonus", bonus), ("hidden", prep["draft_hidden"]),
                     ("slots", prep["slot_mapping"])):
            assert np.array_equal(from_torch(v), ref[k]), f"replay {rep}: {k} differs from the eager round"
        for got, want in zip((from_torch(k) for k in db["k_cache"]), ref_k):
            assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), f"replay {rep}: KV cache differs"
    _say("  4 replays identical to the eager round; oracle")
    spec = wl.model
    w = host_weights(spec, wl.wseed)
    ref = oracle.parallel_draft_step(spec, w, b, precision="mirror")
    check_prepare_exact(prep, ref["meta"], ref["draft_hidden"])
    fw = ref["forward"]
    tol = LOGIT_TOL[spec.dtype]
    g_tok = from_torch(tokens).astype(np.int64)
    exact = check_tokens(g_tok.reshape(-1), fw["logits"].reshape(c * K, -1), tol)
    check_cache(spec, b.k_cache, b.v_cache, [from_torch(k) for k in db["k_cache"]],
                [from_torch(v) for v in db["v_cache"]], from_torch(prep["slot_mapping"]), fw["cache_writes"],
                spec.dtype)
    oa, ob = oracle.accept(g_tok, from_torch(tgt))
    assert np.array_equal(from_torch(acc), oa) and np.array_equal(from_torch(bonus), ob)
    _say(f"  replayed round vs oracle: tokens identical to its argmax {exact:.3f}, cache and acceptance equal")
