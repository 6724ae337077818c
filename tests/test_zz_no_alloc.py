"""The allocation-free drafter pass (pe_draft_forward_noalloc, for callers
that cannot allocate) against pe_draft_forward on the same inputs.

Two calls in a row share the library's static scratch, the second on a
smaller batch, so stale contents of the first call must not reach the second.
Both entry points run the same kernels on the same inputs, so tokens, top-2
gaps, logits and the KV cache they write must be identical bit for bit.  A
batch whose scratch exceeds the static array is refused.
"""

import numpy as np
import pytest
import torch

import synth
from synth.device import from_torch, upload_batch

from gpu_harness import DEV, _say, device_model

pytestmark = pytest.mark.gpu


def _both(pe, model, batch):
    """Run the pass through pe_draft_forward and pe_draft_forward_noalloc on
    separate copies of the caches; return both sets of outputs."""
    K, V = batch.K, model.desc.vocab
    outs = {}
    for name in ("workspace", "noalloc"):
        db = upload_batch(batch, DEV)
        prep = pe.prepare_draft_batch(model, K, db["query_lens"], db["target_ids"], db["target_pos"],
                                      db["num_accepted"], db["bonus_ids"], db["target_hidden"], db["block_table"])
        c = prep["num_seqs"]
        tokens = torch.full((c, K), -1, dtype=torch.int32, device=DEV)
        logits = torch.full((c * K, V), float("nan"), dtype=torch.float32, device=DEV)
        gap = torch.full((c * K,), float("nan"), dtype=torch.float32, device=DEV)
        if name == "workspace":
            pe.draft_forward(model, prep, db["block_table"], db["k_cache"], db["v_cache"], tokens=tokens,
                             logits=logits, top2_gap=gap)
        else:
            pe.draft_forward_noalloc(model, prep, db["block_table"], db["k_cache"], db["v_cache"], tokens,
                                     logits=logits, top2_gap=gap)
        torch.cuda.synchronize()
        outs[name] = [from_torch(tokens).copy(), from_torch(gap).copy(), from_torch(logits).copy()] + \
                     [from_torch(t).copy() for t in db["k_cache"] + db["v_cache"]]
        del db, prep
    return outs


def _same(outs, where):
    names = ["tokens", "top2_gap", "logits"] + ["k/v cache"] * (len(outs["workspace"]) - 3)
    for n, a, b in zip(names, outs["workspace"], outs["noalloc"]):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{where}: {n} differs"


@pytest.mark.parametrize("shape", ["gptoss-c1", "small-bf16"])
def test_noalloc_matches_workspace_forward_twice(shape):
    import drafting_draft_expand_amd as pe
    if shape == "gptoss-c1":
        big = synth.WORKLOADS["gptoss20b-bf16-c1-k7"]
        small = synth.WORKLOADS["gptoss20b-bf16-c1-k3"]
    else:
        spec = synth.ModelSpec(hidden=256, vocab=1000, n_layers=1, n_q=8, n_kv=2, head_dim=64, inter=512)
        big = synth.Workload("noalloc-big", spec, c=6, K=5, ctx_lo=10, ctx_hi=300, accept_hi=5, seed=81)
        small = synth.Workload("noalloc-small", spec, c=2, K=3, ctx_lo=10, ctx_hi=300, accept_hi=3, seed=82)
    model = device_model(big.model, big.wseed)
    for wl in (big, small):
        b = synth.make_batch(wl)
        need = model.workspace_bytes(b.c, b.K, b.N)
        _say(f"noalloc {wl.name}: c={b.c} K={b.K} N={b.N}, scratch {need / 2**20:.1f} MiB")
        assert need <= pe._lib.STATIC_SCRATCH_BYTES
        _same(_both(pe, model, b), wl.name)


def test_noalloc_refuses_batch_beyond_its_scratch():
    import drafting_draft_expand_amd as pe
    wl = synth.WORKLOADS["qwen3coder30b-bf16-c16-k7"]
    model = device_model(wl.model, wl.wseed)
    b = synth.make_batch(wl)
    assert model.workspace_bytes(b.c, b.K, b.N) > pe._lib.STATIC_SCRATCH_BYTES
    db = upload_batch(b, DEV)
    prep = pe.prepare_draft_batch(model, b.K, db["query_lens"], db["target_ids"], db["target_pos"],
                                  db["num_accepted"], db["bonus_ids"], db["target_hidden"], db["block_table"])
    tokens = torch.empty((b.c, b.K), dtype=torch.int32, device=DEV)
    with pytest.raises(pe.PeError) as e:
        pe.draft_forward_noalloc(model, prep, db["block_table"], db["k_cache"], db["v_cache"], tokens)
    assert e.value.status == pe._lib.PE_EWORKSPACE
    torch.cuda.synchronize()
