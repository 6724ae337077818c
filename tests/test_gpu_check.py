"""GPU tests of pe_check_verified_batch, the device-side check of the verified
batch that the expansion assumes well formed ("P-EAGLE: Parallel Speculative
Decoding in vLLM", vLLM Implementation Details: Fused Triton Kernel lists its
fields).  A well-formed batch sets no bits; each malformed field sets its bit.
The check reads only in-bounds locations, so the malformed batches are safe to
hand to it (they are never handed to the expansion)."""

import numpy as np
import pytest
import torch

import synth
from synth.device import to_torch, upload_batch

from gpu_harness import DEV, _say, device_model

pytestmark = pytest.mark.gpu


def _bits(model, K, d):
    import drafting_draft_expand_amd as pe
    e = pe.check_verified_batch(model, K, d["query_lens"], d["target_ids"], d["target_pos"], d["num_accepted"],
                                d["bonus_ids"], d["block_table"])
    torch.cuda.synchronize()
    return int(e.cpu()[0])


@pytest.mark.parametrize("name", ["tiny-fp32-c2-k3", "prep-bf16-c64-k7-h2880"])
def test_check_verified_batch(name):
    import drafting_draft_expand_amd as pe
    wl = synth.WORKLOADS[name]
    _say(f"check {name}")
    model = device_model(wl.model, wl.wseed, prep_only=wl.prep_only)
    b = synth.make_batch(wl)
    d = upload_batch(b, DEV)
    assert _bits(model, wl.K, d) == 0
    V = wl.model.vocab
    L0 = int(b.query_lens[0])

    def mutated(key, fn, bit, exact=True):
        host = d[key].cpu().numpy().copy()
        host = fn(host)
        dd = dict(d)
        dd[key] = to_torch(np.ascontiguousarray(host), device=DEV)
        got = _bits(model, wl.K, dd)
        _say(f"  {key}: bits {got:#x}")
        assert (got == bit) if exact else (got & bit), (key, got, bit)

    def setv(idx, v):
        def f(a):
            a[idx] = v
            return a
        return f

    mutated("num_accepted", setv(0, L0), pe.PE_CHECK_ACCEPTED)
    mutated("num_accepted", setv(wl.c - 1, -1), pe.PE_CHECK_ACCEPTED)
    mutated("target_ids", setv(1, V), pe.PE_CHECK_TOKEN_ID)
    mutated("target_ids", setv(-1, -3), pe.PE_CHECK_TOKEN_ID)
    mutated("bonus_ids", setv(0, V + 7), pe.PE_CHECK_TOKEN_ID)
    mutated("target_pos", setv(0, -1), pe.PE_CHECK_POSITION, exact=False)
    mutated("target_pos", lambda a: (a.__setitem__(L0 - 1, a[L0 - 1] + 5), a)[1], pe.PE_CHECK_POSITION, exact=False)
    mutated("query_lens", setv(0, 0), pe.PE_CHECK_QUERY_LEN, exact=False)
    mutated("query_lens", setv(wl.c - 1, int(b.query_lens[-1]) + 1), pe.PE_CHECK_QUERY_LEN, exact=False)
    mutated("block_table", lambda a: (a.__setitem__((0, 0), -1), a)[1], pe.PE_CHECK_BLOCK_TABLE)
    mutated("block_table", lambda a: a[:, :1], pe.PE_CHECK_BLOCK_TABLE, exact=False)
    # checks accumulate into a caller word
    e = torch.full((1,), pe.PE_CHECK_POSITION, dtype=torch.int32, device=DEV)
    pe.check_verified_batch(model, wl.K, d["query_lens"], d["target_ids"], d["target_pos"], d["num_accepted"],
                            d["bonus_ids"], d["block_table"], error_bits=e)
    torch.cuda.synchronize()
    assert int(e.cpu()[0]) == pe.PE_CHECK_POSITION
