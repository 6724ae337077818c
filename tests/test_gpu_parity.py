"""GPU parity: the HIP path through the C ABI vs the CPU oracle, same inputs.

Bars: integer outputs, masks, slot mappings, cache bytes outside the written
slots and the placed hidden rows are bit-exact; logits within max-abs 1e-5
(fp32 drafter) or 2e-2 (bf16 drafter); every draft token is an oracle argmax
up to that tolerance; written KV entries match the oracle's rounded values.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.device import from_torch, upload_batch
from gpu_harness import (LOGIT_TOL, check_cache, check_prepare_exact, check_tokens, device_model, gpu_round,
                         host_weights)
from conftest import make_verified_batch

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _oracle_meta(spec, b):
    return oracle.expand_batch(b.query_lens, b.target_ids, b.target_pos, b.num_accepted, b.bonus_ids,
                               b.block_table, b.K, spec.mask_token_id, spec.block_size)


# ----------------------------------------------------------------------------- expansion
@pytest.mark.parametrize("name", ["tiny-fp32-c2-k3", "prep-bf16-c64-k7-h2880", "gptoss20b-bf16-c64-k7"])
def test_prepare_bit_exact(name):
    wl = synth.WORKLOADS[name]
    _say(f"prepare {name}")
    spec = wl.model
    b = synth.make_batch(wl, with_cache=False)
    w = host_weights(spec, wl.wseed, True)
    model = device_model(spec, wl.wseed, True)
    db = upload_batch(b, "cuda:0")
    import drafting_draft_expand_amd as pe
    prep = pe.prepare_draft_batch(model, wl.K, db["query_lens"], db["target_ids"], db["target_pos"],
                                  db["num_accepted"], db["bonus_ids"], db["target_hidden"], db["block_table"])
    torch.cuda.synchronize()
    meta = _oracle_meta(spec, b)
    hd = oracle.scatter_broadcast(b.target_hidden, meta["hidden_map"], meta["is_masked"], w["h_shared"], b.N)
    check_prepare_exact(prep, meta, hd)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_prepare_sweep_bit_exact(dtype):
    """Every (L, a) with L <= 8 at K in {1, 3, 7}, several sequences per batch."""
    import drafting_draft_expand_amd as pe
    spec = synth.ModelSpec(hidden=64, vocab=512, n_layers=0, n_q=1, n_kv=1, head_dim=16, inter=8, dtype=dtype)
    rng = np.random.default_rng(7)
    hs = synth.store(rng.standard_normal(64).astype(np.float32), dtype)
    model = pe.DraftModel(64, 512, 0, 1, 1, 16, 8, dtype, {"h_shared": synth.device.to_torch(hs)})
    for K in (1, 3, 7):
        _say(f"prepare sweep dtype={dtype} K={K}")
        Ls = [L for L in range(1, 9) for _ in range(L)]
        As = [a for L in range(1, 9) for a in range(L)]
        vb = make_verified_batch(rng, Ls, As, K, vocab=512, H=64)
        th = synth.store(vb["target_hidden"], dtype)
        t = lambda x: synth.device.to_torch(x)  # noqa: E731
        prep = pe.prepare_draft_batch(model, K, t(vb["query_lens"]), t(vb["target_ids"]), t(vb["target_pos"]),
                                      t(vb["num_accepted"]), t(vb["bonus_ids"]), t(th), t(vb["block_table"]))
        torch.cuda.synchronize()
        meta = oracle.expand_batch(vb["query_lens"], vb["target_ids"], vb["target_pos"], vb["num_accepted"],
                                   vb["bonus_ids"], vb["block_table"], K, 511, 16)
        hd = oracle.scatter_broadcast(th, meta["hidden_map"], meta["is_masked"], hs, len(meta["draft_ids"]))
        check_prepare_exact(prep, meta, hd)


# ----------------------------------------------------------------------------- forward
def _forward_case(wl, seqs=None, batch=None, model_spec=None, wseed=None, pack=True):
    spec = model_spec or wl.model
    wseed = wl.wseed if wseed is None else wseed
    _say(f"forward {wl.name} seqs={seqs} pack={pack}")
    w = host_weights(spec, wseed)
    model = device_model(spec, wseed, pack=pack)
    b = synth.make_batch(wl) if batch is None else batch
    db = upload_batch(b, "cuda:0")
    prep, tokens, logits, gap = gpu_round(model, db, b.K)
    _say(f"  gpu done, oracle for seqs={seqs}")
    ref = oracle.parallel_draft_step(spec, w, b, precision="mirror", seqs=seqs)
    check_prepare_exact(prep, ref["meta"], ref["draft_hidden"])
    fw = ref["forward"]
    sel = fw["seqs"]
    K = b.K
    rows = np.concatenate([np.arange(i * K, (i + 1) * K) for i in sel])
    g_logits = from_torch(logits)[rows]
    o_logits = fw["logits"].reshape(len(rows), -1)
    tol = LOGIT_TOL[spec.dtype]
    err = np.max(np.abs(g_logits - o_logits))
    if spec.dtype == "bf16":
        # reported beside the gate: the distance to the unrounded float64 pass
        ref64 = oracle.parallel_draft_step(spec, w, b, precision="fp64", seqs=seqs)["forward"]
        err64 = np.max(np.abs(g_logits - ref64["logits"].reshape(len(rows), -1)))
        _say(f"  max|dlogit| = {err:.3e} vs the bf16-operand oracle (gate, tol {tol}); "
             f"{err64:.3e} vs the pure fp64 oracle (reported)")
        del ref64
    else:
        _say(f"  max|dlogit| = {err:.3e} (tol {tol})")
    assert np.isfinite(g_logits).all()
    assert err <= tol
    g_tok = from_torch(tokens).reshape(-1)[rows]
    exact = check_tokens(g_tok, o_logits, tol)
    _say(f"  tokens identical to oracle argmax: {exact:.3f}")
    # gap reported by the GPU is consistent with its own logits
    g_gap = from_torch(gap)[rows]
    srt = np.sort(g_logits, axis=1)
    np.testing.assert_allclose(g_gap, srt[:, -1] - srt[:, -2], rtol=0, atol=1e-6)
    slots = from_torch(prep["slot_mapping"])
    check_cache(spec, b.k_cache, b.v_cache, [from_torch(k) for k in db["k_cache"]],
                [from_torch(v) for v in db["v_cache"]], slots, fw["cache_writes"], spec.dtype)
    return dict(prep=prep, tokens=from_torch(tokens), oracle=ref, batch=b)


def test_forward_tiny_fp32():
    _forward_case(synth.WORKLOADS["tiny-fp32-c2-k3"])


def test_forward_tiny_fp32_two_layers_ragged():
    spec = synth.ModelSpec(hidden=96, vocab=300, n_layers=2, n_q=6, n_kv=2, head_dim=32, inter=160, dtype="fp32")
    wl = synth.Workload("two-layer", spec, c=5, K=4, ctx_lo=0, ctx_hi=70, accept_hi=4, seed=12)
    _forward_case(wl)


@pytest.mark.parametrize("K", [1, 2, 5])
def test_forward_depths_fp32(K):
    spec = synth.TINY
    wl = synth.Workload(f"tiny-k{K}", spec, c=3, K=K, ctx_lo=1, ctx_hi=40, accept_hi=K, seed=20 + K, weight_seed=0)
    _forward_case(wl)


def test_forward_prefill_like_fp32():
    spec = synth.TINY
    wl = synth.Workload("tiny-prefill", spec, c=3, K=3, ctx_lo=0, ctx_hi=20, accept_hi=3, seed=31, weight_seed=0)
    b = synth.make_batch(wl, accepted=np.full(3, 3))
    _forward_case(wl, batch=b)


@pytest.mark.parametrize("dtype,d", [("fp32", 64), ("fp32", 128), ("bf16", 16), ("bf16", 32)])
def test_forward_head_dims(dtype, d):
    spec = synth.ModelSpec(hidden=128, vocab=700, n_layers=1, n_q=4, n_kv=2, head_dim=d, inter=256, dtype=dtype)
    wl = synth.Workload(f"hd{d}-{dtype}", spec, c=3, K=4, ctx_lo=5, ctx_hi=150, accept_hi=4, seed=50 + d)
    _forward_case(wl)


def test_forward_bf16_few_rows_unfused():
    """c=1, K=3: 6 draft rows with a hidden size that is not a multiple of 32
    (200), so every projection takes the VALU path with the separate gather /
    norm / RoPE kernels."""
    spec = synth.ModelSpec(hidden=200, vocab=1000, n_layers=1, n_q=8, n_kv=2, head_dim=64, inter=512)
    wl = synth.Workload("few-rows-bf16", spec, c=1, K=3, ctx_lo=30, ctx_hi=90, accept_hi=3, seed=43)
    _forward_case(wl)


@pytest.mark.parametrize("pack", [True, False])
@pytest.mark.parametrize("K", [1, 3])
def test_forward_bf16_fewest_rows_mfma(K, pack):
    """One sequence, 2 and 6 draft rows: the weight-streaming MFMA projections
    with most of the 16-row fragment padding, while the LM head over 1 and 3
    sampled rows stays on the LDS kernel."""
    spec = synth.ModelSpec(hidden=544, vocab=1000, n_layers=1, n_q=6, n_kv=2, head_dim=32, inter=5120)
    wl = synth.Workload(f"fewest-rows-mfma-k{K}", spec, c=1, K=K, ctx_lo=40, ctx_hi=200, accept_hi=K, seed=70 + K)
    _forward_case(wl, pack=pack)


@pytest.mark.parametrize("pack", [True, False])
@pytest.mark.parametrize("K", [5, 8])
def test_forward_bf16_few_rows_mfma(K, pack):
    """One sequence, 9..16 draft rows: the weight-streaming MFMA projections,
    on the packed copy (tile groups of 1, 2 and 4 with ragged ends, fc split
    over K into partials that the RMSNorm adds up) and on row-major weights."""
    spec = synth.ModelSpec(hidden=544, vocab=1000, n_layers=1, n_q=6, n_kv=2, head_dim=32, inter=5120)
    wl = synth.Workload(f"few-rows-mfma-k{K}", spec, c=1, K=K, ctx_lo=40, ctx_hi=200, accept_hi=K, seed=60 + K)
    _forward_case(wl, pack=pack)


def test_forward_two_layer_bf16_mfma_splits():
    """Two layers at 14 rows, every projection split over K where allowed: the
    second layer's first RMSNorm adds the first layer's down-projection
    partials to the residual rows."""
    spec = synth.ModelSpec(hidden=1024, vocab=700, n_layers=2, n_q=8, n_kv=2, head_dim=64, inter=2048)
    wl = synth.Workload("two-layer-mfma", spec, c=1, K=7, ctx_lo=20, ctx_hi=300, accept_hi=7, seed=66)
    _forward_case(wl)


def test_forward_qwen_c1_full():
    """Qwen-shaped drafter at one sequence: 14 rows, so the packed few-row
    projections with 128-dim heads (q/k/v tiles in pairs, RoPE pairs 64 apart)."""
    wl = synth.Workload("qwen3coder30b-bf16-c1-k7", synth.QWEN3CODER30B, c=1, K=7, ctx_lo=1024, ctx_hi=3000,
                        accept_hi=7, seed=81, weight_seed=4)
    _forward_case(wl)


def test_forward_small_bf16():
    spec = synth.ModelSpec(hidden=256, vocab=1000, n_layers=1, n_q=8, n_kv=2, head_dim=64, inter=512)
    wl = synth.Workload("small-bf16", spec, c=6, K=5, ctx_lo=10, ctx_hi=300, accept_hi=5, seed=41)
    _forward_case(wl)


@pytest.mark.parametrize("pack", [True, False])
def test_forward_bf16_many_sampled_rows(pack):
    """200 sampled rows over a 1000-token vocab: with the tile-major LM-head copy
    the prefetching ring kernel (two 128-row tiles, the second ragged; the last
    256-row vocab group mostly padding), else the register-staged GEMM.  About
    300 draft rows, so the layer projections run the ring kernel on row-major
    weights (K split for the residual-writing ones)."""
    spec = synth.ModelSpec(hidden=256, vocab=1000, n_layers=1, n_q=8, n_kv=2, head_dim=64, inter=512)
    wl = synth.Workload("many-sampled-bf16", spec, c=40, K=5, ctx_lo=10, ctx_hi=200, accept_hi=5, seed=47)
    _forward_case(wl, pack=pack)


def _random_case(seed):
    """A bf16 drafter and batch drawn from a seeded generator: widths on and off
    the 64-wide K grid, 16- to 128-dim heads, GQA groups of 1-8, one or two
    layers, 1-40 sequences, K = 1-8, contexts up to ~1000 tokens, packed or
    not; the shape fixes which projection, attention and LM-head kernels run."""
    r = np.random.default_rng(np.random.SeedSequence([seed, 9901]))
    d = int(r.choice([16, 32, 64, 128]))
    n_kv = int(r.choice([1, 2, 4]))
    n_q = n_kv * int(r.choice([1, 2, 4, 8]))
    spec = synth.ModelSpec(hidden=int(r.choice([64, 128, 160, 192, 256, 288, 320, 384, 416, 448, 512])),
                           vocab=int(r.integers(300, 3001)), n_layers=int(r.choice([1, 2])), n_q=n_q, n_kv=n_kv,
                           head_dim=d, inter=int(r.choice([96, 128, 224, 256, 320, 352, 448, 512, 640])))
    K = int(r.integers(1, 9))
    lo = int(r.integers(0, 201))
    wl = synth.Workload(f"random-{seed}", spec, c=int(r.integers(1, 41)), K=K, ctx_lo=lo,
                        ctx_hi=lo + int(r.integers(0, 801)), accept_hi=K, seed=2000 + seed)
    return wl, bool(r.integers(0, 2))


@pytest.mark.parametrize("seed", range(32))
def test_forward_bf16_random_shapes(seed):
    """Seeded sweep over drafter and batch shapes (see _random_case), each
    against the oracle like the fixed cases."""
    wl, pack = _random_case(seed)
    s = wl.model
    _say(f"random case {seed}: H={s.hidden} V={s.vocab} layers={s.n_layers} q/kv={s.n_q}/{s.n_kv} d={s.head_dim} "
         f"I={s.inter} c={wl.c} K={wl.K} ctx={wl.ctx_lo}..{wl.ctx_hi} pack={pack}")
    _forward_case(wl, pack=pack)


@pytest.mark.parametrize("c", [2, 3, 20, 32, 33])
def test_forward_bf16_row_count_boundaries(c):
    """Draft-row counts at the projection path boundaries (K = 7, so c * 8
    rows and c * 7 sampled rows): 16 rows (few-row kernels), 24 (the 64 x 64
    ring with 64-deep stages), 160 (a 140-row LM head whose second 128-row tile
    has an all-padding wave pair), 256 (the last row count on the 64 x 64 ring)
    and 264 (the 128-row ring tiles, on tile-major operands for packed models)."""
    spec = synth.ModelSpec(hidden=256, vocab=1000, n_layers=1, n_q=8, n_kv=2, head_dim=64, inter=512)
    wl = synth.Workload(f"rows-c{c}", spec, c=c, K=7, ctx_lo=10, ctx_hi=300, accept_hi=7, seed=120 + c)
    _forward_case(wl)


def test_forward_bf16_more_than_512_sequences():
    """520 sequences at K = 2: the ring attention past its KV-length ranking
    (at most 512 sequences; launch order beyond), 2080 draft rows on the
    tile-major path (16.25 row groups) and 1040 sampled rows for the LM head
    (nine 128-row tiles, the last one mostly padding)."""
    spec = synth.ModelSpec(hidden=128, vocab=600, n_layers=1, n_q=4, n_kv=2, head_dim=64, inter=256)
    wl = synth.Workload("many-seqs-c520", spec, c=520, K=2, ctx_lo=0, ctx_hi=60, accept_hi=2, seed=777)
    _forward_case(wl)


def test_forward_bf16_widths_off_the_64_grid():
    """hidden 288 at 160 rows: q/k/v and gate/up (K = 288) are off the 64-wide
    K grid of the tiled kernels, so the pass takes the unfused plan: the fc
    input built by its own kernel and projected on the 64 x 64 ring (K = 576),
    q/k/v and gate/up on the LDS kernel with the rotation and the KV write in
    their own kernel, o and down on the 64 x 64 ring."""
    spec = synth.ModelSpec(hidden=288, vocab=700, n_layers=1, n_q=4, n_kv=2, head_dim=64, inter=320)
    wl = synth.Workload("odd-width-bf16", spec, c=20, K=7, ctx_lo=10, ctx_hi=300, accept_hi=7, seed=131)
    _forward_case(wl)


@pytest.mark.parametrize("d", [64, 128])
def test_forward_bf16_mid_rows(d):
    """200 draft rows (four 64-row tiles, the last ragged): the LDS-DMA ring
    with 64-deep stages on 64 x 64 tiles for q/k/v with RoPE and gate/up, and
    K split into partials for the residual projections; the fc input is
    gathered by the register-staged tiled GEMM."""
    spec = synth.ModelSpec(hidden=256, vocab=900, n_layers=1, n_q=4, n_kv=2, head_dim=d, inter=320)
    wl = synth.Workload(f"mid-rows-d{d}", spec, c=20, K=5, ctx_lo=10, ctx_hi=200, accept_hi=5, seed=95 + d)
    _forward_case(wl)


def test_forward_bf16_many_rows_ragged():
    """About 300 draft rows on a drafter whose widths are not multiples of the
    ring kernel's tiles: hidden 320 (two 256-column tiles, the second ragged),
    q/k/v 448 columns in 128-column tiles, gate/up 448 outputs in 128-column
    tiles, ragged last 128-row tile."""
    spec = synth.ModelSpec(hidden=320, vocab=700, n_layers=1, n_q=5, n_kv=1, head_dim=64, inter=448)
    wl = synth.Workload("many-rows-ragged-bf16", spec, c=40, K=5, ctx_lo=10, ctx_hi=150, accept_hi=5, seed=48)
    _forward_case(wl)


@pytest.mark.parametrize("d", [64, 128])
def test_forward_bf16_equal_kv_lengths(d):
    """Every sequence with the same KV length (equal contexts, nothing accepted):
    the attention kernels order sequences longest first and fall back to the
    sequence index on ties; each sequence must still be attended exactly once."""
    spec = synth.ModelSpec(hidden=256, vocab=600, n_layers=1, n_q=4, n_kv=2, head_dim=d, inter=384)
    wl = synth.Workload(f"equal-kv-d{d}", spec, c=9, K=3, ctx_lo=200, ctx_hi=200, accept_hi=0, seed=90 + d)
    _forward_case(wl)


def test_forward_bf16_d128_mixed_contexts():
    """bf16 128-dim heads over contexts from empty to several hundred tokens:
    KV splits with no tile, a partial last tile, sequences in longest-first
    order."""
    spec = synth.ModelSpec(hidden=256, vocab=600, n_layers=1, n_q=4, n_kv=2, head_dim=128, inter=384)
    wl = synth.Workload("mixed-kv-d128", spec, c=11, K=4, ctx_lo=0, ctx_hi=900, accept_hi=4, seed=93)
    _forward_case(wl)


@pytest.mark.parametrize("d", [64, 128])
def test_forward_bf16_page_list_beyond_lds(d):
    """A block table wider than a KV split's page list can hold in LDS (17 300
    columns, those past each sequence's pages unused): attention takes the
    register-staged kernel that reads the block table directly."""
    spec = synth.ModelSpec(hidden=256, vocab=600, n_layers=1, n_q=4, n_kv=2, head_dim=d, inter=384)
    wl = synth.Workload(f"wide-table-d{d}", spec, c=3, K=3, ctx_lo=50, ctx_hi=400, accept_hi=3, seed=97 + d)
    b = synth.make_batch(wl)
    extra = 17300 - b.block_table.shape[1]
    b.block_table = np.ascontiguousarray(
        np.concatenate([b.block_table, np.repeat(b.block_table[:, :1], extra, axis=1)], axis=1))
    _forward_case(wl, batch=b)


def test_forward_gptoss_c1_full():
    _forward_case(synth.WORKLOADS["gptoss20b-bf16-c1-k7"])


def test_forward_gptoss_c64_full():
    """All 64 sequences (448 sampled rows, every logit) and every KV entry the
    pass writes, at the benchmark's c=64 shape."""
    _forward_case(synth.WORKLOADS["gptoss20b-bf16-c64-k7"])


def test_forward_gptoss_c64_k8_full():
    """All 64 sequences at K=8: 1024 draft rows (eight whole 128-row groups of
    the tile-major operands) and 512 sampled rows (four LM-head row tiles, none
    of them padded)."""
    _forward_case(synth.WORKLOADS["gptoss20b-bf16-c64-k8"])


@pytest.mark.parametrize("K", [3, 5, 7])
def test_forward_qwen_c16_full(K):
    """All 16 sequences of the Qwen-shaped drafter at each depth."""
    _forward_case(synth.WORKLOADS[f"qwen3coder30b-bf16-c16-k{K}"])


@pytest.mark.parametrize("name", ["gptoss20b-bf16-c1-k7", "small-bf16-c2", "gptoss20b-bf16-c64-k7"])
def test_forward_without_logits_matches(name):
    """The token-only pass (what the bench times) picks the same tokens and
    top-2 gaps as the pass that also writes the logits."""
    if name == "small-bf16-c2":
        spec = synth.ModelSpec(hidden=256, vocab=1000, n_layers=1, n_q=8, n_kv=2, head_dim=64, inter=512)
        wl = synth.Workload(name, spec, c=2, K=7, ctx_lo=10, ctx_hi=300, accept_hi=7, seed=44)
    else:
        wl = synth.WORKLOADS[name]
    _say(f"no-logits path {wl.name}")
    model = device_model(wl.model, wl.wseed)
    b = synth.make_batch(wl)
    db = upload_batch(b, "cuda:0")
    _, tok_a, _, gap_a = gpu_round(model, db, b.K, want_logits=True)
    tok_a, gap_a = from_torch(tok_a).copy(), from_torch(gap_a).copy()
    _, tok_b, _, gap_b = gpu_round(model, db, b.K, want_logits=False)
    assert np.array_equal(tok_a, from_torch(tok_b))
    assert np.array_equal(gap_a, from_torch(gap_b))


@pytest.mark.parametrize("name", ["gptoss20b-bf16-c64-k7", "qwen3coder30b-bf16-c16-k5", "tiny-fp32-c2-k3"])
def test_compact_layout(name):
    """Compacted layout (rejected rows dropped): the expansion is bit-exact
    against the oracle's, the pass over it matches the oracle's compacted pass
    (logits within tolerance, tokens oracle argmaxes), and it returns exactly
    the fixed layout's tokens, gaps and logits on the same batch."""
    import drafting_draft_expand_amd as pe
    wl = synth.WORKLOADS[name]
    spec = wl.model
    _say(f"compact layout {wl.name}")
    w = host_weights(spec, wl.wseed)
    model = device_model(spec, wl.wseed)
    b = synth.make_batch(wl)
    db = upload_batch(b, "cuda:0")
    meta = oracle.expand_batch(b.query_lens, b.target_ids, b.target_pos, b.num_accepted, b.bonus_ids,
                               b.block_table, b.K, spec.mask_token_id, spec.block_size, compact=True)
    hd = oracle.scatter_broadcast(b.target_hidden, meta["hidden_map"], meta["is_masked"], w["h_shared"],
                                  len(meta["draft_ids"]))
    outs = {}
    for compact in (False, True):
        prep = pe.prepare_draft_batch(model, b.K, db["query_lens"], db["target_ids"], db["target_pos"],
                                      db["num_accepted"], db["bonus_ids"], db["target_hidden"], db["block_table"],
                                      compact=compact)
        logits = torch.empty((wl.c * b.K, spec.vocab), dtype=torch.float32, device="cuda:0")
        gap = torch.empty(wl.c * b.K, dtype=torch.float32, device="cuda:0")
        tokens = pe.draft_forward(model, prep, db["block_table"], db["k_cache"], db["v_cache"], logits=logits,
                                  top2_gap=gap)
        torch.cuda.synchronize()
        if compact:
            check_prepare_exact(prep, meta, hd)
        outs[compact] = (from_torch(tokens).copy(), from_torch(gap).copy(), from_torch(logits).copy())
    live = int(meta["cu_draft"][-1])
    _say(f"  live rows {live} of {len(meta['draft_ids'])}")
    ref = oracle.parallel_draft_step(spec, w, b, precision="mirror", compact=True)["forward"]
    o_logits = ref["logits"].reshape(wl.c * b.K, -1)
    tol = LOGIT_TOL[spec.dtype]
    err = np.max(np.abs(outs[True][2] - o_logits))
    _say(f"  compacted pass: max|dlogit| = {err:.3e} vs the oracle (tol {tol})")
    assert err <= tol
    check_tokens(outs[True][0].reshape(-1), o_logits, tol)
    for a_, b_ in zip(outs[False], outs[True]):
        assert np.array_equal(a_, b_)


# ----------------------------------------------------------------------------- acceptance
@pytest.mark.parametrize("name", ["tiny-fp32-c2-k3", "qwen3coder30b-bf16-c16-k7"])
def test_accept_matches_oracle(name):
    import drafting_draft_expand_amd as pe
    wl = synth.WORKLOADS[name]
    rng = np.random.default_rng(3)
    for trial in range(4):
        c = [1, wl.c, 64, 1000][trial]
        drafts = rng.integers(0, 50, size=(c, wl.K)).astype(np.int32)
        u = rng.random((c, wl.K))
        alt = rng.integers(0, wl.model.vocab - 2, size=(c, wl.K + 1))
        tgt = synth.target_tokens_from_drafts(drafts, u, alt, wl.agree_probs(), wl.model.vocab)
        acc, bonus = pe.accept(synth.device.to_torch(drafts), synth.device.to_torch(tgt))
        torch.cuda.synchronize()
        oa, ob = oracle.accept(drafts, tgt)
        assert np.array_equal(from_torch(acc), oa) and np.array_equal(from_torch(bonus), ob)


def test_round_trip_accept_on_gpu_drafts():
    """Drafts from the GPU pass, targets from the synthetic agreement process:
    GPU acceptance equals the oracle's on the same arrays."""
    import drafting_draft_expand_amd as pe
    wl = synth.WORKLOADS["tiny-fp32-c2-k3"]
    model = device_model(wl.model, wl.wseed)
    b = synth.make_batch(wl)
    db = upload_batch(b, "cuda:0")
    _, tokens, _, _ = gpu_round(model, db, b.K, want_logits=False)
    u, alt = synth.make_agreement_draws(wl)
    tgt = synth.target_tokens_from_drafts(from_torch(tokens), u, alt, wl.agree_probs(), wl.model.vocab)
    acc, bonus = pe.accept(tokens, synth.device.to_torch(tgt))
    torch.cuda.synchronize()
    oa, ob = oracle.accept(from_torch(tokens), tgt)
    assert np.array_equal(from_torch(acc), oa) and np.array_equal(from_torch(bonus), ob)
