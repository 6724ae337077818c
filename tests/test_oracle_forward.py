"""Pins of the oracle's drafter pass (CPU only).

Each building block is compared with an independent library routine or a
closed form, the whole pass with an independent torch composition, and the
method-level properties with metamorphic checks:

* RMSNorm vs torch.nn.functional.rms_norm; SiLU vs torch silu;
* rotate-half RoPE vs multiplication by e^{i p theta_j} on complex pairs;
* paged GQA attention vs torch scaled_dot_product_attention (enable_gqa) with
  an explicit position mask; one visible key returns its value exactly;
* the whole float64 pass vs a torch composition that rebuilds contiguous
  KV from the block table position by position;
* MASK rows see identical inputs emb(mask) + h_shared (Input_i equation);
* the first draft token does not depend on K (later rows are causally after);
* physical block relabelling, sequence permutation and perturbing rejected
  rows leave the valid outputs unchanged; reading past the KV length would
  hit NaN canaries, and the result stays finite;
* a RoPE position off by one (the pitfall named in section 6.1 of the
  DSpark survey page) changes the logits far beyond tolerance;
* argmax ties resolve to the lowest vocabulary id.
"""

import copy

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.peagle_oracle as po
import synth
from conftest import make_verified_batch

f64 = torch.float64


def _t(x):
    return torch.tensor(np.asarray(x, dtype=np.float32), dtype=f64)


# ----------------------------------------------------------------------------- blocks
def test_rms_norm_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 64)) * 3
    g = rng.standard_normal(64)
    ref = F.rms_norm(torch.tensor(x), (64,), weight=torch.tensor(g), eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.rms_norm(x, g, 1e-6), ref, rtol=1e-13, atol=1e-13)


def test_silu_matches_torch():
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(oracle.silu(z), F.silu(torch.tensor(z)).numpy(), rtol=1e-13, atol=1e-300)


def _rope_complex(x, pos, theta):
    d = x.shape[-1]
    half = d // 2
    z = torch.complex(torch.tensor(x[..., :half]), torch.tensor(x[..., half:]))
    j = torch.arange(half, dtype=f64)
    ang = torch.tensor(pos, dtype=f64)[:, None] * torch.pow(torch.tensor(theta, dtype=f64), -2.0 * j / d)
    r = z * torch.polar(torch.ones_like(ang), ang)[:, None, :]
    return torch.cat([r.real, r.imag], dim=-1).numpy()


@pytest.mark.parametrize("d", [16, 64, 128])
def test_rope_matches_complex_rotation(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((9, 3, d))
    pos = rng.integers(0, 16384, size=9)
    got = oracle.rope_rotate_half(x, pos, 10000.0)
    np.testing.assert_allclose(got, _rope_complex(x, pos, 10000.0), rtol=1e-10, atol=1e-10)
    # rotation preserves norms; scores depend only on the position difference
    np.testing.assert_allclose(np.linalg.norm(got, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
    q, k = x[:1], x[1:2]
    s1 = np.sum(oracle.rope_rotate_half(q, [100], 1e4) * oracle.rope_rotate_half(k, [37], 1e4))
    s2 = np.sum(oracle.rope_rotate_half(q, [1100], 1e4) * oracle.rope_rotate_half(k, [1037], 1e4))
    assert abs(s1 - s2) < 1e-9


def test_attention_matches_sdpa_gqa():
    rng = np.random.default_rng(1)
    rows, nq, nkv, d, L = 6, 8, 2, 16, 29
    q = rng.standard_normal((rows, nq, d))
    k = rng.standard_normal((L, nkv, d))
    v = rng.standard_normal((L, nkv, d))
    qpos = np.array([3, 10, 20, 28, 28, 0])
    mask = torch.tensor(np.arange(L)[None, :] <= qpos[:, None])
    ref = F.scaled_dot_product_attention(torch.tensor(q).transpose(0, 1), torch.tensor(k).transpose(0, 1),
                                         torch.tensor(v).transpose(0, 1), attn_mask=mask, enable_gqa=True)
    got = oracle.paged_attention(q, qpos, k, v)
    np.testing.assert_allclose(got, ref.transpose(0, 1).numpy(), rtol=1e-12, atol=1e-12)


def test_attention_single_visible_key_returns_value():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 4, 16))
    k = rng.standard_normal((5, 2, 16))
    v = rng.standard_normal((5, 2, 16))
    out = oracle.paged_attention(q, np.array([0]), k, v)
    np.testing.assert_array_equal(out[0, :2], np.repeat(v[0:1, 0], 2, axis=0))
    np.testing.assert_array_equal(out[0, 2:], np.repeat(v[0:1, 1], 2, axis=0))


# ----------------------------------------------------------------------------- whole pass
def _torch_pass(spec, w, meta, hd, bt, kc, vc):
    """Independent float64 composition of the drafter pass (library routines only)."""
    H, nq, nkv, d, bs = spec.hidden, spec.n_q, spec.n_kv, spec.head_dim, spec.block_size
    ids = torch.tensor(meta["draft_ids"])
    pos = np.asarray(meta["draft_pos"])
    x = F.linear(torch.cat([_t(w["embed"])[ids], _t(hd)], dim=1), _t(w["w_fc"]))
    for li, lw in enumerate(w["layers"]):
        a = F.rms_norm(x, (H,), weight=_t(lw["ln1"]), eps=spec.rms_eps)
        q = F.linear(a, _t(lw["wq"])).view(-1, nq, d).numpy()
        k = F.linear(a, _t(lw["wk"])).view(-1, nkv, d).numpy()
        v = F.linear(a, _t(lw["wv"])).view(-1, nkv, d)
        q = torch.tensor(_rope_complex(q, pos, spec.rope_theta))
        k = torch.tensor(_rope_complex(k, pos, spec.rope_theta))
        kcache, vcache = _t(kc[li]).clone(), _t(vc[li]).clone()
        for r, sl in enumerate(meta["slot_mapping"]):
            if sl >= 0:
                kcache[sl // bs, :, sl % bs] = k[r]
                vcache[sl // bs, :, sl % bs] = v[r]
        attn = torch.zeros(len(ids), nq, d, dtype=f64)
        for i in range(len(meta["kv_lens"])):
            rows = np.arange(meta["cu_draft"][i], meta["cu_draft"][i + 1])
            n = int(meta["kv_lens"][i])
            keys = torch.stack([kcache[bt[i][p // bs], :, p % bs] for p in range(n)])
            vals = torch.stack([vcache[bt[i][p // bs], :, p % bs] for p in range(n)])
            mask = torch.tensor(np.arange(n)[None, :] <= pos[rows][:, None])
            o = F.scaled_dot_product_attention(q[rows].transpose(0, 1), keys.transpose(0, 1),
                                               vals.transpose(0, 1), attn_mask=mask, enable_gqa=True)
            attn[rows] = o.transpose(0, 1)
        x = x + F.linear(attn.reshape(len(ids), nq * d), _t(lw["wo"]))
        m = F.rms_norm(x, (H,), weight=_t(lw["ln2"]), eps=spec.rms_eps)
        x = x + F.linear(F.silu(F.linear(m, _t(lw["w_gate"]))) * F.linear(m, _t(lw["w_up"])), _t(lw["w_down"]))
    f = F.rms_norm(x[torch.tensor(meta["sample_idx"])], (H,), weight=_t(w["ln_f"]), eps=spec.rms_eps)
    return F.linear(f, _t(w["w_lm"])).numpy()


def _meta(spec, b):
    return oracle.expand_batch(b.query_lens, b.target_ids, b.target_pos, b.num_accepted, b.bonus_ids,
                               b.block_table, b.K, spec.mask_token_id, spec.block_size)


def _run(spec, w, b, precision="fp64", **kw):
    return oracle.parallel_draft_step(spec, w, b, precision=precision, **kw)


def test_whole_pass_matches_torch_composition(tiny):
    wl, w, b = tiny
    r = _run(wl.model, w, b)
    ref = _torch_pass(wl.model, w, r["meta"], r["draft_hidden"], b.block_table, b.k_cache, b.v_cache)
    got = r["forward"]["logits"].reshape(ref.shape)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)
    assert np.array_equal(r["forward"]["tokens"].reshape(-1), ref.argmax(axis=1))


def test_two_layers_match_torch_composition():
    spec = synth.ModelSpec(hidden=32, vocab=97, n_layers=2, n_q=4, n_kv=1, head_dim=8, inter=48, dtype="fp32")
    wl = synth.Workload("t2", spec, c=3, K=4, ctx_lo=5, ctx_hi=40, accept_hi=4, seed=11)
    w = synth.make_weights(spec, 11)
    b = synth.make_batch(wl)
    r = _run(spec, w, b)
    ref = _torch_pass(spec, w, r["meta"], r["draft_hidden"], b.block_table, b.k_cache, b.v_cache)
    np.testing.assert_allclose(r["forward"]["logits"].reshape(ref.shape), ref, rtol=1e-10, atol=1e-12)


def test_mask_rows_share_one_input(tiny):
    wl, w, b = tiny
    r = _run(wl.model, w, b)
    meta, inter = r["meta"], r["forward"]["intermediates"]
    xm = inter["x_fc"][meta["is_masked"].astype(bool)]
    assert len(xm) == b.c * (b.K - 1)
    assert np.all(xm == xm[0])
    emb = oracle.decode(w["embed"][wl.model.mask_token_id], "fp32")
    hs = oracle.decode(w["h_shared"], "fp32")
    np.testing.assert_allclose(xm[0], oracle.decode(w["w_fc"], "fp32") @ np.concatenate([emb, hs]), rtol=1e-12)


def test_all_outputs_finite_despite_nan_canaries(tiny):
    wl, w, b = tiny
    # canaries sit in every slot the pass must write and beyond the KV length
    assert np.isnan(b.k_cache[0]).any()
    r = _run(wl.model, w, b)
    assert np.isfinite(r["forward"]["logits"]).all()


def test_first_draft_token_independent_of_depth():
    spec = synth.TINY
    w = synth.make_weights(spec, 5)
    rng = np.random.default_rng(5)
    vb = make_verified_batch(rng, [4, 6, 2], [1, 5, 0], 3, vocab=spec.vocab, ctx=[16, 3, 30], H=spec.hidden)
    outs = {}
    for K in (1, 2, 5):
        need = [int(-(-(vb["context"][i] + vb["query_lens"][i] + K - 1) // 16)) for i in range(3)]
        b = _verified_to_batch(spec, vb, K, max(need))
        outs[K] = _run(spec, w, b)["forward"]
    for K in (2, 5):
        assert np.array_equal(outs[K]["tokens"][:, 0], outs[1]["tokens"][:, 0])
        np.testing.assert_allclose(outs[K]["logits"][:, 0], outs[1]["logits"][:, 0], rtol=1e-12, atol=1e-14)


def _verified_to_batch(spec, vb, K, min_blocks):
    rng = np.random.default_rng(77)
    c = len(vb["query_lens"])
    bs = spec.block_size
    need = [int(-(-(vb["context"][i] + vb["query_lens"][i] + K - 1) // bs)) for i in range(c)]
    total = sum(need)
    perm = rng.permutation(total).astype(np.int32)
    bt = np.full((c, max(need)), total, np.int32)
    o = 0
    for i in range(c):
        bt[i, :need[i]] = perm[o:o + need[i]]
        o += need[i]
    shape = (total + 1, spec.n_kv, bs, spec.head_dim)
    # cached context values are a function of (sequence, position) only, so the
    # same verified batch at different K sees the same context
    kc = np.full(shape, np.nan, np.float32)
    vc = np.full(shape, np.nan, np.float32)
    for i in range(c):
        for p in range(int(vb["context"][i])):
            g = np.random.default_rng([i, p])
            kc[bt[i, p // bs], :, p % bs] = g.standard_normal((spec.n_kv, spec.head_dim))
            vc[bt[i, p // bs], :, p % bs] = g.standard_normal((spec.n_kv, spec.head_dim))
    hid = np.random.default_rng(9).standard_normal((int(vb["query_lens"].sum()), spec.hidden)).astype(np.float32)
    return synth.Batch(c=c, K=K, context=np.asarray(vb["context"]), query_lens=vb["query_lens"],
                       target_ids=vb["target_ids"], target_pos=vb["target_pos"], num_accepted=vb["num_accepted"],
                       bonus_ids=vb["bonus_ids"], target_hidden=hid, block_table=bt, num_blocks=total + 1,
                       k_cache=[kc], v_cache=[vc])


def test_block_relabel_invariance(tiny):
    wl, w, b = tiny
    base = _run(wl.model, w, b)["forward"]
    rng = np.random.default_rng(3)
    perm = rng.permutation(b.num_blocks)
    b2 = copy.deepcopy(b)
    b2.block_table = perm[b.block_table].astype(np.int32)
    for li in range(wl.model.n_layers):
        b2.k_cache[li] = np.empty_like(b.k_cache[li])
        b2.v_cache[li] = np.empty_like(b.v_cache[li])
        b2.k_cache[li][perm] = b.k_cache[li]
        b2.v_cache[li][perm] = b.v_cache[li]
    got = _run(wl.model, w, b2)["forward"]
    assert np.array_equal(got["logits"], base["logits"])


def test_sequence_permutation_equivariance():
    spec = synth.TINY
    wl = synth.Workload("p", spec, c=4, K=3, ctx_lo=3, ctx_hi=40, accept_hi=3, seed=21)
    w = synth.make_weights(spec, 21)
    b = synth.make_batch(wl)
    base = _run(spec, w, b)["forward"]
    order = np.array([2, 0, 3, 1])
    L = b.query_lens
    starts = np.concatenate([[0], np.cumsum(L)])
    seg = lambda arr: np.concatenate([arr[starts[i]:starts[i + 1]] for i in order])  # noqa: E731
    b2 = copy.deepcopy(b)
    b2.query_lens, b2.num_accepted, b2.bonus_ids = L[order], b.num_accepted[order], b.bonus_ids[order]
    b2.target_ids, b2.target_pos, b2.target_hidden = seg(b.target_ids), seg(b.target_pos), seg(b.target_hidden)
    b2.block_table, b2.context = b.block_table[order], b.context[order]
    got = _run(spec, w, b2)["forward"]
    assert np.array_equal(got["logits"], base["logits"][order])


def test_rejected_rows_are_inert():
    spec = synth.TINY
    wl = synth.Workload("r", spec, c=3, K=3, ctx_lo=3, ctx_hi=40, accept_hi=0, seed=31)
    w = synth.make_weights(spec, 31)
    b = synth.make_batch(wl)                       # a_i = 0: three rejected rows each
    base = _run(spec, w, b)
    b2 = copy.deepcopy(b)
    s = 0
    rng = np.random.default_rng(0)
    for i in range(b.c):
        a, L = int(b.num_accepted[i]), int(b.query_lens[i])
        for j in range(a + 1, L):
            b2.target_ids[s + j] = rng.integers(0, spec.vocab - 1)
            b2.target_hidden[s + j] = rng.standard_normal(spec.hidden)
        s += L
    got = _run(spec, w, b2)
    assert np.array_equal(got["forward"]["logits"], base["forward"]["logits"])
    # the rejected rows themselves did change
    rej = base["meta"]["is_rejected"].astype(bool)
    assert not np.array_equal(got["draft_hidden"][rej], base["draft_hidden"][rej])


def test_context_is_read(tiny):
    wl, w, b = tiny
    base = _run(wl.model, w, b)["forward"]
    b2 = copy.deepcopy(b)
    blk = b.block_table[0, 0]
    b2.k_cache[0][blk, :, 3] += 1.0                # position 3 < P of sequence 0
    got = _run(wl.model, w, b2)["forward"]
    assert np.max(np.abs(got["logits"][0] - base["logits"][0])) > 1e-6
    assert np.array_equal(got["logits"][1], base["logits"][1])


def test_rope_off_by_one_is_visible(tiny, monkeypatch):
    wl, w, b = tiny
    base = _run(wl.model, w, b)["forward"]
    real = po.rope_rotate_half
    monkeypatch.setattr(po, "rope_rotate_half", lambda x, pos, th: real(x, np.asarray(pos) + 1, th))
    bad = _run(wl.model, w, b)["forward"]
    assert np.max(np.abs(bad["logits"] - base["logits"])) > 1e-3


def test_argmax_ties_take_lowest_id(tiny):
    wl, w, b = tiny
    base = _run(wl.model, w, b)["forward"]
    tok = base["tokens"].reshape(-1)
    s = int(np.argmax(tok > 0))
    t = int(tok[s])
    w2 = copy.deepcopy(w)
    j = t // 2
    w2["w_lm"][j] = w2["w_lm"][t]
    got = _run(wl.model, w2, b)["forward"]
    assert got["tokens"].reshape(-1)[s] == j
    assert got["top2_gap"].reshape(-1)[s] == 0.0


def test_bf16_rounding_points_stay_within_logit_tolerance():
    spec = synth.ModelSpec(hidden=256, vocab=1024, n_layers=1, n_q=8, n_kv=2, head_dim=32, inter=512)
    wl = synth.Workload("b", spec, c=2, K=4, ctx_lo=50, ctx_hi=300, accept_hi=4, seed=41)
    w = synth.make_weights(spec, 41)
    b = synth.make_batch(wl)
    mir = _run(spec, w, b, precision="mirror")["forward"]["logits"]
    exact = _run(spec, w, b, precision="fp64")["forward"]["logits"]
    err = np.max(np.abs(mir - exact))
    assert 0 < err < 2e-2
