"""Pins for the oracle's multi-pass and multi-round pieces: the autoregressive
baseline, the cache commit between passes, and the next round's verified
batch.

* autoregressive_draft vs an independent float64 torch loop (library
  routines only, its own cache bookkeeping);
* K = 1 autoregressive drafting is the parallel-draft pass at K = 1, and the
  first autoregressive token equals the first parallel-draft token at any K;
* next_verified_batch chained through expand_batch: positions, tokens,
  KV lengths, and the MASK-row positions the next round's accepted rows
  overwrite;
* apply_cache_writes stores exactly the encoded values and nothing else.
"""

import numpy as np
import torch
import torch.nn.functional as F

import oracle
import synth

f64 = torch.float64


def _t(x):
    return torch.tensor(np.asarray(x, dtype=np.float32), dtype=f64)


def _rope(x, pos, theta):
    """Rotate-half RoPE as a complex rotation (independent of the oracle's)."""
    d = x.shape[-1]
    half = d // 2
    z = torch.complex(x[..., :half], x[..., half:])
    j = torch.arange(half, dtype=f64)
    ang = torch.tensor(pos, dtype=f64)[:, None] * torch.pow(torch.tensor(theta, dtype=f64), -2.0 * j / d)
    r = z * torch.polar(torch.ones_like(ang), ang)[:, None, :]
    return torch.cat([r.real, r.imag], dim=-1)


def _torch_rows(spec, w, ids, hid, pos, seq, kv_lens, kcache, vcache, bt, write):
    """One drafter pass over rows (ids, hid, pos) of sequences seq; rows with
    write[r] append (k, v) at position pos[r].  Returns (final residual rows,
    logits of every row).  kcache / vcache are float64 tensors, updated with
    fp32-rounded values after the pass (the cache dtype)."""
    H, nq, nkv, d, bs = spec.hidden, spec.n_q, spec.n_kv, spec.head_dim, spec.block_size
    x = F.linear(torch.cat([_t(w["embed"])[torch.tensor(ids)], hid], dim=1), _t(w["w_fc"]))
    commits = []
    for li, lw in enumerate(w["layers"]):
        a = F.rms_norm(x, (H,), weight=_t(lw["ln1"]), eps=spec.rms_eps)
        q = _rope(F.linear(a, _t(lw["wq"])).view(-1, nq, d), pos, spec.rope_theta)
        k = _rope(F.linear(a, _t(lw["wk"])).view(-1, nkv, d), pos, spec.rope_theta)
        v = F.linear(a, _t(lw["wv"])).view(-1, nkv, d)
        kc, vc = kcache[li].clone(), vcache[li].clone()
        for r in range(len(ids)):
            if write[r]:
                p = int(pos[r])
                blk = bt[seq[r]][p // bs]
                kc[blk, :, p % bs] = k[r]
                vc[blk, :, p % bs] = v[r]
        commits.append((kc, vc, k, v))
        attn = torch.zeros(len(ids), nq, d, dtype=f64)
        for r in range(len(ids)):
            i, n = seq[r], int(kv_lens[seq[r]])
            keys = torch.stack([kc[bt[i][p // bs], :, p % bs] for p in range(n)])
            vals = torch.stack([vc[bt[i][p // bs], :, p % bs] for p in range(n)])
            mask = torch.tensor(np.arange(n)[None, :] <= pos[r])
            attn[r] = F.scaled_dot_product_attention(q[r:r + 1].transpose(0, 1), keys.transpose(0, 1),
                                                     vals.transpose(0, 1), attn_mask=mask,
                                                     enable_gqa=True).transpose(0, 1)[0]
        x = x + F.linear(attn.reshape(len(ids), nq * d), _t(lw["wo"]))
        m = F.rms_norm(x, (H,), weight=_t(lw["ln2"]), eps=spec.rms_eps)
        x = x + F.linear(F.silu(F.linear(m, _t(lw["w_gate"]))) * F.linear(m, _t(lw["w_up"])), _t(lw["w_down"]))
    # commit this pass's writes, rounded to the fp32 cache
    for li, (kc, vc, k, v) in enumerate(commits):
        for r in range(len(ids)):
            if write[r]:
                p = int(pos[r])
                blk = bt[seq[r]][p // bs]
                kcache[li][blk, :, p % bs] = k[r].to(torch.float32).to(f64)
                vcache[li][blk, :, p % bs] = v[r].to(torch.float32).to(f64)
    f = F.rms_norm(x, (H,), weight=_t(w["ln_f"]), eps=spec.rms_eps)
    return x, F.linear(f, _t(w["w_lm"]))


def _torch_autoregressive(spec, w, b, K):
    """K one-token passes written from the definition: pass 0 over the
    verified rows (token shift, bonus in the last accepted row, rejected rows
    not written), then one row per sequence fed with its previous token and
    its own final residual (rounded to fp32)."""
    c = len(b.query_lens)
    bt = np.asarray(b.block_table)
    kcache = [_t(k) for k in b.k_cache]
    vcache = [_t(v) for v in b.v_cache]
    starts = np.concatenate([[0], np.cumsum(b.query_lens)])
    ids, hid, pos, seq, write, samp = [], [], [], [], [], []
    kv = np.zeros(c, np.int64)
    for i in range(c):
        s, L, a = int(starts[i]), int(b.query_lens[i]), int(b.num_accepted[i])
        for r in range(L):
            tok = b.target_ids[s + r + 1] if r < a else (b.bonus_ids[i] if r == a else
                                                         (b.target_ids[s + r + 1] if r + 1 < L else b.bonus_ids[i]))
            ids.append(int(tok))
            pos.append(int(b.target_pos[s + r]))
            seq.append(i)
            write.append(r <= a)
            if r == a:
                samp.append(len(ids) - 1)
        kv[i] = int(b.target_pos[s + a]) + 1
    hid = _t(b.target_hidden)
    base = kv - 1
    toks = np.zeros((c, K), np.int64)
    logits = []
    for k in range(K):
        x, lg = _torch_rows(spec, w, ids, hid, np.array(pos), seq, kv, kcache, vcache, bt, write)
        lg = lg[torch.tensor(samp)].numpy()
        logits.append(lg)
        toks[:, k] = lg.argmax(axis=1)
        xs = x[torch.tensor(samp)].to(torch.float32).to(f64)
        ids = [int(t) for t in toks[:, k]]
        hid = xs
        pos = [int(base[i]) + k + 1 for i in range(c)]
        seq = list(range(c))
        write = [True] * c
        samp = list(range(c))
        kv = base + k + 2
    return toks, np.stack(logits, axis=1), kcache, vcache


def _tiny_ar_case(K=3, seed=61):
    spec = synth.ModelSpec(hidden=32, vocab=97, n_layers=2, n_q=4, n_kv=2, head_dim=8, inter=48, dtype="fp32")
    wl = synth.Workload("ar-tiny", spec, c=3, K=K, ctx_lo=3, ctx_hi=30, accept_hi=K, seed=seed)
    return spec, synth.make_weights(spec, seed), synth.make_batch(wl)


def test_autoregressive_matches_torch_loop():
    spec, w, b = _tiny_ar_case(K=4)
    got = oracle.autoregressive_draft(spec, w, b, 4, precision="fp64")
    toks, logits, kref, vref = _torch_autoregressive(spec, w, b, 4)
    np.testing.assert_allclose(got["logits"], logits, rtol=1e-9, atol=1e-11)
    assert np.array_equal(got["tokens"], toks)
    for li in range(spec.n_layers):
        written = ~np.isnan(kref[li].numpy())
        np.testing.assert_allclose(got["k_cache"][li][written], kref[li].numpy()[written], rtol=1e-6, atol=1e-6)
        np.testing.assert_allclose(got["v_cache"][li][written], vref[li].numpy()[written], rtol=1e-6, atol=1e-6)


def test_autoregressive_k1_is_the_parallel_pass():
    spec, w, b = _tiny_ar_case(K=1, seed=62)
    ar = oracle.autoregressive_draft(spec, w, b, 1, precision="fp64")
    pe = oracle.parallel_draft_step(spec, w, b, precision="fp64")["forward"]
    assert np.array_equal(ar["tokens"], pe["tokens"])
    np.testing.assert_array_equal(ar["logits"], pe["logits"])


def test_first_autoregressive_token_is_the_first_parallel_token():
    spec, w, b = _tiny_ar_case(K=5, seed=63)
    ar = oracle.autoregressive_draft(spec, w, b, 5, precision="fp64")
    pe = oracle.parallel_draft_step(spec, w, b, precision="fp64")["forward"]
    assert np.array_equal(ar["tokens"][:, 0], pe["tokens"][:, 0])
    np.testing.assert_allclose(ar["logits"][:, 0], pe["logits"][:, 0], rtol=1e-12, atol=1e-12)


def test_teacher_forcing_feeds_the_given_tokens():
    spec, w, b = _tiny_ar_case(K=3, seed=64)
    own = oracle.autoregressive_draft(spec, w, b, 3, precision="fp64")
    forced = own["tokens"].copy()
    forced[:, 0] = (forced[:, 0] + 1) % (spec.vocab - 1)
    f = oracle.autoregressive_draft(spec, w, b, 3, precision="fp64", forced_tokens=forced)
    # step 0 does not depend on the fed tokens; later steps do
    np.testing.assert_array_equal(f["logits"][:, 0], own["logits"][:, 0])
    assert not np.allclose(f["logits"][:, 1], own["logits"][:, 1])


def test_next_verified_batch_chains_through_expand():
    rng = np.random.default_rng(5)
    c, K = 4, 5
    kv_lens = rng.integers(20, 60, size=c)
    bonus = rng.integers(0, 90, size=c)
    drafts = rng.integers(0, 90, size=(c, K))
    acc = np.array([0, 2, K, 1])
    nb = rng.integers(0, 90, size=c)
    nxt = oracle.next_verified_batch(kv_lens, bonus, drafts, acc, nb, K)
    base = kv_lens - K
    for i in range(c):
        ids = nxt["target_ids"][i * (K + 1):(i + 1) * (K + 1)]
        pos = nxt["target_pos"][i * (K + 1):(i + 1) * (K + 1)]
        assert ids[0] == bonus[i] and np.array_equal(ids[1:], drafts[i])
        assert np.array_equal(pos, base[i] + 1 + np.arange(K + 1))
    assert np.all(nxt["query_lens"] == K + 1)
    bs = 16
    need = int((kv_lens.max() + 2 * K + 2) // bs + 1)
    bt = np.arange(c * need, dtype=np.int32).reshape(c, need)
    meta = oracle.expand_batch(nxt["query_lens"], nxt["target_ids"], nxt["target_pos"], nxt["num_accepted"],
                               nxt["bonus_ids"], bt, K, 96, bs)
    for i in range(c):
        r0, a = int(meta["cu_draft"][i]), int(acc[i])
        rows = np.arange(r0, r0 + a + 1)
        # accepted drafts, then the new bonus, at positions base+1 .. base+1+a
        assert np.array_equal(meta["draft_ids"][rows], np.concatenate([drafts[i, :a], [nb[i]]]))
        assert np.array_equal(meta["draft_pos"][rows], base[i] + 1 + np.arange(a + 1))
        assert meta["kv_lens"][i] == base[i] + 1 + a + K
        # this round's MASK rows sat at base+1 .. base+K-1; the accepted rows of
        # the next round rewrite the first a of them
        this_mask = set(range(int(base[i]) + 1, int(base[i]) + K))
        rewritten = this_mask & set(meta["draft_pos"][rows].tolist())
        assert rewritten == set(range(int(base[i]) + 1, int(base[i]) + 1 + min(a + 1, K - 1)))


def test_apply_cache_writes_stores_exactly_the_writes():
    spec = synth.ModelSpec(hidden=16, vocab=50, n_layers=1, n_q=2, n_kv=2, head_dim=8, inter=16, dtype="bf16")
    rng = np.random.default_rng(3)
    kc = [rng.integers(0, 1 << 16, size=(4, 2, 16, 8)).astype(np.uint16)]
    vc = [kc[0].copy()]
    before = kc[0].copy()
    slots = np.array([3, 17, 40])
    k = rng.standard_normal((3, 2, 8))
    v = rng.standard_normal((3, 2, 8))
    oracle.apply_cache_writes(spec, kc, vc, [dict(slots=slots, k=k, v=v)])
    # expected bits from torch's own float -> bfloat16 cast, not the oracle's codec
    bits = lambda x: torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    for n, sl in enumerate(slots):
        np.testing.assert_array_equal(kc[0][sl // 16, :, sl % 16], bits(k[n]))
        np.testing.assert_array_equal(vc[0][sl // 16, :, sl % 16], bits(v[n]))
    mask = np.ones(before.shape, bool)
    for sl in slots:
        mask[sl // 16, :, sl % 16] = False
    np.testing.assert_array_equal(kc[0][mask], before[mask])


def test_forced_hidden_rows_feed_the_given_states():
    """Forcing the oracle's own fed-back rows reproduces its free run exactly;
    forcing different rows changes every later pass but not the first."""
    spec, w, b = _tiny_ar_case(K=3, seed=65)
    own = oracle.autoregressive_draft(spec, w, b, 3, precision="mirror")
    assert own["fed_hidden"].shape == (2, b.c, spec.hidden)
    same = oracle.autoregressive_draft(spec, w, b, 3, precision="mirror", forced_tokens=own["tokens"],
                                       forced_hidden=own["fed_hidden"])
    np.testing.assert_array_equal(same["logits"], own["logits"])
    np.testing.assert_array_equal(same["fed_hidden"], own["fed_hidden"])
    other = own["fed_hidden"].copy()
    other[0] = np.float32(0.5) * other[0]
    f = oracle.autoregressive_draft(spec, w, b, 3, precision="mirror", forced_tokens=own["tokens"],
                                    forced_hidden=other)
    np.testing.assert_array_equal(f["logits"][:, 0], own["logits"][:, 0])
    assert np.max(np.abs(f["logits"][:, 1] - own["logits"][:, 1])) > 1e-6
