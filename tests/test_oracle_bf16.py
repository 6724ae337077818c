"""Independent pins of the oracle's bfloat16 arithmetic (CPU only).

Every bf16 parity gate rests on two pieces of the oracle:

* the storage codec -- ``decode`` (bf16 bits -> value), ``encode`` (value ->
  bf16 bits, round to nearest even) and ``round_operand``;
* the points where ``precision="mirror"`` rounds to bf16: the normalised
  activations before q/k/v and before the MLP, q and k after the rotary
  embedding, v (k and v are what the paged cache stores), the attention
  output, SiLU(gate)*up, and the final normalised rows before the LM head.

Neither is checked against the oracle itself here.  The codec is compared bit
for bit with torch's own float32 -> bfloat16 cast over every bf16 pattern and
every rounding tie; the rounding points are checked against a torch
composition of the pass (library routines, complex-number RoPE, SDPA) that
rounds with ``.to(torch.bfloat16)`` at exactly those points.  Dropping any
one point from that composition must move the logits far beyond the 1e-12
agreement bar, so a misplaced or missing rounding point in the oracle cannot
pass.

NaN encodings differ between implementations (torch's CPU cast gives 0xFFFF,
the oracle 0x7FC0); for NaN inputs only NaN-ness is compared.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth

f64 = torch.float64


def _torch_bits_of_f32(x32: np.ndarray) -> np.ndarray:
    """bf16 bits of float32 values by torch's cast."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _torch_value_of_bits(bits: np.ndarray) -> np.ndarray:
    """float64 value of bf16 bit patterns by torch's widening."""
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(f64).numpy()


def _all_patterns() -> np.ndarray:
    return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


# ----------------------------------------------------------------------------- codec
def test_decode_every_pattern_matches_torch():
    bits = _all_patterns()
    got = oracle.decode(bits, "bf16")
    want = _torch_value_of_bits(bits)
    nan = np.isnan(want)
    assert nan.sum() == 2 * 127 * 1  # 0x7F81..0x7FFF and 0xFF81..0xFFFF
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))  # -0.0 stays negative


def _tie_neighbourhood() -> np.ndarray:
    """float32 values at and around every bf16 rounding boundary: for each bf16
    pattern b, the fp32 values with upper half b and lower half 0, 1, 0x7FFF,
    0x8000 (the exact tie), 0x8001 and 0xFFFF."""
    hi = _all_patterns().astype(np.uint32) << np.uint32(16)
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    return (hi[:, None] | lows[None, :]).reshape(-1).view(np.float32)


def test_encode_matches_torch_cast_at_every_tie():
    x32 = _tie_neighbourhood()
    got = oracle.encode(x32.astype(np.float64), "bf16")
    want = _torch_bits_of_f32(x32)
    nan = np.isnan(x32)
    assert np.array_equal(np.isnan(oracle.decode(got[nan], "bf16")), np.ones(nan.sum(), bool))
    assert np.array_equal(got[~nan], want[~nan])
    # ties go to the even pattern: 1 + 2^-8 -> 1.0, 1 + 3 * 2^-8 -> 1 + 2^-6
    assert oracle.encode(np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]), "bf16").tolist() == [0x3F80, 0x3F82]


def test_encode_special_values():
    vals = np.array([0.0, -0.0, np.inf, -np.inf, 3.4028234663852886e38, -3.4028234663852886e38,
                     1e-45, -1e-45, 1.1754943508222875e-38])
    got = oracle.encode(vals, "bf16")
    want = _torch_bits_of_f32(vals.astype(np.float32))
    assert np.array_equal(got, want)
    # the largest float32 overflows bf16's range under round to nearest even
    assert got[4] == 0x7F80 and got[5] == 0xFF80
    assert got[1] == 0x8000


def test_encode_float64_rounds_through_float32_like_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200_000) * 10.0 ** rng.integers(-30, 30, size=200_000),
                        1.0 + 2.0 ** -8 + rng.integers(-4, 5, size=1000) * 2.0 ** -30])
    got = oracle.encode(x, "bf16")
    want = torch.tensor(x, dtype=f64).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    np.testing.assert_array_equal(oracle.round_operand(x, "bf16"), torch.tensor(x).to(torch.bfloat16).to(f64).numpy())
    np.testing.assert_array_equal(oracle.round_operand(x, "bf16", precision="fp64"), x)


def test_fp32_codec_matches_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(10_000) * 1e3
    np.testing.assert_array_equal(oracle.encode(x, "fp32"), torch.tensor(x).to(torch.float32).numpy())
    np.testing.assert_array_equal(oracle.round_operand(x, "fp32"), torch.tensor(x).to(torch.float32).to(f64).numpy())
    x32 = x.astype(np.float32)
    np.testing.assert_array_equal(oracle.decode(x32, "fp32"), torch.from_numpy(x32).to(f64).numpy())


# ----------------------------------------------------------------------------- rounding points
POINTS = ("norm1", "q", "k", "v", "attn", "norm2", "mlp", "final")


def _tv(arr) -> torch.Tensor:
    """Stored tensor -> float64 torch tensor (bf16 bits via torch's own view)."""
    arr = np.asarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(f64)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(f64)


def _rope(x: torch.Tensor, pos: np.ndarray, theta: float) -> torch.Tensor:
    """Rotate-half RoPE as a complex multiplication of (x_j, x_{j+d/2}) by e^{i p theta^(-2j/d)}."""
    d = x.shape[-1]
    half = d // 2
    z = torch.complex(x[..., :half], x[..., half:])
    j = torch.arange(half, dtype=f64)
    ang = torch.tensor(np.asarray(pos), dtype=f64)[:, None] * torch.pow(torch.tensor(theta, dtype=f64), -2.0 * j / d)
    r = z * torch.polar(torch.ones_like(ang), ang)[:, None, :]
    return torch.cat([r.real, r.imag], dim=-1)


def _torch_bf16_pass(spec, w, meta, hd, bt, kc, vc, points):
    """Drafter pass in float64 torch, rounding to bf16 (torch's cast) at the
    named points only.  Returns the sampled rows' logits and the (k, v) rows
    written to each layer's cache (as rounded values)."""
    H, nq, nkv, d, bs = spec.hidden, spec.n_q, spec.n_kv, spec.head_dim, spec.block_size

    def rnd(t, name):
        return t.to(torch.bfloat16).to(f64) if name in points else t

    ids = torch.tensor(np.asarray(meta["draft_ids"], dtype=np.int64))
    pos = np.asarray(meta["draft_pos"], dtype=np.int64)
    slots = np.asarray(meta["slot_mapping"], dtype=np.int64)
    x = F.linear(torch.cat([_tv(w["embed"])[ids], _tv(hd)], dim=1), _tv(w["w_fc"]))
    writes = []
    for li, lw in enumerate(w["layers"]):
        a = rnd(F.rms_norm(x, (H,), weight=_tv(lw["ln1"]), eps=spec.rms_eps), "norm1")
        q = rnd(_rope(F.linear(a, _tv(lw["wq"])).view(-1, nq, d), pos, spec.rope_theta), "q")
        k = rnd(_rope(F.linear(a, _tv(lw["wk"])).view(-1, nkv, d), pos, spec.rope_theta), "k")
        v = rnd(F.linear(a, _tv(lw["wv"])).view(-1, nkv, d), "v")
        kcache, vcache = _tv(kc[li]).clone(), _tv(vc[li]).clone()
        for r, sl in enumerate(slots):
            if sl >= 0:
                kcache[sl // bs, :, sl % bs] = k[r]
                vcache[sl // bs, :, sl % bs] = v[r]
        live = slots >= 0
        writes.append((k[torch.tensor(live)], v[torch.tensor(live)]))
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
        attn = rnd(attn.reshape(len(ids), nq * d), "attn")
        x = x + F.linear(attn, _tv(lw["wo"]))
        m = rnd(F.rms_norm(x, (H,), weight=_tv(lw["ln2"]), eps=spec.rms_eps), "norm2")
        hmid = rnd(F.silu(F.linear(m, _tv(lw["w_gate"]))) * F.linear(m, _tv(lw["w_up"])), "mlp")
        x = x + F.linear(hmid, _tv(lw["w_down"]))
    samp = torch.tensor(np.asarray(meta["sample_idx"], dtype=np.int64))
    f = rnd(F.rms_norm(x[samp], (H,), weight=_tv(w["ln_f"]), eps=spec.rms_eps), "final")
    return F.linear(f, _tv(w["w_lm"])).numpy(), writes


def _bf16_case(n_layers):
    """Small bf16 drafter whose q/k projections are scaled up 8x, so that the
    attention scores are sharp: with N(0, 0.02) projections the scores of the
    keys written in the pass are so flat that rounding k moves no bf16
    rounding of the attention output, and that point would go unseen."""
    spec = synth.ModelSpec(hidden=128, vocab=512, n_layers=n_layers, n_q=4, n_kv=2, head_dim=32, inter=192)
    wl = synth.Workload(f"bf16-pin-{n_layers}", spec, c=3, K=4, ctx_lo=5, ctx_hi=60, accept_hi=4,
                        seed=60 + n_layers)
    w = synth.make_weights(spec, wl.seed)
    for lw in w["layers"]:
        for n in ("wq", "wk"):
            lw[n] = synth.store(synth.bf16_bits_to_f32(lw[n]) * np.float32(8.0), "bf16")
    return spec, w, synth.make_batch(wl)


@pytest.mark.parametrize("n_layers", [1, 2])
def test_mirror_pass_matches_torch_bf16_composition(n_layers):
    spec, w, b = _bf16_case(n_layers)
    r = oracle.parallel_draft_step(spec, w, b, precision="mirror")
    meta, hd = r["meta"], r["draft_hidden"]
    logits, writes = _torch_bf16_pass(spec, w, meta, hd, b.block_table, b.k_cache, b.v_cache, set(POINTS))
    got = r["forward"]["logits"].reshape(logits.shape)
    assert np.max(np.abs(got - logits)) <= 1e-12
    # the cache writes are the composition's rounded k and v, value for value
    for li, (k, v) in enumerate(writes):
        cw = r["forward"]["cache_writes"][li]
        np.testing.assert_array_equal(cw["k"], k.numpy())
        np.testing.assert_array_equal(cw["v"], v.numpy())
    # with no rounding point the composition is the oracle's fp64 pass
    exact = oracle.parallel_draft_step(spec, w, b, precision="fp64")["forward"]["logits"].reshape(logits.shape)
    unrounded, _ = _torch_bf16_pass(spec, w, meta, hd, b.block_table, b.k_cache, b.v_cache, set())
    np.testing.assert_allclose(exact, unrounded, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("drop", POINTS)
def test_every_rounding_point_is_visible(drop):
    """The 1e-12 agreement above is sensitive to each point on its own: the
    composition without it moves the logits far from the oracle's mirror."""
    spec, w, b = _bf16_case(1)
    r = oracle.parallel_draft_step(spec, w, b, precision="mirror")
    logits, _ = _torch_bf16_pass(spec, w, r["meta"], r["draft_hidden"], b.block_table, b.k_cache, b.v_cache,
                                 set(POINTS) - {drop})
    got = r["forward"]["logits"].reshape(logits.shape)
    assert np.max(np.abs(got - logits)) > 1e-7
