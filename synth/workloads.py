"""Workload shapes and seeded generators for the P-EAGLE parallel-draft step.

The shapes follow the drafter sizes and batch mixes used to exercise the
method (GPT-OSS-20B-shaped and Qwen3-Coder-30B-shaped drafters, concurrency
1..64, depth K in {3,5,7}); the pages run on real benchmarks, which these
seeded synthetic batches stand in for.

Storage conventions (shared by every consumer):

* ``fp32`` tensors are ``numpy.float32`` arrays.
* ``bf16`` tensors are ``numpy.uint16`` arrays holding the raw bfloat16 bit
  patterns (upper 16 bits of an IEEE float32).
* Matrices are row-major ``[out_features, in_features]``.
* The paged KV cache of each layer is ``[num_blocks, n_kv, block_size, head_dim]``;
  logical position ``p`` of sequence ``i`` lives in physical block
  ``block_table[i, p // block_size]`` at offset ``p % block_size``.
* Cache slots at positions the current pass must write (``p >= P_i``) and a
  spare padding block are pre-filled with NaN canaries, so reading a slot that
  was never written poisons the result.

Random streams: every tensor is drawn from its own counter-keyed PCG64 stream
``SeedSequence([seed, tensor_id, chunk])``, generated in parallel chunks.  The
values therefore do not depend on the thread count.
"""

from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field
from typing import Callable, List, Optional

import numpy as np

NAN_BF16_BITS = np.uint16(0x7FC0)
_CHUNK = 1 << 22


# ----------------------------------------------------------------------------
# bfloat16 encoding of generated data (input encoding, not model arithmetic)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even), return bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)

    def work(lo: int, hi: int) -> None:
        v = flat_u[lo:hi]
        nan = (v & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
        r = (v + np.uint32(0x7FFF) + ((v >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        r = r.astype(np.uint16)
        r[nan] = NAN_BF16_BITS
        flat_o[lo:hi] = r

    _parallel_ranges(flat_u.size, work)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 values."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _parallel_ranges(n: int, fn: Callable[[int, int], None]) -> None:
    ranges = [(lo, min(n, lo + _CHUNK)) for lo in range(0, n, _CHUNK)]
    if len(ranges) <= 1:
        for lo, hi in ranges:
            fn(lo, hi)
        return
    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(lambda r: fn(*r), ranges))


def _normal(shape, std: float, seed: int, tensor_id: int) -> np.ndarray:
    """N(0, std^2) float32 tensor from counter-keyed streams (thread-count independent)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)

    def work(lo: int, hi: int) -> None:
        rng = np.random.default_rng(np.random.SeedSequence([seed, tensor_id, lo // _CHUNK]))
        rng.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        if std != 1.0:
            out[lo:hi] *= np.float32(std)

    _parallel_ranges(n, work)
    return out.reshape(shape)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Encode float32 values in storage dtype ("fp32" or "bf16" bits)."""
    if dtype == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# Shapes
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class ModelSpec:
    hidden: int
    vocab: int
    n_layers: int
    n_q: int
    n_kv: int
    head_dim: int
    inter: int
    dtype: str = "bf16"
    block_size: int = 16
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0

    @property
    def mask_token_id(self) -> int:
        # emb(mask) is a learned row of the embedding table; the synthetic
        # drafters reserve the last vocabulary id for it.
        return self.vocab - 1


@dataclass(frozen=True)
class Workload:
    name: str
    model: ModelSpec
    c: int                      # sequences in the batch
    K: int                      # draft depth (tokens proposed per sequence)
    ctx_lo: int                 # cached context P_i ~ U{ctx_lo..ctx_hi}
    ctx_hi: int
    accept_hi: int              # accepted drafts a_i ~ U{0..accept_hi}
    agree_p0: float = 0.7       # target agrees with draft d w.p. p0 * decay^d
    agree_decay: float = 1.0
    seed: int = 0               # batch / cache / agreement draws
    weight_seed: int = -1       # drafter weights (-1: same as seed); shared per drafter shape
    prep_only: bool = False     # batch expansion + hidden placement only
    description: str = ""

    @property
    def wseed(self) -> int:
        return self.seed if self.weight_seed < 0 else self.weight_seed

    @property
    def L(self) -> int:
        # verified rows per sequence: the previous round proposed K drafts,
        # so the verify batch holds the last accepted token plus K drafts.
        return self.K + 1

    def agree_probs(self) -> np.ndarray:
        return self.agree_p0 * self.agree_decay ** np.arange(self.K, dtype=np.float64)


TINY = ModelSpec(hidden=64, vocab=512, n_layers=1, n_q=4, n_kv=2, head_dim=16, inter=128, dtype="fp32")
GPTOSS20B = ModelSpec(hidden=2880, vocab=201088, n_layers=1, n_q=64, n_kv=8, head_dim=64, inter=7680)
QWEN3CODER30B = ModelSpec(hidden=2048, vocab=151936, n_layers=1, n_q=32, n_kv=4, head_dim=128, inter=6144)


def _workloads() -> dict:
    w = {}
    w["tiny-fp32-c2-k3"] = Workload(
        "tiny-fp32-c2-k3", TINY, c=2, K=3, ctx_lo=16, ctx_hi=16, accept_hi=3,
        agree_p0=0.7, seed=0,
        description="tiny fp32 drafter (H=64, V=512, 4x16 q heads, 2 kv heads, I=128), "
                    "2 sequences with 16 cached tokens, K=3")
    w["prep-bf16-c64-k7-h2880"] = Workload(
        "prep-bf16-c64-k7-h2880", GPTOSS20B, c=64, K=7, ctx_lo=512, ctx_hi=8192, accept_hi=7,
        seed=1, prep_only=True,
        description="batch expansion + hidden scatter/broadcast only, bf16 H=2880, "
                    "c=64, K=7, contexts U{512..8192} in 16-token pages")
    w["gptoss20b-bf16-c1-k7"] = Workload(
        "gptoss20b-bf16-c1-k7", GPTOSS20B, c=1, K=7, ctx_lo=2048, ctx_hi=2048, accept_hi=7,
        seed=2, weight_seed=2,
        description="GPT-OSS-20B-shaped drafter (H=2880, 64x64 q heads, 8 kv heads, I=7680, "
                    "V=201088), c=1, K=7, 2048 cached tokens")
    for k in (3, 5):
        w[f"gptoss20b-bf16-c1-k{k}"] = Workload(
            f"gptoss20b-bf16-c1-k{k}", GPTOSS20B, c=1, K=k, ctx_lo=2048, ctx_hi=2048, accept_hi=k,
            seed=2, weight_seed=2,
            description=f"GPT-OSS-20B-shaped drafter, c=1, K={k}, 2048 cached tokens (depth sweep)")
    w["gptoss20b-bf16-c64-k7"] = Workload(
        "gptoss20b-bf16-c64-k7", GPTOSS20B, c=64, K=7, ctx_lo=512, ctx_hi=8192, accept_hi=7,
        seed=3, weight_seed=2,
        description="GPT-OSS-20B-shaped drafter, c=64, K=7, contexts U{512..8192} paged")
    w["gptoss20b-bf16-c64-k8"] = Workload(
        "gptoss20b-bf16-c64-k8", GPTOSS20B, c=64, K=8, ctx_lo=512, ctx_hi=8192, accept_hi=8,
        seed=3, weight_seed=2,
        description="GPT-OSS-20B-shaped drafter, c=64, K=8: 512 sampled rows into the LM head "
                    "(the 512-row LM-head figure beside the 448 rows of K=7)")
    for k in (3, 5, 7):
        name = f"qwen3coder30b-bf16-c16-k{k}"
        w[name] = Workload(
            name, QWEN3CODER30B, c=16, K=k, ctx_lo=1024, ctx_hi=16384, accept_hi=k,
            agree_p0=0.8, agree_decay=0.9, seed=4 + k, weight_seed=4,
            description=f"Qwen3-Coder-30B-shaped drafter (H=2048, 32x128 q heads, 4 kv heads, "
                        f"I=6144, V=151936), c=16, K={k}, contexts U{{1024..16384}} paged")
    return w


WORKLOADS = _workloads()


# ----------------------------------------------------------------------------
# Weights
# ----------------------------------------------------------------------------
def make_weights(spec: ModelSpec, seed: int, prep_only: bool = False) -> dict:
    """Random-init drafter weights in storage dtype.

    Matrices are N(0, 0.02); RMSNorm gains are 1; the MASK row of the
    embedding table and the shared hidden placeholder are N(0, 1).
    """
    H, V, d = spec.hidden, spec.vocab, spec.head_dim
    dt = spec.dtype
    tid = iter(range(1, 10_000))
    w: dict = {}
    if prep_only:
        w["h_shared"] = store(_normal((H,), 1.0, seed, 9000), dt)
        return w
    emb = _normal((V, H), 0.02, seed, next(tid))
    emb[spec.mask_token_id] = _normal((H,), 1.0, seed, 9001)
    w["embed"] = store(emb, dt)
    del emb
    w["w_fc"] = store(_normal((H, 2 * H), 0.02, seed, next(tid)), dt)
    layers = []
    for _ in range(spec.n_layers):
        lw = {
            "ln1": store(np.ones(H, np.float32), dt),
            "wq": store(_normal((spec.n_q * d, H), 0.02, seed, next(tid)), dt),
            "wk": store(_normal((spec.n_kv * d, H), 0.02, seed, next(tid)), dt),
            "wv": store(_normal((spec.n_kv * d, H), 0.02, seed, next(tid)), dt),
            "wo": store(_normal((H, spec.n_q * d), 0.02, seed, next(tid)), dt),
            "ln2": store(np.ones(H, np.float32), dt),
            "w_gate": store(_normal((spec.inter, H), 0.02, seed, next(tid)), dt),
            "w_up": store(_normal((spec.inter, H), 0.02, seed, next(tid)), dt),
            "w_down": store(_normal((H, spec.inter), 0.02, seed, next(tid)), dt),
        }
        layers.append(lw)
    w["layers"] = layers
    w["ln_f"] = store(np.ones(H, np.float32), dt)
    w["w_lm"] = store(_normal((V, H), 0.02, seed, next(tid)), dt)
    w["h_shared"] = store(_normal((H,), 1.0, seed, 9000), dt)
    return w


# ----------------------------------------------------------------------------
# Verified batch + paged cache
# ----------------------------------------------------------------------------
@dataclass
class Batch:
    c: int
    K: int
    context: np.ndarray          # P_i, int64 [c]
    query_lens: np.ndarray       # L_i, int32 [c]
    target_ids: np.ndarray       # int32 [T]
    target_pos: np.ndarray       # int32 [T]
    num_accepted: np.ndarray     # a_i, int32 [c]
    bonus_ids: np.ndarray        # b_i, int32 [c]
    target_hidden: np.ndarray    # [T, H] storage dtype
    block_table: np.ndarray      # int32 [c, max_blocks]
    num_blocks: int
    k_cache: List[Optional[np.ndarray]] = field(default_factory=list)
    v_cache: List[Optional[np.ndarray]] = field(default_factory=list)

    @property
    def T(self) -> int:
        return int(self.query_lens.sum())

    @property
    def N(self) -> int:
        return self.T + self.c * (self.K - 1)


def _canary(dtype: str):
    return NAN_BF16_BITS if dtype == "bf16" else np.float32(np.nan)


def make_batch(wl: Workload, seed: Optional[int] = None, with_cache: Optional[bool] = None,
               accepted: Optional[np.ndarray] = None, extra_positions: int = 0) -> Batch:
    """Verified batch for one parallel-draft round of workload ``wl``.

    ``accepted`` overrides the drawn a_i (used by exhaustive sweeps);
    ``extra_positions`` extends every block table (and the NaN-filled pages
    behind it) that many positions further, for later rounds.
    """
    spec = wl.model
    seed = wl.seed if seed is None else seed
    with_cache = (not wl.prep_only) if with_cache is None else with_cache
    rng = np.random.default_rng(np.random.SeedSequence([seed, 7001]))
    c, K, L = wl.c, wl.K, wl.L
    P = rng.integers(wl.ctx_lo, wl.ctx_hi + 1, size=c).astype(np.int64)
    a = rng.integers(0, wl.accept_hi + 1, size=c).astype(np.int32)
    if accepted is not None:
        a = np.asarray(accepted, dtype=np.int32).copy()
    a = np.minimum(a, L - 1)
    qlen = np.full(c, L, dtype=np.int32)
    T = int(qlen.sum())
    ids = rng.integers(0, spec.vocab - 1, size=T).astype(np.int32)   # MASK id never drawn
    bonus = rng.integers(0, spec.vocab - 1, size=c).astype(np.int32)
    pos = np.concatenate([P[i] + np.arange(L) for i in range(c)]).astype(np.int32)
    hid = store(_normal((T, spec.hidden), 1.0, seed, 7002), spec.dtype)

    bs = spec.block_size
    # blocks cover every position a draft row can occupy: P_i .. P_i + L + K - 2
    need = [int(-(-(P[i] + L + K - 1 + extra_positions) // bs)) for i in range(c)]
    total = int(sum(need))
    perm = rng.permutation(total).astype(np.int32)
    max_blocks = max(need)
    spare = total                      # extra NaN block used as table padding
    bt = np.full((c, max_blocks), spare, dtype=np.int32)
    off = 0
    for i in range(c):
        bt[i, :need[i]] = perm[off:off + need[i]]
        off += need[i]
    num_blocks = total + 1

    kc: List[Optional[np.ndarray]] = []
    vc: List[Optional[np.ndarray]] = []
    if with_cache:
        shape = (num_blocks, spec.n_kv, bs, spec.head_dim)
        can = _canary(spec.dtype)
        for layer in range(spec.n_layers):
            pair = []
            for which in range(2):
                x = store(_normal(shape, 1.0, seed, 7100 + 2 * layer + which), spec.dtype)
                x[spare] = can
                for i in range(c):
                    # positions >= P_i belong to this round's draft rows
                    first = int(P[i])
                    for j in range(first // bs, need[i]):
                        o0 = max(0, first - j * bs)
                        x[bt[i, j], :, o0:, :] = can
                pair.append(x)
            kc.append(pair[0])
            vc.append(pair[1])
    return Batch(c=c, K=K, context=P, query_lens=qlen, target_ids=ids, target_pos=pos,
                 num_accepted=a, bonus_ids=bonus, target_hidden=hid, block_table=bt,
                 num_blocks=num_blocks, k_cache=kc, v_cache=vc)


# ----------------------------------------------------------------------------
# Synthetic target tokens for greedy acceptance
# ----------------------------------------------------------------------------
def make_agreement_draws(wl: Workload, seed: Optional[int] = None):
    """Uniform draws that decide, per draft depth, whether the synthetic target agrees."""
    seed = wl.seed if seed is None else seed
    rng = np.random.default_rng(np.random.SeedSequence([seed, 7201]))
    u = rng.random((wl.c, wl.K))
    alt = rng.integers(0, wl.model.vocab - 2, size=(wl.c, wl.K + 1)).astype(np.int64)
    return u, alt


def target_tokens_from_drafts(drafts: np.ndarray, u: np.ndarray, alt: np.ndarray,
                              p: np.ndarray, vocab: int) -> np.ndarray:
    """Target tokens [c, K+1]: depth d equals the draft w.p. p[d], else a different id.

    The disagreeing id is ``alt`` drawn from the vocabulary minus the MASK id
    and minus the draft itself; the last column (the token after K accepted
    drafts) is ``alt`` over the vocabulary minus the MASK id.
    """
    drafts = np.asarray(drafts, dtype=np.int64)
    c, K = drafts.shape
    t = np.empty((c, K + 1), dtype=np.int64)
    other = alt[:, :K] + (alt[:, :K] >= drafts)          # skip the draft's own id
    t[:, :K] = np.where(u < p[None, :], drafts, other)
    t[:, K] = np.minimum(alt[:, K], vocab - 2)
    return t.astype(np.int32)
