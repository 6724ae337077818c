"""Float64 reference definitions of one P-EAGLE parallel-draft round.

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.

Sources (cited by page title and section):

* [PF]  "P-EAGLE: Faster LLM Inference with Parallel Speculative Decoding in
  vLLM" (papercache notes): "怎么做的" (how it works) with the Input_i
  equation; "vLLM中的工程实现细节" (vLLM implementation details) with the
  hidden-state placement listing.
* [PP]  "P-EAGLE: Parallel Speculative Decoding in vLLM" (agentlenshq):
  "Step 2: Parallel Drafting"; "vLLM Implementation Details" -> "Fused Triton
  Kernel", "Hidden State Management", "KV Cache and CUDA Graphs";
  "Acceptance Length (AL)".
* [PD]  "并行草稿机制解析：从P-EAGLE到DSpark": section 6.1 (RoPE positions must
  match exactly).

Where the pages leave a step open, the reading taken is stated at the
function; every such reading is also listed in the design notes.

Precision model: inputs are the exact stored values (fp32 or bf16) widened to
float64.  ``precision="mirror"`` rounds to the storage dtype exactly at the
points where the HIP path stores a tensor or feeds a matrix operand (KV cache
entries, the normalised activations, q, the attention output, SiLU(gate)*up,
the final normalised rows); everything else stays float64.
``precision="fp64"`` never rounds.  parity: pinned by tests/test_oracle_*.py
(the bf16 codec bit for bit against torch's cast over every pattern and tie,
the mirror rounding points against a torch composition that rounds at exactly
those points, each point shown to be observable).
"""

from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

# Rejected tokens are sent to a padding KV slot so that they never write the
# cache ([PP] "KV Cache and CUDA Graphs").
PADDING_SLOT_ID = -1


# ----------------------------------------------------------------------------
# storage decoding and operand rounding
# ----------------------------------------------------------------------------
def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored tensor -> float64 values (bf16 stored as raw uint16 bits)."""
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def _bf16_bits(x64: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bits, rounding to nearest even via the float32 value."""
    u = np.ascontiguousarray(x64, dtype=np.float32).view(np.uint32)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    r[nan] = np.uint16(0x7FC0)
    return r


def encode(x64: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> storage representation of ``dtype``."""
    if dtype == "fp32":
        return np.asarray(x64, dtype=np.float32)
    if dtype == "bf16":
        return _bf16_bits(x64)
    raise ValueError(dtype)


def round_operand(x64: np.ndarray, dtype: str, precision: str = "mirror") -> np.ndarray:
    """Value of ``x64`` after storing it in ``dtype`` (identity when precision='fp64')."""
    if precision == "fp64":
        return np.asarray(x64, dtype=np.float64)
    return decode(encode(x64, dtype), dtype)


# ----------------------------------------------------------------------------
# Step 1: expand the verified batch into the draft layout
# ----------------------------------------------------------------------------
def expand_batch(query_lens, target_ids, target_pos, num_accepted, bonus_ids, block_table,
                 K: int, mask_id: int, block_size: int = 16, compact: bool = False) -> Dict[str, np.ndarray]:
    """Draft-batch metadata, one row kind at a time.

    [PP] "Fused Triton Kernel": in one pass the previous token ids and
    positions are copied, the bonus token is inserted, the parallel-drafting
    slots are filled with the MASK id, and the rejected-token mask, the
    masked-token mask and the hidden-state mapping are produced.
    [PF] "怎么做的", Input_i: the first prediction row pairs emb(new) with
    h_context; rows 2..K pair emb(mask) with h_shared.
    [PP] "Step 2: Parallel Drafting": each earlier position pairs its token
    embedding with the target hidden state shifted by one position.
    [PP] "KV Cache and CUDA Graphs": rejected tokens map to slot -1.

    Readings taken (the pages fix the fields but not the layout):
      * sequence i occupies draft rows D_i .. D_i+L_i+K-2 with
        D_i = sum_{j<i} L_j + i*(K-1);
      * rows 0..a_i copy the accepted rows (row r carries the token of verified
        row r+1 and sits at verified row r's position); row a_i carries the
        bonus token b_i (the NTP row);
      * the K-1 MASK rows follow directly at positions P_i+a_i+1 ..
        P_i+a_i+K-1 with P_i = target_pos of the sequence's first row;
      * the L_i-1-a_i rejected verified rows come last, keep their (shifted)
        ids and original positions, and get slot -1;
      * the K sampled rows are the NTP row and the MASK rows;
      * the sequence's KV length after the pass is target_pos[s+a_i] + K.

    ``compact``: the rejected rows are dropped instead of kept as slot -1
    rows, so sequence i owns a_i + K rows from D_i = sum_{j<i} (a_j + K);
    cu_draft[c] is the number of live rows and the arrays keep the fixed
    layout's length N, the rows past the live ones being inert padding (slot
    -1, flagged rejected, id = the sequence's bonus token, position 0); target
    rows past the accepted prefix map to -1 (no draft row inherits them).
    """
    query_lens = np.asarray(query_lens, dtype=np.int64)
    target_ids = np.asarray(target_ids, dtype=np.int64)
    target_pos = np.asarray(target_pos, dtype=np.int64)
    num_accepted = np.asarray(num_accepted, dtype=np.int64)
    bonus_ids = np.asarray(bonus_ids, dtype=np.int64)
    block_table = np.asarray(block_table, dtype=np.int64)
    c = len(query_lens)
    T = int(query_lens.sum())
    N = T + c * (K - 1)

    ids = np.zeros(N, np.int64)
    pos = np.zeros(N, np.int64)
    slot = np.zeros(N, np.int64)
    rej = np.zeros(N, np.uint8)
    msk = np.zeros(N, np.uint8)
    hmap = np.zeros(T, np.int64)
    cu_draft = np.zeros(c + 1, np.int64)
    kv_lens = np.zeros(c, np.int64)
    sample_idx = np.zeros(c * K, np.int64)

    s = 0
    live = int(num_accepted.sum()) + c * K if compact else N
    pad = live                                  # next padding row (compact)
    Dc = 0                                      # next live row (compact)
    for i in range(c):
        L = int(query_lens[i])
        a = int(num_accepted[i])
        b = int(bonus_ids[i])
        if not (0 <= a <= L - 1):
            raise ValueError(f"sequence {i}: accepted count {a} outside 0..{L - 1}")
        D = Dc if compact else s + i * (K - 1)
        cu_draft[i] = D
        base = int(target_pos[s + a])
        kv_lens[i] = base + K
        if compact:
            for r in range(L - 1 - a):          # this sequence's share of padding rows
                ids[pad] = b
                rej[pad] = 1
                slot[pad] = PADDING_SLOT_ID
                pad += 1
            Dc += a + K
        for r in range(a + K if compact else L + K - 1):
            row = D + r
            if r <= a:                          # accepted rows, then the bonus (NTP) row
                ids[row] = target_ids[s + r + 1] if r < a else b
                pos[row] = target_pos[s + r]
            elif r < a + K:                     # parallel-drafting MASK rows
                ids[row] = mask_id
                pos[row] = base + (r - a)
                msk[row] = 1
            else:                               # rejected verified rows
                j = r - (K - 1)
                ids[row] = target_ids[s + j + 1] if j + 1 < L else b
                pos[row] = target_pos[s + j]
                rej[row] = 1
            if rej[row]:
                slot[row] = PADDING_SLOT_ID
            else:
                p = int(pos[row])
                slot[row] = block_table[i, p // block_size] * block_size + p % block_size
        for j in range(L):
            hmap[s + j] = D + j if j <= a else (-1 if compact else D + j + K - 1)
        for k in range(K):
            sample_idx[i * K + k] = D + a + k
        s += L
    cu_draft[c] = live
    return dict(draft_ids=ids, draft_pos=pos, slot_mapping=slot, is_rejected=rej,
                is_masked=msk, hidden_map=hmap, cu_draft=cu_draft, kv_lens=kv_lens,
                sample_idx=sample_idx)


# ----------------------------------------------------------------------------
# Step 2: place target hidden states, broadcast h_shared into MASK rows
# ----------------------------------------------------------------------------
def scatter_broadcast(target_hidden: np.ndarray, hidden_map, is_masked, h_shared: np.ndarray,
                      num_rows: int) -> np.ndarray:
    """[PF] "vLLM中的工程实现细节" and [PP] "Hidden State Management": every
    target hidden row is copied to its mapped draft row, then every masked
    row receives the learned shared hidden state.  Works on any dtype (pure
    copies, bit-exact)."""
    target_hidden = np.asarray(target_hidden)
    out = np.zeros((num_rows,) + target_hidden.shape[1:], dtype=target_hidden.dtype)
    for t, r in enumerate(np.asarray(hidden_map)):
        if r >= 0:                      # -1: dropped (compacted layout)
            out[int(r)] = target_hidden[t]
    for r in range(num_rows):
        if is_masked[r]:
            out[r] = h_shared
    return out


# ----------------------------------------------------------------------------
# Step 3 building blocks
# ----------------------------------------------------------------------------
def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gain over the last axis."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * gain


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def rope_rotate_half(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary embedding, rotate-half pairing (j, j+d/2), angle pos * theta^(-2j/d).

    x: [rows, heads, d]; pos: [rows].  Positions must be the tokens' true
    positions ([PD] 6.1 warns that an off-by-one here silently ruins drafts).
    """
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def paged_attention(q: np.ndarray, q_pos: np.ndarray, keys: np.ndarray, values: np.ndarray) -> np.ndarray:
    """Causal-by-position grouped-query attention for the rows of one sequence.

    q: [rows, n_q, d]; keys/values: [kv_len, n_kv, d] with key j at position j.
    Row at position p sees keys 0..p; q head h reads kv head h // (n_q / n_kv).
    Scale 1/sqrt(d); softmax with max subtraction, all in float64.
    """
    rows, n_q, d = q.shape
    n_kv = keys.shape[1]
    grp = n_q // n_kv
    # per query head h: its kv head's keys and values (head-major for matmul)
    kh = np.repeat(keys, grp, axis=1).transpose(1, 2, 0)      # [n_q, d, kv_len]
    vh = np.repeat(values, grp, axis=1).transpose(1, 0, 2)    # [n_q, kv_len, d]
    qh = q.transpose(1, 0, 2)                                  # [n_q, rows, d]
    scores = np.matmul(qh, kh) / np.sqrt(d)                    # [n_q, rows, kv_len]
    kpos = np.arange(keys.shape[0])
    visible = kpos[None, None, :] <= np.asarray(q_pos)[None, :, None]
    scores = np.where(visible, scores, -np.inf)
    m = np.max(scores, axis=-1, keepdims=True)
    e = np.exp(scores - m)
    w = e / np.sum(e, axis=-1, keepdims=True)
    return np.matmul(w, vh).transpose(1, 0, 2)                 # [rows, n_q, d]


def _slots_of(block_table_row: np.ndarray, positions: np.ndarray, block_size: int) -> np.ndarray:
    return block_table_row[positions // block_size] * block_size + positions % block_size


def _matmul_t(x: np.ndarray, w_stored: np.ndarray, dtype: str, chunk: int = 16384) -> np.ndarray:
    """x @ W^T with W stored [out, in]; W widened to float64 in row chunks."""
    out = np.empty((x.shape[0], w_stored.shape[0]), dtype=np.float64)
    for lo in range(0, w_stored.shape[0], chunk):
        hi = min(w_stored.shape[0], lo + chunk)
        out[:, lo:hi] = x @ decode(w_stored[lo:hi], dtype).T
    return out


# ----------------------------------------------------------------------------
# Step 3: the single drafter pass
# ----------------------------------------------------------------------------
def draft_forward(spec, weights: dict, meta: Dict[str, np.ndarray], draft_hidden: np.ndarray,
                  block_table: np.ndarray, k_cache: Sequence[np.ndarray], v_cache: Sequence[np.ndarray],
                  K: int, precision: str = "mirror", seqs: Optional[Sequence[int]] = None,
                  want_logits: bool = True) -> dict:
    """All K draft tokens of every sequence from one pass.

    [PF] "怎么做的" and [PP] "Step 2: Parallel Drafting": all positions go
    through the drafter's transformer layer(s) and LM head together and the
    K draft tokens come out of that single pass.

    Reading of the drafter (the pages name only "N transformer layers and an
    LM head"): u = [emb(id) ; h] (concatenation order as in Input_i), x = W_fc u;
    per layer a Llama-style pre-norm block -- RMSNorm, q/k/v projections,
    rotate-half RoPE at the row's position, (k, v) written to the paged cache
    at the row's slot unless it is the padding slot, grouped-query attention
    over cache positions 0..p of the row's own sequence, output projection
    with residual, RMSNorm, SwiGLU MLP with residual; then RMSNorm and the LM
    head on the K sampled rows, greedy argmax with the lowest index on ties.
    All cache writes of a layer happen before its attention reads.

    ``seqs`` restricts the computation to a subset of sequences (they are
    independent), for sampled checks at full size.  Returns the tokens
    [len(seqs), K], the sampled logits (optional), the top-2 logit gap, the
    cache writes and per-row intermediates.
    """
    dt = spec.dtype
    H, nq, nkv, d = spec.hidden, spec.n_q, spec.n_kv, spec.head_dim
    c = len(meta["kv_lens"])
    seqs = list(range(c)) if seqs is None else [int(i) for i in seqs]
    cu = meta["cu_draft"]
    rows = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in seqs]).astype(np.int64)
    seq_of_row = np.concatenate([np.full(cu[i + 1] - cu[i], i) for i in seqs])
    ids = meta["draft_ids"][rows]
    pos = meta["draft_pos"][rows]
    slot = meta["slot_mapping"][rows]
    rnd = lambda v: round_operand(v, dt, precision)   # noqa: E731

    emb = decode(weights["embed"][ids], dt)
    hid = decode(np.asarray(draft_hidden)[rows], dt)
    u = np.concatenate([emb, hid], axis=1)
    x = _matmul_t(u, weights["w_fc"], dt)
    inter = {"x_fc": x.copy()}
    cache_writes = []
    for li, lw in enumerate(weights["layers"]):
        a = rnd(rms_norm(x, decode(lw["ln1"], dt), spec.rms_eps))
        q = _matmul_t(a, lw["wq"], dt).reshape(-1, nq, d)
        k = _matmul_t(a, lw["wk"], dt).reshape(-1, nkv, d)
        v = _matmul_t(a, lw["wv"], dt).reshape(-1, nkv, d)
        q = rnd(rope_rotate_half(q, pos, spec.rope_theta))
        k = rnd(rope_rotate_half(k, pos, spec.rope_theta))
        v = rnd(v)
        # cache writes of every non-rejected row first
        written = slot != PADDING_SLOT_ID
        w_slots = slot[written]
        cache_writes.append(dict(slots=w_slots, k=k[written], v=v[written]))
        kw, vw = k[written], v[written]
        order = np.argsort(w_slots, kind="stable")
        sorted_slots = w_slots[order]
        attn = np.zeros((len(rows), nq, d))
        for i in seqs:
            sel = np.nonzero(seq_of_row == i)[0]
            kp = np.arange(int(meta["kv_lens"][i]))
            sl = _slots_of(np.asarray(block_table[i], dtype=np.int64), kp, spec.block_size)
            keys = decode(k_cache[li][sl // spec.block_size, :, sl % spec.block_size, :], dt)
            vals = decode(v_cache[li][sl // spec.block_size, :, sl % spec.block_size, :], dt)
            if len(sorted_slots):
                hit = np.minimum(np.searchsorted(sorted_slots, sl), len(sorted_slots) - 1)
                own = sorted_slots[hit] == sl          # written in this pass
                keys[own] = kw[order[hit[own]]]
                vals[own] = vw[order[hit[own]]]
            attn[sel] = paged_attention(q[sel], pos[sel], keys, vals)
        attn = rnd(attn.reshape(len(rows), nq * d))
        x = x + _matmul_t(attn, lw["wo"], dt)
        m = rnd(rms_norm(x, decode(lw["ln2"], dt), spec.rms_eps))
        g = _matmul_t(m, lw["w_gate"], dt)
        up = _matmul_t(m, lw["w_up"], dt)
        h = rnd(silu(g) * up)
        x = x + _matmul_t(h, lw["w_down"], dt)
        inter[f"attn{li}"] = attn
        inter[f"x{li}"] = x.copy()

    # sampled rows: NTP row and MASK rows of each selected sequence
    local = {int(r): n for n, r in enumerate(rows)}
    samp = np.array([local[int(meta["sample_idx"][i * K + kk])] for i in seqs for kk in range(K)],
                    dtype=np.int64)
    f = rnd(rms_norm(x[samp], decode(weights["ln_f"], dt), spec.rms_eps))
    logits = _matmul_t(f, weights["w_lm"], dt)
    tokens = np.argmax(logits, axis=1)
    top = np.max(logits, axis=1)
    masked = logits.copy()
    masked[np.arange(len(samp)), tokens] = -np.inf
    gap = top - np.max(masked, axis=1)
    out = dict(tokens=tokens.reshape(len(seqs), K).astype(np.int64), top2_gap=gap.reshape(len(seqs), K),
               rows=rows, cache_writes=cache_writes, intermediates=inter, seqs=np.array(seqs))
    if want_logits:
        out["logits"] = logits.reshape(len(seqs), K, -1)
    return out


# ----------------------------------------------------------------------------
# Step 4: greedy acceptance
# ----------------------------------------------------------------------------
def accept(draft_tokens: np.ndarray, target_tokens: np.ndarray):
    """[PP] "Acceptance Length (AL)" and [PF] results: the accepted length is
    the number of draft tokens the verifier keeps in a round.  Under greedy
    verification that is the length of the longest prefix on which draft and
    target agree; the next target token becomes the new bonus token.

    draft_tokens [c, K]; target_tokens [c, K+1] -> (accepted [c], bonus [c]).
    """
    draft_tokens = np.asarray(draft_tokens)
    target_tokens = np.asarray(target_tokens)
    c, K = draft_tokens.shape
    acc = np.zeros(c, np.int64)
    bonus = np.zeros(c, np.int64)
    for i in range(c):
        n = 0
        while n < K and draft_tokens[i, n] == target_tokens[i, n]:
            n += 1
        acc[i] = n
        bonus[i] = target_tokens[i, n]
    return acc, bonus


# ----------------------------------------------------------------------------
# cache state across passes and rounds
# ----------------------------------------------------------------------------
def apply_cache_writes(spec, k_cache: Sequence[np.ndarray], v_cache: Sequence[np.ndarray],
                       cache_writes) -> None:
    """Store one pass's (k, v) writes into the caches (in place), in the
    cache dtype.  ``draft_forward`` overlays a pass's own writes when it reads
    the cache but leaves the arrays untouched; passes that build on earlier
    ones (the autoregressive baseline, later rounds) commit them here."""
    bs = spec.block_size
    for li, w in enumerate(cache_writes):
        sl = np.asarray(w["slots"], dtype=np.int64)
        if len(sl) == 0:
            continue
        k_cache[li][sl // bs, :, sl % bs, :] = encode(np.asarray(w["k"]), spec.dtype)
        v_cache[li][sl // bs, :, sl % bs, :] = encode(np.asarray(w["v"]), spec.dtype)


def next_verified_batch(kv_lens, bonus_ids, draft_tokens, num_accepted_next, bonus_next, K: int) -> dict:
    """The batch the next round drafts from ([PF] "怎么做的": every round the
    K drafts are verified by the target).  For sequence i the verifier saw
    the K+1 rows [bonus_i, d_0 .. d_{K-1}] at positions base_i+1 .. base_i+K+1
    (base_i = kv_lens[i] - K, the position of this round's bonus row) and
    kept num_accepted_next[i] drafts, with bonus_next[i] as the new bonus."""
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    drafts = np.asarray(draft_tokens, dtype=np.int64).reshape(len(kv_lens), K)
    ids, pos = [], []
    for i in range(len(kv_lens)):
        base = int(kv_lens[i]) - K
        ids.append(np.concatenate([[int(bonus_ids[i])], drafts[i]]))
        pos.append(base + 1 + np.arange(K + 1))
    c = len(kv_lens)
    return dict(query_lens=np.full(c, K + 1, np.int32), target_ids=np.concatenate(ids).astype(np.int32),
                target_pos=np.concatenate(pos).astype(np.int32),
                num_accepted=np.asarray(num_accepted_next, dtype=np.int32).copy(),
                bonus_ids=np.asarray(bonus_next, dtype=np.int32).copy())


# ----------------------------------------------------------------------------
# autoregressive baseline
# ----------------------------------------------------------------------------
def autoregressive_draft(spec, weights: dict, batch, K: int, precision: str = "mirror",
                         seqs: Optional[Sequence[int]] = None, forced_tokens: Optional[np.ndarray] = None,
                         forced_hidden: Optional[np.ndarray] = None) -> dict:
    """K drafts from K sequential one-token passes, the drafting scheme whose
    latency grows with K ([PP] "Solving the Autoregressive Drafting
    Bottleneck").

    Pass 0 is the parallel-draft pass with K = 1 over the verified batch (the
    bonus row, no MASK rows).  Pass k >= 1 has one row per sequence: token
    k-1 at position base+k (base = position of the bonus row), its hidden
    input being the drafter's own final residual (before the final RMSNorm)
    of the row that produced token k-1, stored in the model dtype -- the
    pages do not say which feature an autoregressive drafter feeds back; this
    reading takes the drafter's last hidden state.  Each pass's cache writes
    are committed before the next pass.

    ``forced_tokens`` [c, K] feeds those tokens forward instead of the
    oracle's own argmax, and ``forced_hidden`` [K-1, c, H] (storage dtype)
    those hidden rows instead of the oracle's own rounded residuals (teacher
    forcing against another implementation's drafts and fed-back states).
    Returns tokens and logits per step, the hidden rows the oracle itself
    would feed back ([K-1, len(seqs), H], storage dtype) and the final caches.
    """
    dt = spec.dtype
    c = len(batch.query_lens)
    seqs = list(range(c)) if seqs is None else [int(i) for i in seqs]
    kc = [np.array(k, copy=True) for k in batch.k_cache]
    vc = [np.array(v, copy=True) for v in batch.v_cache]
    last = f"x{spec.n_layers - 1}"
    meta = expand_batch(batch.query_lens, batch.target_ids, batch.target_pos, batch.num_accepted,
                        batch.bonus_ids, batch.block_table, 1, spec.mask_token_id, spec.block_size)
    hd = scatter_broadcast(batch.target_hidden, meta["hidden_map"], meta["is_masked"], weights["h_shared"],
                           len(meta["draft_ids"]))
    base = np.asarray(meta["kv_lens"], dtype=np.int64) - 1
    tokens = np.zeros((len(seqs), K), np.int64)
    logits = []
    own_hidden = []
    for k in range(K):
        f = draft_forward(spec, weights, meta, hd, batch.block_table, kc, vc, 1, precision=precision, seqs=seqs)
        apply_cache_writes(spec, kc, vc, f["cache_writes"])
        tokens[:, k] = f["tokens"][:, 0]
        logits.append(f["logits"][:, 0])
        if k == K - 1:
            break
        feed = tokens[:, k] if forced_tokens is None else np.asarray(forced_tokens)[seqs, k]
        local = {int(r): n for n, r in enumerate(f["rows"])}
        xs = f["intermediates"][last][[local[int(meta["sample_idx"][i])] for i in seqs]]
        ids = np.zeros(c, np.int32)
        hid = np.zeros((c, spec.hidden), dtype=np.uint16 if dt == "bf16" else np.float32)
        ids[seqs] = feed
        own_hidden.append(encode(xs, dt))
        hid[seqs] = own_hidden[-1] if forced_hidden is None else np.asarray(forced_hidden)[k][seqs]
        pos = (base + k + 1).astype(np.int32)
        slot = np.array([_slots_of(np.asarray(batch.block_table[i], dtype=np.int64), np.array([pos[i]]),
                                   spec.block_size)[0] for i in range(c)], dtype=np.int64)
        meta = dict(draft_ids=ids, draft_pos=pos, slot_mapping=slot, is_rejected=np.zeros(c, np.uint8),
                    is_masked=np.zeros(c, np.uint8), cu_draft=np.arange(c + 1, dtype=np.int32),
                    kv_lens=(pos.astype(np.int64) + 1).astype(np.int32), sample_idx=np.arange(c, dtype=np.int32))
        hd = hid
    hdt = np.uint16 if dt == "bf16" else np.float32
    fed = np.stack(own_hidden) if own_hidden else np.zeros((0, len(seqs), spec.hidden), hdt)
    return dict(tokens=tokens, logits=np.stack(logits, axis=1), fed_hidden=fed, k_cache=kc, v_cache=vc,
                seqs=np.array(seqs))


# ----------------------------------------------------------------------------
# whole round
# ----------------------------------------------------------------------------
def parallel_draft_step(spec, weights: dict, batch, precision: str = "mirror",
                        seqs: Optional[Sequence[int]] = None, want_logits: bool = True,
                        compact: bool = False) -> dict:
    """Expand, place hidden states, run the drafter pass (no acceptance)."""
    meta = expand_batch(batch.query_lens, batch.target_ids, batch.target_pos, batch.num_accepted,
                        batch.bonus_ids, batch.block_table, batch.K, spec.mask_token_id,
                        spec.block_size, compact=compact)
    hd = scatter_broadcast(batch.target_hidden, meta["hidden_map"], meta["is_masked"],
                           weights["h_shared"], len(meta["draft_ids"]))
    fwd = draft_forward(spec, weights, meta, hd, batch.block_table, batch.k_cache, batch.v_cache,
                        batch.K, precision=precision, seqs=seqs, want_logits=want_logits)
    return dict(meta=meta, draft_hidden=hd, forward=fwd)

