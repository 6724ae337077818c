"""Parallel-draft step benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one whole parallel-draft round on a seeded synthetic batch whose
inputs already sit in HBM: batch expansion + hidden placement
(prepare_draft_batch), the single drafter pass with LM head and argmax
(draft_forward) and greedy acceptance (accept).  The value is draft tokens
per second (c * K tokens per step).  One JSON line is printed, with the
roofline of the dominant kernel (the LM head) measured with HIP events on its
own stream during the timed steps, and the CPU oracle timed on the host on a
bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft tokens/s per parallel-draft step (K=7, c=1/64); % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lm_head_traffic.json")
DEFAULT_WORKLOAD = "gptoss20b-bf16-c1-k7"
COPY_BYTES = 1 << 30


def _src_hash(files) -> str:
    """Hash of the kernel sources a traffic record was measured with."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "drafting_draft_expand_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def lm_head_bytes(spec, S: int) -> int:
    """Algorithmic HBM bytes of one LM-head launch: every vocabulary row of the
    weight once (H elements each) plus the S normalised activation rows."""
    eb = 4 if spec.dtype == "fp32" else 2
    return spec.vocab * spec.hidden * eb + S * spec.hidden * eb


def step_bytes(spec, wl, b) -> int:
    """Algorithmic bytes of one whole round (weights once, KV read once per
    (sequence, kv head), hidden/metadata once)."""
    eb = 4 if spec.dtype == "fp32" else 2
    H, d = spec.hidden, spec.head_dim
    qd, kvd = spec.n_q * d, spec.n_kv * d
    w = 2 * H * H + spec.n_layers * (H * (qd + 2 * kvd) + qd * H + 3 * H * spec.inter) + spec.vocab * H
    kv_read = 0
    for i in range(b.c):
        kv_len = int(b.target_pos[int(b.query_lens[:i].sum()) + int(b.num_accepted[i])]) + b.K
        kv_read += kv_len * kvd * 2 * spec.n_layers
    T, N = b.T, b.N
    hid = (T * H + N * H) * eb          # placement read + write
    emb = N * H * eb                     # embedding rows gathered
    return (w + kv_read) * eb + hid + emb


def _cpu_baseline(wl, w, b, budget_s: float, mode: str = "peagle"):
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    u, alt = __import__("synth").make_agreement_draws(wl)
    rounds = 0
    t0 = time.perf_counter()
    while True:
        if mode == "ar":
            drafts = oracle.autoregressive_draft(wl.model, w, b, wl.K)["tokens"]
        else:
            drafts = oracle.parallel_draft_step(wl.model, w, b, want_logits=False)["forward"]["tokens"]
        tgt = __import__("synth").target_tokens_from_drafts(drafts, u, alt, wl.agree_probs(), wl.model.vocab)
        oracle.accept(drafts, tgt)
        rounds += 1
        el = time.perf_counter() - t0
        if el >= budget_s or rounds >= 20:
            break
    del np
    return dict(value=round(rounds * wl.c * wl.K / el, 3), unit="draft tokens/s", cores=int(threads),
                kind="oracle",
                sample=f"{rounds} full round(s) of {wl.name} through the float64 oracle "
                       + ("(K one-token drafter passes, argmax, acceptance)" if mode == "ar" else
                          "(expand, placement, drafter pass, argmax, acceptance)") + f", {el:.1f} s")


def _calibrate_copy() -> int:
    """A plain device-to-device copy of known size: each launch reads and
    writes COPY_BYTES, so the FETCH_SIZE / WRITE_SIZE counters it produces give
    the factor between those counters and true HBM bytes."""
    import torch
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0").uniform_()
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_per_launch": COPY_BYTES, "launches": 5}))
    return 0


PREP_WORKLOAD = "prep-bf16-c64-k7-h2880"
PREP_SETS = 64


def prep_bytes(spec, b, K) -> int:
    """Algorithmic bytes of one expansion + placement: target hidden rows read
    once, draft hidden rows written once, the metadata read and written once
    (one block-table entry per draft row)."""
    eb = 4 if spec.dtype == "fp32" else 2
    c, T, N = b.c, b.T, b.N
    meta = 4 * 3 * c + 8 * T + 4 * N + N * (4 + 4 + 8 + 1 + 1) + 4 * T + 4 * (c + 1) + 4 * c + 4 * c * K
    return (T + N) * spec.hidden * eb + meta


def _bench_prep(args) -> int:
    """Time pe_prepare_draft_batch alone.  Every step uses the next of
    PREP_SETS buffer sets (target hidden rows in, draft rows out), so the
    working set (PREP_SETS x ~8 MB) exceeds the 256 MB memory-side cache and
    every step reads and writes HBM."""
    import torch
    import drafting_draft_expand_amd as pe
    import synth
    from synth.device import upload_batch, upload_weights

    wl = synth.WORKLOADS[PREP_WORKLOAD if args.workload == DEFAULT_WORKLOAD else args.workload]
    spec, K = wl.model, wl.K
    dev = "cuda:0"
    w = synth.make_weights(spec, wl.wseed, prep_only=True)
    dw = upload_weights(w, dev)
    model = pe.DraftModel(spec.hidden, spec.vocab, 0, 1, 1, 16, 8, spec.dtype, dw, mask_token_id=spec.mask_token_id)
    b = synth.make_batch(wl)
    db = upload_batch(b, dev)
    stream = torch.cuda.current_stream()
    hid = [db["target_hidden"].clone() for _ in range(PREP_SETS)]
    outs = []
    for s in range(PREP_SETS):
        outs.append(pe.prepare_draft_batch(model, K, db["query_lens"], db["target_ids"], db["target_pos"],
                                           db["num_accepted"], db["bonus_ids"], hid[s], db["block_table"],
                                           stream=stream))
    torch.cuda.synchronize()
    it = [0]

    def step():
        s = it[0] % PREP_SETS
        it[0] += 1
        pe.prepare_draft_batch(model, K, db["query_lens"], db["target_ids"], db["target_pos"], db["num_accepted"],
                               db["bonus_ids"], hid[s], db["block_table"], out=outs[s], stream=stream)

    for _ in range(args.warmup):
        step()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pe.timing_enable(pe.PE_KERNEL_PREPARE, True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    k_ms, k_n, _ = pe.timing_read(pe.PE_KERNEL_PREPARE)
    pe.timing_enable(pe.PE_KERNEL_PREPARE, False)
    k_s = k_ms / max(k_n, 1) / 1e3
    nbytes = prep_bytes(spec, b, K)
    gbs = nbytes / (ms / 1e3) / 1e9
    print(f"# prep {wl.name}: {ms * 1e3:.2f} us/step launch-inclusive, {k_s * 1e6:.2f} us per launch (events)",
          file=sys.stderr, flush=True)
    out = {
        "metric": "draft-batch expansion + hidden placement throughput (a1-a3)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "launch_mode": "eager",
        "mode": "prep",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if spec.dtype == "bf16" else "f32",
        "data": f"synthetic: N(0,1) target hidden states and h_shared, uniform accepted counts, "
                f"{PREP_SETS} rotated buffer sets",
        "config": {"workload": wl.name, "num_seqs": b.c, "draft_depth": K, "target_rows": b.T, "draft_rows": b.N,
                   "hidden": spec.hidden},
        "roofline": {"bound": "hbm", "kernel": "prepare", "achieved": round(nbytes / k_s / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(nbytes / k_s / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": None, "algorithmic_bytes": nbytes, "avg_launch_us": round(k_s * 1e6, 2),
                     "launches": k_n},
    }
    model.close()
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--eager", action="store_true", help="time eager launches only (no HIP graph replay)")
    ap.add_argument("--mode", choices=("peagle", "ar", "loop", "prep"), default="peagle",
                    help="peagle: one parallel-draft round per step; ar: the K-pass autoregressive baseline "
                         "on the same kernels; loop: rounds chained through the device-built next batch; "
                         "prep: the batch expansion and hidden placement alone (default workload "
                         f"{PREP_WORKLOAD}), over {PREP_SETS} rotated buffer sets")
    ap.add_argument("--layout", choices=("fixed", "compact"), default="fixed",
                    help="draft layout: fixed (rejected rows kept as inert rows) or compact (dropped)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy five times (reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        return 2
    if args.calibrate_copy:
        return _calibrate_copy()
    if args.mode == "prep":
        return _bench_prep(args)

    import torch
    import drafting_draft_expand_amd as pe
    import synth
    from synth.device import to_torch, upload_batch, upload_weights

    wl = synth.WORKLOADS[args.workload]
    spec = wl.model
    dev = "cuda:0"
    t_setup = time.perf_counter()
    w = synth.make_weights(spec, wl.wseed)
    # the chained loop advances every sequence by up to K+1 positions a round
    b = synth.make_batch(wl, extra_positions=(args.steps + args.warmup + 2) * (wl.K + 1) if args.mode == "loop"
                         else 0)
    dw = upload_weights(w, dev)
    db = upload_batch(b, dev)
    model = pe.DraftModel.from_spec(spec, dw)
    rng = __import__("numpy").random.default_rng(wl.seed + 99)
    tgt = to_torch(rng.integers(0, spec.vocab - 1, size=(wl.c, wl.K + 1)), device=dev)
    c, K, T, N = wl.c, wl.K, b.T, b.N
    compact = args.layout == "compact"
    prep = pe.prepare_draft_batch(model, K, db["query_lens"], db["target_ids"], db["target_pos"],
                                  db["num_accepted"], db["bonus_ids"], db["target_hidden"], db["block_table"],
                                  compact=compact)
    ws = torch.empty(model.workspace_bytes(c, K, N), dtype=torch.uint8, device=dev)
    tokens = torch.empty((c, K), dtype=torch.int32, device=dev)
    acc = torch.empty(c, dtype=torch.int32, device=dev)
    bonus = torch.empty(c, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    print(f"# setup {time.perf_counter() - t_setup:.1f}s workload={wl.name} N={N} T={T}", file=sys.stderr,
          flush=True)

    def step():
        pe.prepare_draft_batch(model, K, db["query_lens"], db["target_ids"], db["target_pos"], db["num_accepted"],
                               db["bonus_ids"], db["target_hidden"], db["block_table"], out=prep, stream=stream,
                               compact=compact)
        pe.draft_forward(model, prep, db["block_table"], db["k_cache"], db["v_cache"], workspace=ws,
                         tokens=tokens, stream=stream)
        pe.accept(tokens, tgt, acc, bonus, stream=stream)

    if args.mode == "ar":
        ar_ws = torch.empty(model.autoregressive_workspace_bytes(c, K, T), dtype=torch.uint8, device=dev)

        def step():  # noqa: F811 -- K one-token passes instead of one parallel pass
            pe.draft_autoregressive(model, K, db["query_lens"], db["target_ids"], db["target_pos"],
                                    db["num_accepted"], db["bonus_ids"], db["target_hidden"], db["block_table"],
                                    db["k_cache"], db["v_cache"], workspace=ar_ws, tokens=tokens, stream=stream)
            pe.accept(tokens, tgt, acc, bonus, stream=stream)
    elif args.mode == "loop":
        # rounds chained on the device: accept's outputs and the next verified
        # batch feed the next prepare; the verifier's tokens and hidden states
        # are fixed synthetic buffers (the target model is not part of the path)
        cur = {k: db[k] for k in ("query_lens", "target_ids", "target_pos", "num_accepted", "bonus_ids")}
        nxt = pe.next_verified_batch(K, prep["kv_lens"], cur["bonus_ids"], tokens, acc, bonus)
        hid_next = db["target_hidden"]

        def step():  # noqa: F811
            pe.prepare_draft_batch(model, K, cur["query_lens"], cur["target_ids"], cur["target_pos"],
                                   cur["num_accepted"], cur["bonus_ids"], hid_next, db["block_table"], out=prep,
                                   stream=stream, compact=compact)
            pe.draft_forward(model, prep, db["block_table"], db["k_cache"], db["v_cache"], workspace=ws,
                             tokens=tokens, stream=stream)
            pe.accept(tokens, tgt, acc, bonus, stream=stream)
            pe.next_verified_batch(K, prep["kv_lens"], cur["bonus_ids"], tokens, acc, bonus, out=nxt, stream=stream)
            for k in cur:
                cur[k].copy_(nxt[k])

    def timed(fn, n):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(n):
            fn()
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / n

    # eager launches: every step goes through the C ABI; the LM-head kernel is
    # timed with HIP events on its own stream over these steps
    for _ in range(args.warmup):
        step()
    pe.timing_enable(pe.PE_KERNEL_LM_HEAD, True)
    eager_ms = timed(step, args.steps)
    lm_ms, lm_n, _ = pe.timing_read(pe.PE_KERNEL_LM_HEAD)
    pe.timing_enable(pe.PE_KERNEL_LM_HEAD, False)
    ms_per_step, mode = eager_ms, "eager"
    graph_ms = None
    if not args.eager and args.mode == "peagle":
        # the same round captured once into a HIP graph and replayed (the
        # deployment form: fixed shapes, one submission per round)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            pe.prepare_draft_batch(model, K, db["query_lens"], db["target_ids"], db["target_pos"],
                                   db["num_accepted"], db["bonus_ids"], db["target_hidden"], db["block_table"],
                                   out=prep, compact=compact)
            pe.draft_forward(model, prep, db["block_table"], db["k_cache"], db["v_cache"], workspace=ws,
                             tokens=tokens)
            pe.accept(tokens, tgt, acc, bonus)
        for _ in range(args.warmup):
            graph.replay()
        graph_ms = timed(graph.replay, args.steps)
        ms_per_step, mode = graph_ms, "hip_graph"
    value = c * K / (ms_per_step / 1e3)
    print(f"# timed {args.steps} steps: eager {eager_ms * 1e3:.1f} us/step, graph "
          f"{'-' if graph_ms is None else f'{graph_ms * 1e3:.1f}'} us/step; "
          f"lm-head {lm_ms / max(lm_n, 1) * 1e3:.1f} us x {lm_n}", file=sys.stderr, flush=True)

    lm_avg_s = lm_ms / max(lm_n, 1) / 1e3
    lm_b = lm_head_bytes(spec, c * K)
    lm_f = 2.0 * c * K * spec.vocab * spec.hidden
    # the LM head is HBM-bound below the ridge (peak flops / peak bytes) and
    # MFMA-bound above it (c=64: 448 rows, ~447 flop/B)
    mfma_bound = spec.dtype == "bf16" and lm_f / lm_b > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        achieved, peak, unit = lm_f / lm_avg_s / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = lm_b / lm_avg_s / 1e9, HBM_PEAK_GBS, "GB/s"
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tf = json.load(open(TRAFFIC_FILE))
        rec = tf.get(wl.name)
        if rec and rec.get("src_hash") == _src_hash(rec.get("sources", [])):
            traffic = rec.get("bytes_per_launch")
    sb = step_bytes(spec, wl, b) * (K if args.mode == "ar" else 1)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "launch_mode": mode,
        "mode": args.mode,
        "layout": args.layout,
        "eager_ms_per_step": round(eager_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if spec.dtype == "bf16" else "f32",
        "data": "synthetic: seeded N(0,0.02) weights, N(0,1) target hidden states and cached KV, "
                "uniform accepted counts",
        "config": {"workload": wl.name, "num_seqs": c, "draft_depth": K, "draft_rows": N, "sampled_rows": c * K,
                   "hidden": spec.hidden, "vocab": spec.vocab, "layers": spec.n_layers,
                   "q_heads": spec.n_q, "kv_heads": spec.n_kv, "head_dim": spec.head_dim,
                   "intermediate": spec.inter, "context": [int(b.context.min()), int(b.context.max())]},
        "roofline": {"bound": "mfma" if mfma_bound else "hbm", "kernel": "lm_head_argmax",
                     "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic, "algorithmic_bytes": lm_b,
                     "algorithmic_flops": lm_f, "avg_launch_us": round(lm_avg_s * 1e6, 2), "launches": lm_n},
        "step_roofline": {"bound": "hbm", "algorithmic_bytes": sb,
                          "achieved": round(sb / (ms_per_step / 1e3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(sb / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = _cpu_baseline(wl, w, b, args.cpu_budget, args.mode)
    model.close()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
