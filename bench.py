"""Parallel-draft step benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one whole parallel-draft round on a seeded synthetic batch whose
inputs already sit in HBM: batch expansion + hidden placement
(prepare_draft_batch), the single drafter pass with LM head and argmax
(draft_forward) and greedy acceptance (accept), captured once into a HIP graph
and replayed.  The value is draft tokens per second (c * K tokens per step)
from the median step time.  Consecutive steps rotate over --sets full copies
of the weights (with their packed copies), the batch and the KV cache, so no
step finds the previous step's data in the 256 MB memory-side cache; the same
figures without rotation are reported as "warm".

One JSON line is printed: the headline workload (GPT-OSS-20B-shaped drafter,
one sequence, K=7), the roofline of its dominant kernel (the LM head) from HIP
events recorded around that kernel's launches on its own stream during timed
steps, the whole step against max(bytes / HBM peak, flops / bf16 peak), the
same drafter at 64 sequences as the "c64" object (the c=64 half of the
metric), and the CPU oracle timed on the host on a bounded sample of the
headline workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
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


def step_flops(spec, b) -> float:
    """Algorithmic flops of one round over the valid rows (accepted rows, the
    bonus row and the MASK rows; rejected rows excluded): fc, every layer's
    projections, attention of each row over its visible positions (q k^T and
    P V), and the LM head over the c*K sampled rows."""
    H, d = spec.hidden, spec.head_dim
    qd, kvd = spec.n_q * d, spec.n_kv * d
    per_row = 2.0 * (H * 2 * H + spec.n_layers * (H * (qd + 2 * kvd) + qd * H + 3 * H * spec.inter))
    rows, attn, s = 0, 0.0, 0
    for i in range(b.c):
        a = int(b.num_accepted[i])
        p0 = int(b.target_pos[s])
        n = a + b.K                       # valid rows of the sequence, positions p0 .. p0 + n - 1
        rows += n
        visible = sum(p0 + r + 1 for r in range(n))
        attn += 4.0 * spec.n_q * d * visible * spec.n_layers
        s += int(b.query_lens[i])
    return rows * per_row + attn + 2.0 * b.c * b.K * spec.vocab * H


def step_roofline(spec, b, ms: float, mult: int = 1) -> dict:
    """The whole step against max(bytes / HBM peak, flops / bf16 peak)."""
    nbytes = step_bytes(spec, None, b) * mult
    flops = step_flops(spec, b) * mult
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (BF16_PEAK_TFLOPS * 1e12)
    t = ms / 1e3
    return {"bound": "hbm" if t_hbm >= t_mfma else "mfma", "algorithmic_bytes": nbytes,
            "algorithmic_flops": flops, "roofline_us": round(max(t_hbm, t_mfma) * 1e6, 2),
            "achieved_gbs": round(nbytes / t / 1e9, 1), "achieved_tflops": round(flops / t / 1e12, 1),
            "frac": round(max(t_hbm, t_mfma) / t, 4)}


def _cpu_info() -> dict:
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0))}


def _oracle_rounds(wl, w, b, budget_s: float, mode: str, max_rounds: int = 20):
    import oracle
    import synth
    u, alt = synth.make_agreement_draws(wl)
    rounds = 0
    t0 = time.perf_counter()
    while True:
        if mode == "ar":
            drafts = oracle.autoregressive_draft(wl.model, w, b, wl.K)["tokens"]
        else:
            drafts = oracle.parallel_draft_step(wl.model, w, b, want_logits=False)["forward"]["tokens"]
        tgt = synth.target_tokens_from_drafts(drafts, u, alt, wl.agree_probs(), wl.model.vocab)
        oracle.accept(drafts, tgt)
        rounds += 1
        el = time.perf_counter() - t0
        if el >= budget_s or rounds >= max_rounds:
            return rounds, el


def _cpu_baseline(wl, w, b, budget_s: float, mode: str = "peagle", single_budget_s: float = 8.0):
    """The float64 oracle on the host: whole rounds of the workload with every
    BLAS thread the process may use, then with one thread."""
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threadpool_limits, threads = None, 1
    rounds, el = _oracle_rounds(wl, w, b, budget_s, mode)
    what = ("(K one-token drafter passes, argmax, acceptance)" if mode == "ar" else
            "(expand, placement, drafter pass, argmax, acceptance)")
    out = dict(value=round(rounds * wl.c * wl.K / el, 3), unit="draft tokens/s", cores=int(threads),
               kind="oracle",
               sample=f"{rounds} full round(s) of {wl.name} through the float64 oracle {what}, {el:.1f} s, "
                      f"{threads} BLAS threads")
    out.update(_cpu_info())
    if threadpool_limits is not None and single_budget_s > 0:
        with threadpool_limits(limits=1):
            r1, e1 = _oracle_rounds(wl, w, b, single_budget_s, mode)
        out["single_core"] = {"value": round(r1 * wl.c * wl.K / e1, 3), "unit": "draft tokens/s", "cores": 1,
                              "sample": f"{r1} round(s), {e1:.1f} s, one BLAS thread"}
    return out


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


def _clone(x):
    """Deep copy of a (nested) structure of device tensors."""
    import torch
    if isinstance(x, torch.Tensor):
        return x.clone()
    if isinstance(x, dict):
        return {k: _clone(v) for k, v in x.items()}
    if isinstance(x, list):
        return [_clone(v) for v in x]
    return x


def _timed(fns, n: int, stream) -> dict:
    """Run fns[i % len(fns)] for i < n with an event after each; per-step times
    from consecutive events (median reported), total from the first to the last."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(n):
        fns[i % len(fns)]()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(n)]
    return {"median_ms": statistics.median(per), "mean_ms": evs[0].elapsed_time(evs[n]) / n,
            "min_ms": min(per), "max_ms": max(per)}


def _launch_stats(kernel) -> dict:
    import drafting_draft_expand_amd as pe
    total, n, per = pe.timing_read(kernel)
    return {"mean_ms": total / max(n, 1), "median_ms": statistics.median(per) if per else 0.0, "launches": n}


class Bench:
    """One workload on --sets rotated copies of everything a round reads."""

    def __init__(self, pe, wl, w, models, args, dev, extra_positions=0):
        import numpy as np
        import torch
        import synth
        from synth.device import to_torch, upload_batch
        self.pe, self.wl, self.spec, self.args = pe, wl, wl.model, args
        self.b = synth.make_batch(wl, extra_positions=extra_positions)
        db0 = upload_batch(self.b, dev)
        rng = np.random.default_rng(wl.seed + 99)
        self.tgt = to_torch(rng.integers(0, self.spec.vocab - 1, size=(wl.c, wl.K + 1)), device=dev)
        self.compact = args.layout == "compact"
        c, K, N = wl.c, wl.K, self.b.N
        self.stream = torch.cuda.current_stream()
        self.sets = []
        for s, model in enumerate(models):
            db = db0 if s == 0 else _clone(db0)
            prep = pe.prepare_draft_batch(model, K, db["query_lens"], db["target_ids"], db["target_pos"],
                                          db["num_accepted"], db["bonus_ids"], db["target_hidden"],
                                          db["block_table"], compact=self.compact)
            self.sets.append(dict(
                model=model, db=db, prep=prep,
                ws=torch.empty(model.workspace_bytes(c, K, N), dtype=torch.uint8, device=dev),
                tokens=torch.empty((c, K), dtype=torch.int32, device=dev),
                acc=torch.empty(c, dtype=torch.int32, device=dev),
                bonus=torch.empty(c, dtype=torch.int32, device=dev)))
        torch.cuda.synchronize()

    def round_fn(self, st, mode):
        pe, K, db = self.pe, self.wl.K, st["db"]
        stream = self.stream if mode != "capture" else None

        def run():
            pe.prepare_draft_batch(st["model"], K, db["query_lens"], db["target_ids"], db["target_pos"],
                                   db["num_accepted"], db["bonus_ids"], db["target_hidden"], db["block_table"],
                                   out=st["prep"], stream=stream, compact=self.compact)
            pe.draft_forward(st["model"], st["prep"], db["block_table"], db["k_cache"], db["v_cache"],
                             workspace=st["ws"], tokens=st["tokens"], stream=stream)
            pe.accept(st["tokens"], self.tgt, st["acc"], st["bonus"], stream=stream)
        return run

    def ar_fn(self, st, mode):
        import torch
        pe, K, db, b = self.pe, self.wl.K, st["db"], self.b
        if "ar_ws" not in st:
            st["ar_ws"] = torch.empty(st["model"].autoregressive_workspace_bytes(b.c, K, b.T), dtype=torch.uint8,
                                      device=st["tokens"].device)
        stream = self.stream if mode != "capture" else None

        def run():
            pe.draft_autoregressive(st["model"], K, db["query_lens"], db["target_ids"], db["target_pos"],
                                    db["num_accepted"], db["bonus_ids"], db["target_hidden"], db["block_table"],
                                    db["k_cache"], db["v_cache"], workspace=st["ar_ws"], tokens=st["tokens"],
                                    stream=stream)
            pe.accept(st["tokens"], self.tgt, st["acc"], st["bonus"], stream=stream)
        return run

    def graphs(self, make):
        import torch
        out = []
        for st in self.sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                make(st, "capture")()
            out.append(g.replay)
        torch.cuda.synchronize()
        return out

    def run(self, make, graph: bool, lm_kernel: bool = True) -> dict:
        """Warm-up, then the timed steps: eager launches (with the LM-head
        launches timed) and, with graph, the same rounds replayed from HIP
        graphs; rotated over every set and on the first set alone ("warm")."""
        import drafting_draft_expand_amd as pe
        args = self.args
        eager = [make(st, "eager") for st in self.sets]
        for i in range(args.warmup):
            eager[i % len(eager)]()
        if lm_kernel:
            pe.timing_enable(pe.PE_KERNEL_LM_HEAD, True)
        res = {"eager": _timed(eager, args.steps, self.stream)}
        if lm_kernel:
            res["lm_head"] = _launch_stats(pe.PE_KERNEL_LM_HEAD)
            pe.timing_enable(pe.PE_KERNEL_LM_HEAD, False)
        if graph:
            reps = self.graphs(make)
            for i in range(args.warmup):
                reps[i % len(reps)]()
            res["graph"] = _timed(reps, args.steps, self.stream)
            res["graph_warm"] = _timed(reps[:1], args.steps, self.stream)
        res["eager_warm"] = _timed(eager[:1], args.steps, self.stream)
        return res

    def mean_accepted(self, rounds: int) -> dict:
        """Mean accepted length of the GPU's own drafts when the synthetic target
        agrees with draft d with probability p_d (fresh draws every round),
        against the closed form sum_j prod_{d<j} p_d."""
        import numpy as np
        import synth
        from synth.device import from_torch, to_torch
        st, wl = self.sets[0], self.wl
        rng = np.random.default_rng(np.random.SeedSequence([wl.seed, 7301]))
        p = wl.agree_probs()
        accs = []
        for _ in range(rounds):
            self.round_fn(st, "eager")()
            drafts = from_torch(st["tokens"]).astype(np.int64)
            u = rng.random((wl.c, wl.K))
            alt = rng.integers(0, wl.model.vocab - 2, size=(wl.c, wl.K + 1))
            tgt = synth.target_tokens_from_drafts(drafts, u, alt, p, wl.model.vocab)
            acc, _ = self.pe.accept(st["tokens"], to_torch(tgt, device=st["tokens"].device))
            accs.append(from_torch(acc).copy())
        a = np.concatenate(accs).astype(np.float64)
        closed = float(sum(np.prod(p[:j]) for j in range(1, wl.K + 1)))
        return {"value": round(float(a.mean()), 4), "stderr": round(float(a.std() / np.sqrt(len(a))), 4),
                "closed_form": round(closed, 4), "samples": int(len(a)),
                "agreement": f"p_d = {wl.agree_p0} * {wl.agree_decay}^d"}


def _lm_roofline(spec, S, lm) -> dict:
    s = lm["mean_ms"] / 1e3
    nbytes = lm_head_bytes(spec, S)
    flops = 2.0 * S * spec.vocab * spec.hidden
    mfma = spec.dtype == "bf16" and flops / nbytes > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if mfma:
        achieved, peak, unit = flops / s / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = nbytes / s / 1e9, HBM_PEAK_GBS, "GB/s"
    return {"bound": "mfma" if mfma else "hbm", "kernel": "lm_head_argmax", "achieved": round(achieved, 1),
            "peak": peak, "unit": unit, "frac": round(achieved / peak, 4), "algorithmic_bytes": nbytes,
            "algorithmic_flops": flops, "avg_launch_us": round(lm["mean_ms"] * 1e3, 2),
            "median_launch_us": round(lm["median_ms"] * 1e3, 2), "launches": lm["launches"]}


def _traffic(name):
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE)).get(name)
    if rec and rec.get("src_hash") == _src_hash(rec.get("sources", [])):
        return rec.get("bytes_per_launch")
    return None


C64_WORKLOAD = "gptoss20b-bf16-c64-k7"


def _short_kernel(n: str) -> str:
    import re
    n = re.sub(r"\(pe::GemvArgs.*|\(pe::AttnArgs.*|\(pe::PrepareArgs.*|\(int,.*|\(pe::Top2.*|\(pe::PackArgs.*", "", n)
    n = n.replace("void ", "").replace("pe::(anonymous namespace)::", "").replace("(pe::Epi)", "E")
    return n.replace("(pe::AMode)", "A").replace("unsigned short", "bf16")[:72]


def _summarize_trace(paths) -> int:
    """Markdown table of a rocprofv3 kernel trace (run_kernel_trace.csv): the
    rounds (each starts at the expansion kernel), grouped by kernel sequence,
    with the median duration of the kernel at each position."""
    import csv
    from collections import defaultdict
    for path in paths:
        rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))
        rounds, cur = [], None
        for r in rows:
            if "prepare_kernel" in r["Kernel_Name"]:
                cur = []
                rounds.append(cur)
            if cur is not None:
                threads = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
                wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
                cur.append((_short_kernel(r["Kernel_Name"]), threads, wg, int(r["Start_Timestamp"]),
                            int(r["End_Timestamp"])))
        groups = defaultdict(list)
        for rd in rounds:
            groups[tuple((k[0], k[1]) for k in rd)].append(rd)
        print(f"Trace `{path}`\n")
        for sig, rds in sorted(groups.items(), key=lambda kv: -len(kv[1])):
            if len(rds) < 3:
                continue
            span = statistics.median([(rd[-1][4] - rd[0][3]) / 1e3 for rd in rds])
            print(f"{len(rds)} rounds of {len(sig)} kernels; median round span {span:.1f} us (first start to "
                  f"last end)\n")
            print("| # | kernel | workgroups x threads | median us | % of round |")
            print("|---:|---|---:|---:|---:|")
            for i, (name, grid) in enumerate(sig):
                d = statistics.median([(rd[i][4] - rd[i][3]) / 1e3 for rd in rds])
                print(f"| {i} | `{name}` | {grid // rds[0][i][2]} x {rds[0][i][2]} | {d:.2f} | {100 * d / span:.1f} |")
            print()
    return 0


def _summarize_counters(paths) -> int:
    """Markdown table of rocprofv3 --pmc runs (run_counter_collection.csv): per
    kernel (name and grid), the median value per dispatch of every counter,
    with MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD * SIMDs)
    (GRBM_GUI_ACTIVE comes summed over the XCDs, each of which counts the
    kernel's cycles) and MFMA FLOPs = SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512 where
    those were counted."""
    import csv
    from collections import defaultdict
    vals = defaultdict(lambda: defaultdict(list))
    simds, xcc = None, 1
    for path in paths:
        for r in csv.DictReader(open(path)):
            key = (_short_kernel(r["Kernel_Name"]), r.get("Grid_Size", ""))
            vals[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
    for path in paths:
        info = os.path.join(os.path.dirname(path), os.path.basename(path).replace("counter_collection", "agent_info"))
        if os.path.exists(info):
            for r in csv.DictReader(open(info)):
                if r.get("Agent_Type", "").endswith("GPU") and r.get("Simd_Count"):
                    simds = int(r["Simd_Count"])
                    xcc = int(r.get("Num_Xcc") or 1)
    names = sorted({c for v in vals.values() for c in v})
    head = ["kernel", "grid"] + names
    derived = []
    if "SQ_VALU_MFMA_BUSY_CYCLES" in names and "GRBM_GUI_ACTIVE" in names and simds:
        derived.append("MfmaUtil %")
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in names:
        derived.append("MFMA GFLOP")
    print("| " + " | ".join(head + derived) + " |")
    print("|" + "---|" * 2 + "---:|" * (len(names) + len(derived)))
    for (k, grid), cv in sorted(vals.items(), key=lambda kv: -max((sum(v) for v in kv[1].values()), default=0)):
        med = {c: statistics.median(v) for c, v in cv.items()}
        cells = [f"`{k}`", grid] + [f"{med[c]:.6g}" if c in med else "" for c in names]
        if "MfmaUtil %" in derived:
            busy, act = med.get("SQ_VALU_MFMA_BUSY_CYCLES"), med.get("GRBM_GUI_ACTIVE")
            cells.append(f"{100.0 * busy / (act / xcc * simds):.1f}" if busy is not None and act else "")
        if "MFMA GFLOP" in derived:
            mops = med.get("SQ_INSTS_VALU_MFMA_MOPS_BF16")
            cells.append(f"{mops * 512 / 1e9:.2f}" if mops is not None else "")
        print("| " + " | ".join(cells) + " |")
    if simds:
        print(f"\nSIMDs: {simds}; XCDs: {xcc} (GRBM_GUI_ACTIVE above is the sum over the XCDs)")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--sets", type=int, default=3,
                    help="rotated copies of weights, batch and KV cache (1: no rotation)")
    ap.add_argument("--no-c64", action="store_true", help="skip the 64-sequence object of the default run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--cpu-single-budget", type=float, default=8.0)
    ap.add_argument("--accept-rounds", type=int, default=2000,
                    help="rounds for the mean accepted length (workloads with a decaying agreement process)")
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
    ap.add_argument("--summarize-trace", nargs="+", metavar="CSV",
                    help="print per-position kernel times of rocprofv3 kernel traces and exit (no GPU)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                    help="print per-kernel medians of rocprofv3 --pmc counter files and exit (no GPU)")
    args = ap.parse_args()
    if args.summarize_trace:
        return _summarize_trace(args.summarize_trace)
    if args.summarize_counters:
        return _summarize_counters(args.summarize_counters)
    if args.gpus != 1:
        print(json.dumps({"error": "the drafter step runs on one GPU (one GPU's share of a sharded deployment); --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        return 2
    if args.calibrate_copy:
        return _calibrate_copy()
    if args.mode == "prep":
        return _bench_prep(args)

    import torch
    import drafting_draft_expand_amd as pe
    import synth
    from synth.device import upload_weights

    wl = synth.WORKLOADS[args.workload]
    spec = wl.model
    dev = "cuda:0"
    t_setup = time.perf_counter()
    w = synth.make_weights(spec, wl.wseed)
    nsets = max(1, args.sets if args.mode != "loop" else 1)
    dw0 = upload_weights(w, dev)
    models = [pe.DraftModel.from_spec(spec, dw0 if s == 0 else _clone(dw0)) for s in range(nsets)]
    torch.cuda.synchronize()
    if args.mode == "loop":
        return _bench_loop(pe, wl, w, models[0], args, dev)
    bench = Bench(pe, wl, w, models, args, dev)
    b = bench.b
    c, K = wl.c, wl.K
    print(f"# setup {time.perf_counter() - t_setup:.1f}s workload={wl.name} N={b.N} T={b.T} sets={nsets}",
          file=sys.stderr, flush=True)

    make = bench.ar_fn if args.mode == "ar" else bench.round_fn
    res = bench.run(make, graph=not args.eager, lm_kernel=args.mode == "peagle")
    head = res["graph" if not args.eager else "eager"]
    warm = res["graph_warm" if not args.eager else "eager_warm"]
    ms = head["median_ms"]
    print(f"# {wl.name}: {'graph' if not args.eager else 'eager'} median {ms * 1e3:.1f} us/step over {nsets} "
          f"rotated sets (mean {head['mean_ms'] * 1e3:.1f}), warm {warm['median_ms'] * 1e3:.1f}; eager "
          f"{res['eager']['median_ms'] * 1e3:.1f}", file=sys.stderr, flush=True)
    out = {
        "metric": METRIC,
        "value": round(c * K / (ms / 1e3), 2),
        "unit": "draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "mean_ms_per_step": round(head["mean_ms"], 5),
        "launch_mode": "eager" if args.eager else "hip_graph",
        "mode": args.mode,
        "layout": args.layout,
        "eager_ms_per_step": round(res["eager"]["median_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if spec.dtype == "bf16" else "f32",
        "data": f"synthetic: seeded N(0,0.02) weights, N(0,1) target hidden states and cached KV, uniform "
                f"accepted counts; {nsets} full copies of weights, batch and KV cache rotated step to step",
        "config": {"workload": wl.name, "num_seqs": c, "draft_depth": K, "draft_rows": b.N, "sampled_rows": c * K,
                   "hidden": spec.hidden, "vocab": spec.vocab, "layers": spec.n_layers,
                   "q_heads": spec.n_q, "kv_heads": spec.n_kv, "head_dim": spec.head_dim,
                   "intermediate": spec.inter, "context": [int(b.context.min()), int(b.context.max())]},
        "warm": {"ms_per_step": round(warm["median_ms"], 5), "value": round(c * K / (warm["median_ms"] / 1e3), 2),
                 "note": "the same round replayed on one set (weights may stay in the memory-side cache)"},
    }
    if "lm_head" in res:
        out["roofline"] = _lm_roofline(spec, c * K, res["lm_head"])
        out["roofline"]["traffic"] = _traffic(wl.name)
    out["step_roofline"] = step_roofline(spec, b, ms, K if args.mode == "ar" else 1)
    if wl.agree_decay != 1.0 and args.mode == "peagle" and args.accept_rounds > 0:
        out["mean_accepted"] = bench.mean_accepted(args.accept_rounds)
    if args.mode == "peagle" and args.workload == DEFAULT_WORKLOAD and not args.no_c64:
        wl64 = synth.WORKLOADS[C64_WORKLOAD]
        assert wl64.wseed == wl.wseed and wl64.model == spec   # the same drafter: its models are reused
        t0 = time.perf_counter()
        b64 = Bench(pe, wl64, w, models, args, dev)
        r64 = b64.run(b64.round_fn, graph=not args.eager)
        h64 = r64["graph" if not args.eager else "eager"]
        ms64 = h64["median_ms"]
        print(f"# {wl64.name}: median {ms64 * 1e3:.1f} us/step (mean {h64['mean_ms'] * 1e3:.1f}), warm "
              f"{r64['graph_warm' if not args.eager else 'eager_warm']['median_ms'] * 1e3:.1f}; setup+run "
              f"{time.perf_counter() - t0:.1f}s", file=sys.stderr, flush=True)
        roof64 = _lm_roofline(spec, wl64.c * wl64.K, r64["lm_head"])
        roof64["traffic"] = _traffic(wl64.name)
        out["c64"] = {"workload": wl64.name, "num_seqs": wl64.c, "draft_depth": wl64.K, "draft_rows": b64.b.N,
                      "sampled_rows": wl64.c * wl64.K, "context": [int(b64.b.context.min()),
                                                                   int(b64.b.context.max())],
                      "value": round(wl64.c * wl64.K / (ms64 / 1e3), 2), "unit": "draft tokens/s",
                      "ms_per_step": round(ms64, 5), "mean_ms_per_step": round(h64["mean_ms"], 5),
                      "warm_ms_per_step": round(r64["graph_warm" if not args.eager else "eager_warm"]["median_ms"],
                                                5),
                      "roofline": roof64, "step_roofline": step_roofline(spec, b64.b, ms64)}
        del b64
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = _cpu_baseline(wl, w, b, args.cpu_budget, args.mode, args.cpu_single_budget)
    for m in models:
        m.close()
    print(json.dumps(out), flush=True)
    return 0


def _bench_loop(pe, wl, w, model, args, dev) -> int:
    """Rounds chained on the device: accept's outputs and the next verified
    batch feed the next prepare; the verifier's tokens and hidden states are
    fixed synthetic buffers (the target model is not part of the path).
    Eager launches, one set (each round reads what the previous one wrote)."""
    import torch
    K = wl.K
    bench = Bench(pe, wl, w, [model], args, dev, extra_positions=(args.steps + args.warmup + 2) * (K + 1))
    st, db = bench.sets[0], bench.sets[0]["db"]
    cur = {k: db[k] for k in ("query_lens", "target_ids", "target_pos", "num_accepted", "bonus_ids")}
    nxt = pe.next_verified_batch(K, st["prep"]["kv_lens"], cur["bonus_ids"], st["tokens"], st["acc"], st["bonus"])
    stream = bench.stream

    def step():
        pe.prepare_draft_batch(model, K, cur["query_lens"], cur["target_ids"], cur["target_pos"],
                               cur["num_accepted"], cur["bonus_ids"], db["target_hidden"], db["block_table"],
                               out=st["prep"], stream=stream, compact=bench.compact)
        pe.draft_forward(model, st["prep"], db["block_table"], db["k_cache"], db["v_cache"], workspace=st["ws"],
                         tokens=st["tokens"], stream=stream)
        pe.accept(st["tokens"], bench.tgt, st["acc"], st["bonus"], stream=stream)
        pe.next_verified_batch(K, st["prep"]["kv_lens"], cur["bonus_ids"], st["tokens"], st["acc"], st["bonus"],
                               out=nxt, stream=stream)
        for k in cur:
            cur[k].copy_(nxt[k])

    for _ in range(args.warmup):
        step()
    t = _timed([step], args.steps, stream)
    ms = t["median_ms"]
    out = {"metric": METRIC, "value": round(wl.c * K / (ms / 1e3), 2), "unit": "draft tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "mean_ms_per_step": round(t["mean_ms"], 5), "launch_mode": "eager", "mode": "loop",
           "layout": args.layout, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if wl.model.dtype == "bf16" else "f32",
           "data": "synthetic: chained rounds, the device-built next verified batch feeding each prepare",
           "config": {"workload": wl.name, "num_seqs": wl.c, "draft_depth": K}}
    model.close()
    torch.cuda.synchronize()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
