"""Benchmark: exact top-k / top-p candidate-set selection on one MI355X.

One step = one qrita_select call over one batch of a named synthetic workload
(both kernels of the path: the streaming truncation pass and the per-row
tail). The headline is the largest workload, 1024 x 201088 float32 logits
(U(-1,1), k = 4096); the other four named workloads are reported in
"per_config" (the single 32000-logit row as a latency, with the oracle's
seconds).

Timing: W warm-up calls, then K calls between two HIP events on the stream the
library launches on. Inputs rotate over enough buffer sets to keep the
footprint above 1 GiB (at most 256 sets), so the 256 MiB Infinity Cache cannot
serve them. A second loop records an event between the two kernels of every
call (qrita_options.mid_event, recorded by the library on its stream) for each
kernel's average duration: the roofline of the dominant kernel uses it. The
outputs of every timed configuration, ablation legs included, are checked
against the CPU oracle, which is then timed on the headline workload as the
CPU baseline.

Ablations (the pages' "Estudios de Ablación", reproduced on these shapes):
truncation off (every row takes the full-row search), binary vs quaternary
pivots on truncation hits and misses, duplicate handling (rows on a 1/16 grid
vs the same distribution in distinct float32 values), and one fixed tier vs
the tier table.

Also timed and parity-checked: the second workload's shapes (top-512 drafter
marginals in float16, top-64 beam pruning, indices in ascending order) and the
fused draw (qrita_sample: tokens and probabilities) on two named workloads.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "rows/sec and effective HBM GB/s (% of peak) for exact top-k/top-p masks"
HEADLINE = 3
KERNEL_SOURCES = {
    "pass1": ("top_selection_sigma_amd/csrc/select_kernel.hpp", "top_selection_sigma_amd/csrc/device_common.hpp",
              "top_selection_sigma_amd/csrc/params.hpp", "top_selection_sigma_amd/csrc/pass1.hip"),
    "tail": ("top_selection_sigma_amd/csrc/tail_kernel.hpp", "top_selection_sigma_amd/csrc/select_kernel.hpp",
             "top_selection_sigma_amd/csrc/device_common.hpp", "top_selection_sigma_amd/csrc/params.hpp",
             "top_selection_sigma_amd/csrc/tail_light.hip", "top_selection_sigma_amd/csrc/tail_heavy.hip"),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
MAX_SETS = 256
CHUNKS = 0  # --chunks


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_digest(kernel):
    """sha256 over a kernel's sources: counter readings taken on other sources
    do not describe this build."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the rocprofv3 FETCH_SIZE/WRITE_SIZE
    readings in profiles/hbm_traffic.json (already scaled by the copy-kernel
    factors), or None when absent or taken on other sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get("kernels", {}).get(kernel, {})
    if ent.get("sha256") != source_digest(kernel):
        return None
    w = ent.get("workloads", {}).get(workload)
    return None if w is None else w.get("hbm_bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def esize(dtype):
    return 4 if dtype == "f32" else 2


def to_device(x, dev):
    import torch

    if x.dtype == "bf16":
        return torch.from_numpy(x.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    if x.dtype == "f16":
        return torch.from_numpy(x.logits.view(np.int16)).to(dev).view(torch.float16)
    return torch.from_numpy(x.logits).to(dev)


class Runner:
    """Device buffers of one workload (rotated copies of the inputs and outputs).

    sample: each step is a qrita_sample call (token and probabilities as well,
    seed fixed, offset = the step); base: options every step carries."""

    SEED = 20260201

    def __init__(self, x, rotate_bytes, want_mask=True, sample=False, base=None):
        import torch

        import top_selection_sigma_amd as q

        self.q = q
        self.x = x
        self.dev = torch.device("cuda", 0)
        self.sample = sample
        self.base = dict(base or {})
        B, V = x.batch, x.vocab
        self.es = esize(x.dtype)
        self.idx_cap = int(max(64, x.k.max()))
        logits0 = to_device(x, self.dev)
        self.k = torch.from_numpy(x.k).to(self.dev)
        self.p = torch.from_numpy(x.p).to(self.dev)
        set_bytes = B * V * (self.es + (1 if want_mask else 0)) + B * self.idx_cap * 4
        self.nsets = max(2, min(MAX_SETS, math.ceil(rotate_bytes / set_bytes)))
        self.sets = []
        for i in range(self.nsets):
            lg = logits0 if i == 0 else logits0.clone()
            m = torch.empty((B, V), dtype=torch.uint8, device=self.dev) if want_mask else None
            tok = torch.empty(B, dtype=torch.int32, device=self.dev) if sample else None
            prob = torch.empty((B, self.idx_cap), dtype=torch.float32, device=self.dev) if sample else None
            self.sets.append((lg, m, torch.empty((B, self.idx_cap), dtype=torch.int32, device=self.dev),
                              torch.empty(B, dtype=torch.int32, device=self.dev), tok, prob))
        self.code = q.dtype_code(logits0)
        self.ws = q.workspace_for(B, V, self.code, self.idx_cap, self.dev)
        self.stream = torch.cuda.current_stream()
        self.last = 0

    def step(self, i, opts=None):
        lg, m, ix, c, tok, prob = self.sets[i % self.nsets]
        if CHUNKS and (opts is None or opts.chunks == 0):
            opts = opts or self.q.Options()
            opts.chunks = CHUNKS
        if self.base:
            opts = opts or self.q.Options()
            for k, v in self.base.items():
                setattr(opts, k, v)
        if self.sample:
            self.q.qrita_sample(lg, self.k, self.p, self.SEED, i, tok, prob, m, ix, c, self.idx_cap, self.ws,
                                self.stream, opts)
        else:
            self.q.qrita_select_ex(lg, self.k, self.p, m, ix, c, self.idx_cap, self.ws, self.stream, opts)
        self.last = i % self.nsets
        self.last_offset = i

    def time(self, steps, warmup, opts=None):
        """Mean ms per call, per-kernel means (ms) and p10/p50/p90 per call."""
        import torch

        q = self.q
        for i in range(warmup):
            self.step(i, q.Options(**opts) if opts else None)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(self.stream)
        for i in range(steps):
            self.step(warmup + i, q.Options(**opts) if opts else None)
        ev1.record(self.stream)
        torch.cuda.synchronize()
        total_ms = ev0.elapsed_time(ev1) / steps
        # per-kernel durations: the library records mid on its stream between
        # the launches; one launch of each kernel over the whole batch (no
        # chunk overlap), so that each duration is one kernel's
        opts = dict(opts or {})
        opts["chunks"] = 1
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        mids = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        for e in mids:
            e.record(self.stream)  # create the underlying hipEvent before handing it over
        torch.cuda.synchronize()
        for i in range(steps):
            starts[i].record(self.stream)
            o = dict(opts or {})
            o["mid_event"] = mids[i]
            self.step(i, q.Options(**o))
            ends[i].record(self.stream)
        torch.cuda.synchronize()
        p1 = float(np.mean([s.elapsed_time(m) for s, m in zip(starts, mids)]))
        tl = float(np.mean([m.elapsed_time(e) for m, e in zip(mids, ends)]))
        per = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
        return dict(ms_per_step=total_ms, pass1_ms=p1, tail_ms=tl,
                    step_ms_p10_p50_p90=[float(np.percentile(per, v)) for v in (10, 50, 90)])

    def outputs(self):
        lg, m, ix, c, tok, prob = self.sets[self.last]
        return None if m is None else m.cpu().numpy(), ix.cpu().numpy(), c.cpu().numpy()

    def draws(self):
        """(tokens, probabilities, offset) of the last step of a sampling runner."""
        lg, m, ix, c, tok, prob = self.sets[self.last]
        return tok.cpu().numpy(), prob.cpu().numpy(), self.last_offset

    def diag(self, opts=None):
        import torch

        q = self.q
        d = torch.zeros(self.x.batch * q.DIAG_FIELDS, dtype=torch.int32, device=self.dev)
        o = dict(opts or {})
        o["diag"] = d
        self.step(0, q.Options(**o))
        torch.cuda.synchronize()
        return d.cpu().numpy().reshape(self.x.batch, q.DIAG_FIELDS)


def parity(x, ref, outs, idx_cap):
    """Rows that differ from the oracle (band rows: a rank prefix of the right length)."""
    import oracle

    mask, idx, count = outs
    band = ref.band_lo != ref.band_hi
    bad = np.zeros(x.batch, bool)
    bad |= ~band & (count != ref.count)
    if mask is not None:
        bad |= ~band & np.any(mask != ref.mask, axis=1)
    for b in range(x.batch):
        n = min(int(count[b]), idx_cap)
        if not band[b] and not np.array_equal(idx[b, :n], ref.idx[b, :n]):
            bad[b] = True
        if band[b] and not (ref.band_lo[b] <= count[b] <= ref.band_hi[b]):
            bad[b] = True
    brows = np.nonzero(band)[0]
    if len(brows):
        sub = x.take_rows(brows)
        full = oracle.select(sub.logits, sub.dtype, sub.k, sub.p, int(max(ref.band_hi[brows].max(), 1)),
                             want_mask=False)
        for j, b in enumerate(brows):
            c = int(count[b])
            m = np.zeros(x.vocab, np.uint8)
            m[full.idx[j, :c]] = 1
            if (mask is not None and not np.array_equal(mask[b], m)) or \
                    not np.array_equal(idx[b, :min(c, idx_cap)], full.idx[j, :min(c, idx_cap)]):
                bad[b] = True
    return dict(mismatch_rows=int(bad.sum()), band_rows=int(band.sum()))


def parity_index_order(x, ref, outs, idx_cap):
    """Rows whose index-ordered output differs from the oracle's kept set
    (indices ascending; band rows: a rank prefix of a length in the band)."""
    import oracle

    _, idx, count = outs
    band = ref.band_lo != ref.band_hi
    bad = 0
    brows = np.nonzero(band)[0]
    full = None
    if len(brows):
        sub = x.take_rows(brows)
        full = oracle.select(sub.logits, sub.dtype, sub.k, sub.p, int(max(ref.band_hi[brows].max(), 1)),
                             want_mask=False)
    j = 0
    for b in range(x.batch):
        c = int(count[b])
        if band[b]:
            ok = ref.band_lo[b] <= c <= ref.band_hi[b]
            kept = np.sort(full.idx[j, :c])
            j += 1
        else:
            ok = c == ref.count[b]
            kept = np.nonzero(ref.mask[b])[0]
        n = min(c, idx_cap)
        if not ok or not np.array_equal(idx[b, :n], kept[:n]):
            bad += 1
    return dict(mismatch_rows=int(bad), band_rows=int(band.sum()))


def parity_draws(x, ref, tokens, probs, idx_cap, offset):
    """Drawn tokens and probabilities against the oracle's draw with NumPy's
    Philox uniforms (band draws: the rank within the oracle's band)."""
    import oracle

    u = oracle.uniforms(Runner.SEED, offset, x.batch)
    s = oracle.sample(x.logits, x.dtype, x.k, x.p, u, idx_cap)
    band = ref.band_lo != ref.band_hi
    exact = ~band & (s.rank_lo == s.rank_hi)
    tok_bad = int(np.sum(exact & (tokens != s.token)))
    prob_bad = 0
    for b in np.nonzero(~band)[0]:
        n = min(int(ref.count[b]), idx_cap)
        want = s.prob[b, :n].astype(np.float64)
        if np.any(np.abs(probs[b, :n].astype(np.float64) - want) > 1e-6 * want + 1e-12):
            prob_bad += 1
    return dict(token_mismatch_rows=tok_bad, prob_mismatch_rows=prob_bad,
                band_draws=int(np.sum(~band & (s.rank_lo != s.rank_hi))), band_rows=int(band.sum()))


def effective_bytes(x, count, idx_cap, mask=True):
    es = esize(x.dtype)
    kept = np.minimum(count, idx_cap).astype(np.int64).sum()
    return int(x.batch * x.vocab * es + (x.batch * x.vocab if mask else 0) + 4 * kept + 4 * x.batch)


def roofline_for(name, x, t, count, idx_cap, bitmap):
    """The dominant kernel's roofline: its algorithmic bytes per launch over its
    average duration. Pass 1 reads every logit once (and writes the mask bytes
    unless the tail writes whole mask rows); the tail writes the indices, the
    counts and, with whole-row masks, the mask."""
    B, V = x.batch, x.vocab
    es = esize(x.dtype)
    kept = int(np.minimum(count, idx_cap).astype(np.int64).sum())
    p1_bytes = B * V * es + (0 if bitmap or bitmap is None else B * V)
    tail_bytes = 4 * kept + 4 * B + (B * V if bitmap else 0)
    dom = "pass1" if t["pass1_ms"] >= t["tail_ms"] else "tail"
    ms = t["pass1_ms"] if dom == "pass1" else t["tail_ms"]
    alg = p1_bytes if dom == "pass1" else tail_bytes
    ach = alg / (ms * 1e-3) / 1e9
    return {"kernel": "pass1_kernel" if dom == "pass1" else "tail_kernel", "bound": "hbm",
            "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(name, dom), "alg_bytes_per_launch": alg,
            "pass1_us": round(t["pass1_ms"] * 1e3, 2), "tail_us": round(t["tail_ms"] * 1e3, 2),
            "pass1_alg_bytes": p1_bytes, "tail_alg_bytes": tail_bytes}


def bench_workload(index, steps, warmup, rotate_bytes, check, ablate):
    import oracle
    import workloads as w

    t0 = time.time()
    x = w.make_config(index)
    log(f"[bench] workload {index} {x.name}: generated in {time.time() - t0:.1f}s")
    r = Runner(x, rotate_bytes)
    t = r.time(steps, warmup)
    outs = r.outputs()
    dg = r.diag()
    res = dict(index=index, name=x.name, batch=x.batch, vocab=x.vocab, dtype=x.dtype,
               rotation_sets=r.nsets, **{k: v for k, v in t.items()})
    count = outs[2]
    eff = effective_bytes(x, count, r.idx_cap)
    sec = t["ms_per_step"] * 1e-3
    res.update(rows_per_s=x.batch / sec, effective_gbps=eff / sec / 1e9,
               pct_peak_hbm=100.0 * eff / sec / 1e9 / PEAK_HBM_GBS, effective_bytes=eff,
               mean_count=float(count.mean()))
    bitmap = x.batch >= 512  # the tier table's whole-row mask rule (the rows here fit every bitmap)
    res["roofline"] = roofline_for(x.name, x, t, count, r.idx_cap, bitmap)
    path = dg[:, 4]
    res["truncation"] = dict(rows=x.batch, single_pass=int(np.sum(path <= 1)), lds_path=int(np.sum(path == 0)),
                             list_path=int(np.sum(path == 1)),
                             miss_predicted=int(np.sum(dg[:, 7] == 1)), recollected=int(np.sum(path == 2)),
                             full_row=int(np.sum(path == 3)), gaussian_t_hit=int(np.sum(dg[:, 5] == 1)),
                             mean_iterations=float(dg[:, 6].mean()))
    es = esize(x.dtype)
    out_bytes = x.batch * x.vocab + x.batch * r.idx_cap * 4 + x.batch * 4
    res["memory"] = dict(workspace_bytes=int(r.q.qrita_workspace_bytes(x.batch, x.vocab, r.code, r.idx_cap)),
                         output_bytes=out_bytes,
                         sort_based_bytes=int(2 * x.batch * x.vocab * (es + 4)) + out_bytes)
    res["memory"]["ratio"] = round((res["memory"]["workspace_bytes"] + out_bytes) / res["memory"]["sort_based_bytes"],
                                   4)
    ref = None
    if check:
        t1 = time.time()
        ref = oracle.select(x.logits, x.dtype, x.k, x.p, r.idx_cap)
        res["oracle_s"] = round(time.time() - t1, 3)
        res["parity"] = parity(x, ref, outs, r.idx_cap)
        log(f"[bench] {x.name}: {t['ms_per_step'] * 1e3:.1f} us/call, parity mismatches "
            f"{res['parity']['mismatch_rows']}, band rows {res['parity']['band_rows']}")
    if ablate:
        res["ablations"] = ablations(index, r, ref, steps, warmup, t)
    return res, x, r


def leg(r, ref, steps, warmup, opts):
    t = r.time(max(5, steps // 2), max(2, warmup // 2), opts)
    out = dict(us_per_call=round(t["ms_per_step"] * 1e3, 2), pass1_us=round(t["pass1_ms"] * 1e3, 2),
               tail_us=round(t["tail_ms"] * 1e3, 2))
    if ref is not None:
        out["parity"] = parity(r.x, ref, r.outputs(), r.idx_cap)["mismatch_rows"]
    return out


def ablations(index, r, ref, steps, warmup, base):
    """The ablation legs on this workload (each parity-checked against the oracle)."""
    a = {"default_us": round(base["ms_per_step"] * 1e3, 2)}
    if index in (0, 1, 2):
        # one launch: each row's tail workgroup streams its row itself,
        # instead of the streaming pass's (row, slice) workgroups
        a["one_launch"] = leg(r, ref, steps, warmup, dict(launches=1))
    if index in (0, 1, 2, 4):
        # truncation off: no survivors in pass 1, every row searches its full row
        a["truncation_off"] = leg(r, ref, steps, warmup, dict(force_miss=True))
    if index in (0, 1, 2, 4):
        # the pivot searches on every row, also where the candidate set is
        # small enough to sort and scan
        a["pivot_search_every_row"] = leg(r, ref, steps, warmup, dict(pivot_search_only=1))
    if index in (1, 2, 3, 4):
        # one pivot per step (binary) instead of three, same duplicate
        # tracking, with the searches on every row
        a["binary_pivots"] = leg(r, ref, steps, warmup, dict(pivot_mode=2, pivot_search_only=1))
        a["quaternary_pivots"] = leg(r, ref, steps, warmup, dict(pivot_search_only=1)) if index == 3 else \
            a.get("pivot_search_every_row")
    if index in (1, 2):
        a["binary_pivots_on_misses"] = leg(r, ref, steps, warmup, dict(pivot_mode=2, force_miss=True))
        a["quaternary_pivots_on_misses"] = a.get("truncation_off")
    if index in (2, 3, 4):
        # four row chunks, each chunk's tail on a second stream beside the
        # next chunk's streaming pass (slower than one chunk on these shapes)
        a["four_chunks_overlapped"] = leg(r, ref, steps, warmup, dict(chunks=4))
    if index in (1, 2, 3, 4):
        a["light_tier_only"] = leg(r, ref, steps, warmup, dict(tier=1))
        a["heavy_tier_only"] = leg(r, ref, steps, warmup, dict(tier=2))
        a["one_slice_per_row"] = leg(r, ref, steps, warmup, dict(slices=1))
    return a


def duplicate_ablation(steps, warmup, rotate_bytes, check):
    """Duplicate handling: the 256 x 151936 shape (k = 50, p = 0.95) in float32,
    rows on the 1/16 grid (heavy ties, including at the k boundary) vs the same
    normal distribution unquantised (distinct values)."""
    import oracle
    import workloads as w

    out = {}
    for kind in ("ties16", "gauss2"):
        x = w.make_rows(256, 151936, "f32", kind, seed=1002, k=50, p=0.95)
        r = Runner(x, rotate_bytes, base=dict(pivot_search_only=1))  # the searches track the duplicates
        t = r.time(steps, warmup)
        ent = dict(us_per_call=round(t["ms_per_step"] * 1e3, 2), pass1_us=round(t["pass1_ms"] * 1e3, 2),
                   tail_us=round(t["tail_ms"] * 1e3, 2))
        if check:
            ref = oracle.select(x.logits, x.dtype, x.k, x.p, r.idx_cap)
            ent["parity"] = parity(x, ref, r.outputs(), r.idx_cap)["mismatch_rows"]
        out["tied_rows" if kind == "ties16" else "distinct_rows"] = ent
    return out


def second_workload(steps, warmup, rotate_bytes, check):
    """The same selection at other systems' shapes: top-512 marginals of a
    block drafter (2048 x 151936 f16) and top-64 pruning of 64 x 64 beam
    proposals (4096 x 4096 f32); indices in ascending order, no mask."""
    import oracle
    import workloads as w

    out = {}
    for i, c in enumerate(w.EXTRA):
        x = w.make_extra(i)
        r = Runner(x, rotate_bytes, want_mask=False, base=dict(idx_order=1))
        t = r.time(steps, warmup)
        outs = r.outputs()
        sec = t["ms_per_step"] * 1e-3
        eff = effective_bytes(x, outs[2], r.idx_cap, mask=False)
        ent = dict(batch=x.batch, vocab=x.vocab, dtype=x.dtype, k=int(x.k[0]), output="indices ascending",
                   us_per_call=round(t["ms_per_step"] * 1e3, 2), pass1_us=round(t["pass1_ms"] * 1e3, 2),
                   tail_us=round(t["tail_ms"] * 1e3, 2), rows_per_s=round(x.batch / sec, 1),
                   effective_gbps=round(eff / sec / 1e9, 1), pct_peak_hbm=round(100 * eff / sec / 1e9 / PEAK_HBM_GBS, 2),
                   roofline=roofline_for(x.name, x, t, outs[2], r.idx_cap, None))
        if check:
            t1 = time.time()
            ref = oracle.select(x.logits, x.dtype, x.k, x.p, r.idx_cap)
            ent["oracle_s"] = round(time.time() - t1, 3)
            ent["parity"] = parity_index_order(x, ref, outs, r.idx_cap)
        log(f"[bench] {x.name}: {ent['us_per_call']} us/call")
        out[x.name] = ent
        del r
    return out


def sampling(index, steps, warmup, rotate_bytes, check, select_us):
    """qrita_sample (selection + one draw per row, probabilities beside the
    indices) on a named workload, against qrita_select on the same outputs."""
    import oracle
    import workloads as w

    x = w.make_config(index)
    r = Runner(x, rotate_bytes, sample=True)
    t = r.time(steps, warmup)
    ent = dict(workload=x.name, us_per_call=round(t["ms_per_step"] * 1e3, 2),
               select_us_per_call=round(select_us, 2), pass1_us=round(t["pass1_ms"] * 1e3, 2),
               tail_us=round(t["tail_ms"] * 1e3, 2))
    if check:
        outs = r.outputs()
        ref = oracle.select(x.logits, x.dtype, x.k, x.p, r.idx_cap)
        ent["parity"] = parity(x, ref, outs, r.idx_cap)
        tok, prob, off = r.draws()
        ent["draw_parity"] = parity_draws(x, ref, tok, prob, r.idx_cap, off)
    log(f"[bench] sampling {x.name}: {ent['us_per_call']} us/call")
    del r
    return ent


def cpu_baseline(x, idx_cap, target_s):
    """The oracle, as it stands, on all host cores over whole batches of the
    headline workload until about target_s seconds of work."""
    import oracle

    threads = oracle.hardware_threads()
    rows = 0
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.select(x.logits, x.dtype, x.k, x.p, idx_cap, nthreads=threads)
        rows += x.batch
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 1000:
            break
    return dict(value=round(rows / el, 2), unit="rows/s", cores=threads, kind="oracle",
                sample=f"{reps} passes over the full {x.batch}-row batch ({el:.1f}s wall)", cpu_model=cpu_model())


def w_name(index):
    import workloads as w

    return w.CONFIGS[index]["name"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=HEADLINE)
    ap.add_argument("--others", default="0,1,2,4", help="extra workloads for per_config ('' = none)")
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--no-ablation", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-second", dest="second", action="store_false", help="skip the second workload")
    ap.add_argument("--no-sampling", dest="sampling", action="store_false", help="skip the sampling legs")
    ap.add_argument("--chunks", type=int, default=0, help="qrita_options.chunks for every call (0 = automatic)")
    args = ap.parse_args()
    global CHUNKS
    CHUNKS = args.chunks
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import top_selection_sigma_amd as q

    q.lib()
    torch.cuda.init()
    rot = int(args.rotate_gib * (1 << 30))
    check = not args.no_check
    ablate = not args.no_ablation
    head, hx, hr = bench_workload(args.config, args.steps, args.warmup, rot, check, ablate)
    del hr
    per = {}
    for s in [t for t in args.others.split(",") if t.strip()]:
        i = int(s)
        if i == args.config:
            continue
        res, x, r = bench_workload(i, args.steps, args.warmup, rot, check, ablate)
        del r
        if i == 0:
            # the single-row case is a latency, reported with the oracle's seconds
            res["latency_us"] = round(res["ms_per_step"] * 1e3, 2)
        per[res["name"]] = res
        torch.cuda.empty_cache()
    dup = duplicate_ablation(max(5, args.steps // 2), max(2, args.warmup // 2), rot, check) if ablate else None
    second = second_workload(args.steps, args.warmup, rot, check) if args.second else None
    samp = None
    if args.sampling:
        samp = {"headline": sampling(args.config, args.steps, args.warmup, rot, check, head["ms_per_step"] * 1e3)}
        sel1 = per.get(w_name(1), {}).get("ms_per_step")
        if sel1 is not None:
            samp["b64_v128256"] = sampling(1, args.steps, args.warmup, rot, check, sel1 * 1e3)
    cpu = cpu_baseline(hx, int(max(64, hx.k.max())), args.cpu_seconds) if args.cpu_seconds > 0 else None
    props = torch.cuda.get_device_properties(0)
    line = {
        "metric": METRIC,
        "value": round(head["rows_per_s"], 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if head["dtype"] == "f32" else head["dtype"],
        "data": "synthetic",
        "config": {"workload": head["name"], "batch": head["batch"], "vocab": head["vocab"],
                   "logits": head["dtype"], "k": 4096, "p": "1.0 (top-p off)",
                   "outputs": "uint8 mask + int32 indices + counts"},
        "effective_gbps": round(head["effective_gbps"], 1),
        "pct_peak_hbm": round(head["pct_peak_hbm"], 2),
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "parity": head.get("parity"),
        "oracle_s": head.get("oracle_s"),
        "step_ms_p10_p50_p90": [round(v, 5) for v in head["step_ms_p10_p50_p90"]],
        "truncation": head["truncation"],
        "memory": head["memory"],
        "ablations": head.get("ablations"),
        "duplicate_handling_ablation": dup,
        "second_workload": second,
        "sampling": samp,
        "per_config": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                       for k, v in per.items()},
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", None),
                   "compute_units": props.multi_processor_count},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
