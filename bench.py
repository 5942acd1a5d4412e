"""Benchmark of the blockwise-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads a,b] [--no-cpu-baseline]

One "step" is one call of the library on one batch of synthetic, device-
resident input.  The headline line is the GQA ring prefill workload (32 query
heads over 8 KV heads, d = 128, 8192 tokens split into 8 ring chunks, bf16,
causal): its value is useful causal TFLOP/s (4 d h_q per admissible
(query, key) pair).  The same run measures, as extra entries, the dense causal
d = 256 workload, the jagged 1152-sequence workload, the split-KV decode
workload (HBM GB/s), the GQA ring shape with a 2048-key causal sliding window
and the 4-chunk fp32 ring latency case.

Per workload:
  1. settle: the step runs back to back for --settle seconds, which brings the
     GPU from idle to its loaded clock before anything is timed.
  2. W untimed warm-up steps, then K steps back to back between one pair of
     HIP events recorded on the stream the library launches on (torch's
     current stream), the timed region bracketed by device synchronisation:
     ms_per_step is that interval over K.  A second pass of K steps, each
     between its own pair of events, gives median_ms (the event records
     between launches add a few microseconds per step, so that pass does not
     set ms_per_step).
`roofline.achieved` is the dominant kernel's algorithmic work per launch over
that mean.  `roofline.traffic` (HBM bytes per launch) and
`roofline.at_measured_clock` (the peak at the clock the counters measured
under this load: CUs x clock x 4096 dense bf16 FLOP/clk/CU) come from the
committed rocprofv3 counter summary when it was taken on the current kernel
sources, else they are null.

CPU leg (skipped with --no-cpu-baseline): the fp64 NumPy oracle, as it stands,
times a bounded sample of every workload on this host's cores -- whole query
heads of the headline (`cpu_baseline`), whole (sequence, head) blocks or rows
of the others -- and the GPU output of the last timed step is compared with it
on that sample (max |err|, max |err| beyond the bf16 output rounding,
Frobenius-relative error).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, nameplate
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
BF16_FLOP_PER_CLK_CU = 4096    # dense bf16 MFMA FLOP per clock per CU
METRIC = "useful causal TFLOP/s (prefill) and HBM GB/s (split-KV decode), % of roofline"


# Sources each measured kernel is built from: the shared headers and the
# launch code, plus its own translation units.  A counter entry stays valid
# while these files are unchanged, whatever else changes in csrc/.
_SHARED_SOURCES = ("fakv_device.h", "fakv_kernels.h", "api.hip")
_FAMILY_SOURCES = {
    "prefill_bf16": ("prefill_bf16_kernel.h", "prefill_bf16.hip", "prefill_bf16_d256.hip", "prefill_bf16_jagged.hip",
                     "worklist.hip"),
    "decode": ("decode.hip", "merge.hip"),
}
_WORKLOAD_FAMILY = {"gqa_ring": "prefill_bf16", "dense_causal": "prefill_bf16", "jagged": "prefill_bf16",
                    "gqa_swa": "prefill_bf16", "jagged_sched": "prefill_bf16", "jagged_worklist": "prefill_bf16",
                    "jagged_plan": "prefill_bf16",
                    "decode": "decode", "decode_merge": "decode"}


def _code_text(path: str) -> bytes:
    """A source file without its comments and with whitespace collapsed: a
    change to comments or layout alone leaves the hash, and so the counter
    figures taken on that code, unchanged.  (String literals of these files
    hold no comment markers.)"""
    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split()).encode()


def csrc_hash(workload: str = None) -> str:
    """Hash of the kernel code: all of csrc/ (workload None), or the files the
    given workload's kernels are built from, comments and layout excluded,
    plus the build flags."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "flash_attention_kv_amd", "csrc")
    if workload is None:
        names = [f for f in sorted(os.listdir(d)) if f.endswith((".hip", ".h", ".inc"))]
    else:
        fam = _WORKLOAD_FAMILY.get(workload)
        if fam is None:
            return ""
        names = sorted(_SHARED_SOURCES + _FAMILY_SOURCES[fam])
    for f in names:
        h.update(f.encode())
        h.update(_code_text(os.path.join(d, f)))
    h.update(_build_flags())
    return h.hexdigest()[:16]


def _build_flags() -> bytes:
    """The compiler flags of the library build (build.py's FLAGS without its
    include paths, and the per-file FILE_FLAGS): they shape the kernel code
    as much as the sources do."""
    text = open(os.path.join(ROOT, "flash_attention_kv_amd", "build.py"), encoding="utf-8").read()
    parts = [m.group(0) for m in re.finditer(r"^(FLAGS|FILE_FLAGS) = [\[{].*?[\]}]$", text, flags=re.S | re.M)]
    body = " ".join(" ".join(p.split()) for p in parts)
    return re.sub(r'"-I", os\.path\.join\([^)]*\)', "", body).encode()


def load_counter(workload: str, key: str):
    """A per-launch figure of the dominant kernel from the committed rocprofv3
    counter summary (profiles/counters.json), if it was measured on the
    current sources of that kernel, else None."""
    p = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(p):
        return None
    try:
        data = json.load(open(p))
    except ValueError:
        return None
    ent = data.get(workload)
    if not ent or ent.get("csrc_hash") != csrc_hash(workload):
        return None
    return ent.get(key)


def load_traffic(workload: str):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel
    calibration)."""
    return load_counter(workload, "bytes_per_launch")


def settle(fn, seconds: float):
    """Runs fn back to back for `seconds`: from idle the GPU takes its first
    ~20 launches of a sub-millisecond kernel to reach its loaded clock (they
    run ~15 % slow), which a short warm-up would otherwise time."""
    import torch
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def time_steps(fn, steps: int, warmup: int, stream):
    """(mean ms per step of K back-to-back steps, median ms of K steps timed
    one by one, wall seconds of the back-to-back region)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean = start.elapsed_time(end) / steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in evs]
    return mean, statistics.median(per), wall


def prefill_pairs(w, offs):
    import numpy as np
    if offs is not None:
        L = np.diff(offs.astype(np.int64))
        return int((L * (L + 1) // 2).sum()) if w.causal else int((L * L).sum())
    if w.window is not None:
        # query i sees min(i + 1, W) keys
        L, W = w.T_q, w.window
        return w.n_seqs * (W * (W + 1) // 2 + max(0, L - W) * W if W < L else L * (L + 1) // 2)
    return w.n_seqs * (w.T_q * (w.T_q + 1) // 2 if w.causal else w.T_q * w.S_kv)


def bench_prefill(name, steps, warmup, settle_s):
    import torch
    import flash_attention_kv_amd as F
    from workloads import WORKLOADS, make_prefill_inputs
    w = WORKLOADS[name]
    q, k, v, offs = make_prefill_inputs(w, device="cuda")
    o = torch.empty_like(q)
    offs_t = torch.from_numpy(offs).to("cuda") if offs is not None else None
    tq, sk = (w.T_q, w.S_kv) if offs is None else (q.shape[0], q.shape[0])
    dt = F.BF16 if w.dtype == "bf16" else F.F32
    need = F.ring_attn_workspace_bytes(tq, sk, w.h_q, w.h_kv, w.d, w.C, w.causal, w.n_seqs,
                                       offs is not None, dt)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        F.ring_attn_fwd(q, k, v, C=w.C, causal=w.causal, seq_offsets=offs_t, n_seqs=w.n_seqs,
                        workspace=ws, out=o, window=w.window)

    settle(step, settle_s)
    ms, med, wall = time_steps(step, steps, warmup, stream)
    flops = 4 * w.d * w.h_q * prefill_pairs(w, offs)
    res = dict(ms=ms, median_ms=med, wall_s=wall, flops=flops, tflops=flops / (ms * 1e-3) / 1e12)
    # host copies for the CPU leg (inputs and the last step's output)
    res["host"] = (q.cpu(), k.cpu(), v.cpu(), o.cpu(), offs)
    del q, k, v, o, ws
    torch.cuda.empty_cache()
    return res


def bench_decode(steps, warmup, settle_s):
    import torch
    import flash_attention_kv_amd as F
    from workloads import WORKLOADS, make_decode_inputs
    w = WORKLOADS["decode"]
    q, k, v = make_decode_inputs(w, device="cuda")
    o = torch.empty_like(q)
    ws = torch.empty(F.splitkv_decode_workspace_bytes(w.B, w.h_q, w.d, w.n_chunks), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        F.splitkv_decode(q, k, v, n_chunks=w.n_chunks, workspace=ws, out=o)

    settle(step, settle_s)
    ms, med, wall = time_steps(step, steps, warmup, stream)
    kv_bytes = 2 * w.B * w.S_cache * w.h_kv * w.d * 2
    alg = kv_bytes + 2 * w.B * w.h_q * w.d * 2
    parts = 2 * w.n_chunks * w.B * w.h_q * (w.d + 2) * 4      # triplets written, then read
    # host copies for the CPU leg: the rows of the first 2 sequences only
    host = (q[:2].cpu(), k[:2].cpu(), v[:2].cpu(), o[:2].cpu())
    del q, k, v, o, ws
    torch.cuda.empty_cache()
    return dict(ms=ms, median_ms=med, wall_s=wall, bytes=alg, partial_bytes=parts,
                gbs=alg / (ms * 1e-3) / 1e9, host=host)


# ---------------------------------------------------------------------------
# CPU leg: the oracle on a bounded sample, timed, and the GPU output checked on it


def _blas():
    try:
        from threadpoolctl import threadpool_info
        return [(i.get("internal_api"), i.get("num_threads")) for i in threadpool_info()]
    except Exception:   # pragma: no cover
        return []


class ErrAcc:
    """Running parity statistics of GPU output blocks against the oracle."""

    def __init__(self, out_bf16: bool):
        self.out_bf16, self.mx, self.excess, self.se, self.sr = out_bf16, 0.0, 0.0, 0.0, 0.0

    def add(self, got, ref):
        import numpy as np
        got = np.asarray(got, dtype=np.float64)
        err = np.abs(got - ref)
        if self.out_bf16:
            # distance from ref to the set of values that round to the bf16 output
            _, ex = np.frexp(got)
            half_ulp = np.where(got == 0.0, 0.0, np.ldexp(1.0, ex - 9))
            self.excess = max(self.excess, float((err - half_ulp).max()))
        else:
            self.excess = max(self.excess, float(err.max()))
        self.mx = max(self.mx, float(err.max()))
        self.se += float(np.square(got - ref).sum())
        self.sr += float(np.square(ref).sum())

    def report(self):
        return {"max_abs": float(f"{self.mx:.4e}"), "max_abs_beyond_output_rounding": float(f"{self.excess:.4e}"),
                "frob_rel": float(f"{(self.se / max(self.sr, 1e-300)) ** 0.5:.4e}")}


def oracle_prefill_sample(name, host, budget_s: float):
    """Whole (sequence, query head) blocks of a prefill workload, in a fixed
    order, until `budget_s` of oracle time is used.  Returns the CPU rate and
    the parity of the GPU output on those blocks."""
    import numpy as np
    import oracle
    from workloads import WORKLOADS
    w = WORKLOADS[name]
    q, k, v, o, offs = host
    if offs is not None:
        segs = [(int(offs[b]), int(offs[b + 1])) for b in range(len(offs) - 1)]
        order = [(b, h) for b in range(len(segs)) for h in range(w.h_q)]
        keys = lambda b: segs[b]
    else:
        segs = [(b * w.T_q, (b + 1) * w.T_q) for b in range(w.n_seqs)]
        # spread over sequences and heads: head h of sequence h mod n first
        order = [((h + j) % w.n_seqs, h) for j in range(w.n_seqs) for h in range(w.h_q)]
        keys = lambda b: (b * w.S_kv, (b + 1) * w.S_kv)
    acc = ErrAcc(w.dtype == "bf16")
    t_used, flops, blocks, rows = 0.0, 0, 0, 0
    for (b, h) in order:
        q0, q1 = segs[b]
        k0, k1 = keys(b)
        if q1 == q0:
            continue
        kvh = oracle.kv_head_of(h, w.h_q, w.h_kv)
        qb, kb, vb = q[q0:q1, h:h + 1], k[k0:k1, kvh:kvh + 1], v[k0:k1, kvh:kvh + 1]
        t0 = time.perf_counter()
        ref = oracle.attention_ref(qb, kb, vb, causal=w.causal, window=w.window)
        t_used += time.perf_counter() - t0
        acc.add(o[q0:q1, h].double().numpy(), ref[:, 0])
        L, S = q1 - q0, k1 - k0
        if w.window is not None:
            pairs = oracle.windowed_pairs(L, w.window)
        else:
            pairs = oracle.causal_pairs(L) if w.causal else L * S
        flops += oracle.useful_flops_prefill(1, w.d, pairs)
        blocks += 1
        rows += L
        if t_used >= budget_s:
            break
    return {"tflops": flops / t_used / 1e12, "seconds": round(t_used, 2), "blocks": blocks, "rows": rows,
            "of_blocks": sum(1 for (b, h) in order if segs[b][1] > segs[b][0]), "parity": acc.report()}


def oracle_decode_sample(host, budget_s: float):
    import oracle
    from workloads import WORKLOADS
    w = WORKLOADS["decode"]
    q, k, v, o = host
    acc = ErrAcc(True)
    t_used, n, B = 0.0, 0, q.shape[0]
    for b in range(B):
        for h in range(w.h_q):
            kvh = oracle.kv_head_of(h, w.h_q, w.h_kv)
            t0 = time.perf_counter()
            ref = oracle.attention_ref(q[b:b + 1, h:h + 1], k[b, :, kvh:kvh + 1], v[b, :, kvh:kvh + 1])
            t_used += time.perf_counter() - t0
            acc.add(o[b, h].double().numpy(), ref[0, 0])
            n += 1
            if t_used >= budget_s:
                break
        if t_used >= budget_s:
            break
    kv_bytes = 2 * w.S_cache * w.d * 2 * n / (w.h_q // w.h_kv)    # each KV head's cache serves g rows
    return {"gbs": kv_bytes / t_used / 1e9, "seconds": round(t_used, 2), "rows": n,
            "of_rows": w.B * w.h_q, "parity": acc.report()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of back-to-back steps per workload before warm-up and timing")
    ap.add_argument("--workloads", default="gqa_ring,dense_causal,jagged,gqa_swa,decode,ring_tiny")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run one device-to-device copy of BYTES (the reference kernel for "
                         "scaling HBM counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; multi-GPU sharding of the "
                          "ring and decode paths is not built (see the design notes)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if not os.path.exists(os.path.join(ROOT, "flash_attention_kv_amd", "libfakv.so")):
        import __graft_entry__
        __graft_entry__.build()
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        x = torch.ones(args.calibrate_copy // 4, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copied_bytes": args.calibrate_copy}))
        return
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    sel = [s for s in args.workloads.split(",") if s]
    res = {}
    for name in ("gqa_ring", "dense_causal", "jagged", "gqa_swa", "ring_tiny"):
        if name in sel:
            r = bench_prefill(name, args.steps, args.warmup, args.settle)
            res[name] = r
            print(f"# {name}: {r['ms']:.4f} ms/step (median {r['median_ms']:.4f}), {r['tflops']:.1f} TFLOP/s",
                  file=sys.stderr, flush=True)
    if "decode" in sel:
        r = bench_decode(args.steps, args.warmup, args.settle)
        res["decode"] = r
        print(f"# decode: {r['ms']:.4f} ms/step (median {r['median_ms']:.4f}), {r['gbs']:.0f} GB/s",
              file=sys.stderr, flush=True)

    def mfma_roofline(r, name):
        out = {"bound": "mfma", "achieved": round(r["tflops"], 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
               "frac": round(r["tflops"] / PEAK_BF16_TFLOPS, 4), "traffic": load_traffic(name)}
        ghz = load_counter(name, "clock_ghz")
        out["at_measured_clock"] = None
        if ghz:
            pk = n_cu * ghz * 1e9 * BF16_FLOP_PER_CLK_CU / 1e12
            out["at_measured_clock"] = {"clock_ghz": ghz, "cus": n_cu, "peak": round(pk, 1),
                                        "frac": round(r["tflops"] / pk, 4)}
        return out

    extra = {}
    for name in ("dense_causal", "jagged", "gqa_swa"):
        if name in res:
            r = res[name]
            extra[name] = {"value": round(r["tflops"], 2), "unit": "TFLOP/s", "ms_per_step": round(r["ms"], 4),
                           "median_ms": round(r["median_ms"], 4), "useful_flops": r["flops"],
                           "roofline": mfma_roofline(r, name)}
    if "dense_causal" in extra:
        extra["dense_causal"]["page_context"] = "Pallas dense causal flash on the Helion page, same shape, unnamed chip: 225.8 TF/s"
    if "gqa_swa" in extra:
        extra["gqa_swa"]["window"] = 2048
    if "jagged" in extra:
        extra["jagged"]["page_context"] = "Helion page jagged table (softmax 'flash' row, unnamed chip, unknown lengths): 97.7 TF/s"
    if "decode" in res:
        r = res["decode"]
        extra["decode"] = {"value": round(r["gbs"], 1), "unit": "GB/s", "ms_per_step": round(r["ms"], 4),
                           "median_ms": round(r["median_ms"], 4),
                           "algorithmic_bytes": r["bytes"], "partial_triplet_bytes": r["partial_bytes"],
                           "roofline": {"bound": "hbm", "achieved": round(r["gbs"], 1), "peak": PEAK_HBM_GBS,
                                        "unit": "GB/s", "frac": round(r["gbs"] / PEAK_HBM_GBS, 4),
                                        "traffic": load_traffic("decode")}}
    if "ring_tiny" in res:
        r = res["ring_tiny"]
        extra["ring_tiny"] = {"value": round(r["ms"] * 1e3, 2), "unit": "us per call", "dtype": "f32",
                              "median_us": round(r["median_ms"] * 1e3, 2), "useful_flops": r["flops"],
                              "tflops": round(r["tflops"], 3)}

    # CPU leg: the oracle on a bounded sample of every workload
    cpu = None
    if not args.no_cpu_baseline:
        blas = _blas()
        threads = max([n for _, n in blas if n] or [1])
        budgets = {"gqa_ring": 12.0, "dense_causal": 3.0, "jagged": 3.0, "gqa_swa": 3.0, "ring_tiny": 0.5}
        for name, budget in budgets.items():
            if name not in res:
                continue
            s = oracle_prefill_sample(name, res[name]["host"], budget)
            print(f"# oracle {name}: {s['blocks']} blocks in {s['seconds']} s, parity {s['parity']}",
                  file=sys.stderr, flush=True)
            ent = {"seconds": s["seconds"], "value": round(s["tflops"], 4), "unit": "TFLOP/s", "cores": threads,
                   "sample": f"{s['blocks']} of {s['of_blocks']} (sequence, query head) blocks, all rows "
                             f"({s['rows']} rows), fp64 NumPy oracle"}
            if name == "gqa_ring":
                cpu = {"value": s["tflops"], "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                       "sample": f"{s['blocks']} of {w_heads(name)} query heads of the GQA ring prefill workload "
                                 f"(all 8192 causal query rows each), fp64 NumPy oracle, {s['seconds']} s; "
                                 f"BLAS {blas}; host cpus {len(os.sched_getaffinity(0))}",
                       "seconds": s["seconds"], "parity": s["parity"]}
            else:
                extra[name]["oracle_cpu"] = ent
                extra[name]["parity"] = s["parity"]
        if "decode" in res:
            s = oracle_decode_sample(res["decode"]["host"], 3.0)
            print(f"# oracle decode: {s['rows']} rows in {s['seconds']} s, parity {s['parity']}",
                  file=sys.stderr, flush=True)
            extra["decode"]["oracle_cpu"] = {"seconds": s["seconds"], "value": round(s["gbs"], 3), "unit": "GB/s",
                                             "cores": threads,
                                             "sample": f"{s['rows']} of {s['of_rows']} (sequence, query head) "
                                                       f"rows, fp64 NumPy oracle"}
            extra["decode"]["parity"] = s["parity"]

    if "gqa_ring" not in res:
        print(json.dumps({"metric": METRIC, "extra": extra}))
        return
    head = res["gqa_ring"]
    roof = mfma_roofline(head, "gqa_ring")
    roof["kernel"] = "prefill_bf16_kernel<128, 4, 8, false> (d=128, 4 query heads per 8-wave workgroup, 128-key tiles)"
    roof["useful_flops_per_launch"] = head["flops"]
    line = {
        "metric": METRIC, "value": round(head["tflops"], 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(head["ms"], 4),
        "median_ms": round(head["median_ms"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic N(0,1), seeded, generated on the device",
        "config": {"workload": "gqa_ring_prefill", "h_q": 32, "h_kv": 8, "d_head": 128, "T_q": 8192,
                   "S_kv": 8192, "ring_chunks": 8, "causal": True, "global_batch": 1, "seq_len": 8192,
                   "parallelism": "1 GPU (ring ranks laid out on one device)"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "extra": extra,
        "kernel_sources": csrc_hash(),
    }
    print(json.dumps(line), flush=True)


def w_heads(name):
    from workloads import WORKLOADS
    return WORKLOADS[name].h_q


if __name__ == "__main__":
    main()
