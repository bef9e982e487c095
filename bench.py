#!/usr/bin/env python3
"""Benchmark of the block-sparse attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_gqa]

One step is one complete ``msa_kvouter_attention`` call (index build, work
split, attention, combine) over one synthetic batch already resident in HBM.
Two independently drawn batches alternate between steps so that the 256 MB
last-level cache cannot serve a step from the previous one.

Prints ONE JSON line on stdout:
  value      unique-KV bytes per step / seconds per step, in GB/s (the pass's
             headline figure for decode); effective TFLOP/s and the step time
             in microseconds are reported beside it
  roofline   dominant kernel: algorithmic bytes (or flops) per launch divided
             by its average launch time, measured with HIP events recorded on
             the call's stream around that kernel during the timed steps
  cpu_baseline  the fp64 oracle (test infrastructure) timed on this host's
             cores over a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA, published
METRIC = "unique-KV HBM GB/s + effective TFLOP/s, sparse attn fwd; decode step µs"

DESCRIPTIONS = {
    "tiny": "1 seq x 4 queries, Hq=16, Hkv=1, d=128, L=512, page 64, top-2 of 4 blocks, non-causal, bf16",
    "decode_gqa": "64 seqs x 1 query, Hq=64, Hkv=8, d=128, L~U[8192,32768], page 64 shuffled, "
                  "top-16 blocks of 128 (last block forced), causal, bf16",
    "prefill_shared": "1 seq, Tq=L=16384, Hq=64, Hkv=8, d=128, page 128, top-16; chunks of 64 queries "
                      "share 12 picks, diagonal forced, causal, bf16",
    "varlen_mqa": "16 seqs, Tq lognormal(median 256, sigma 1) in [1,2048], L=U[4096,131072]+Tq, "
                  "Hq=32, Hkv=1, d=128, page 128, top-32, causal, fp16",
    "decode_fp8": "256 seqs x 1 query, L=65536, Hq=64, Hkv=8, d=128, page 64, top-16 uniform, "
                  "K/V fp8 e4m3fn, q bf16, causal",
    "decode_mqa": "256 seqs x 1 query, Hq=32, Hkv=1 (MQA), d=128, L~U[8192,32768], page 64 shuffled, "
                  "top-16 blocks of 128 (last block forced), causal, bf16",
    "decode_fp4": "256 seqs x 1 query, L=65536, Hq=64, Hkv=8, d=128, page 64, top-16 uniform, "
                  "K/V MXFP4 (e2m1 codes, e8m0 scale per 32 values), q bf16, causal",
    "prefill_fp4": "1 seq, Tq=L=16384, Hq=64, Hkv=8, d=128, page 128, top-16; chunks of 64 queries "
                   "share 12 picks, diagonal forced, causal, q bf16, K/V MXFP4",
    "dense_causal": "1 seq, Tq=L=8192, Hq=64, Hkv=8, d=128, page 128, every visible block selected "
                    "(top-64), causal, bf16: dense causal attention through the sparse path",
    "kv_store_fp8": "paged K/V store (the step before the pass): 32768 new tokens x Hkv=8 x d=128, "
                    "bf16 -> fp8 e4m3fn cache, page 64, slots shuffled over the cache",
}
STORE_METRIC = "paged K/V store GB/s (bytes read + written), bf16 -> fp8 e4m3fn"
DESCRIPTIONS.update({
    "select_decode": "block selection for 64 decode tokens (one per sequence), L~U[8192,32768], Hkv=8, d=128, "
                     "page 64, fp8 e4m3fn index keys, bf16 index queries, top-16, causal, own block forced",
    "select_prefill": "block selection for 1 seq, Tq=L=8192, Hkv=8, d=128, page 128, bf16 index keys and "
                      "queries, top-16, causal, own block forced",
})
SELECT_METRIC = {"select_decode": ("index-key HBM GB/s, block selection (scores + top-k)", "GB/s"),
                 "select_prefill": ("effective TFLOP/s, block selection (scores + top-k)", "TFLOP/s")}
# Kernels whose summed average launch time the roofline is taken over. In
# the prefill-shaped workloads the attention's MFMA work is split between
# the KV-outer unit kernel and the tile kernel (chains plus the LSE merge),
# so the two are timed together.
DOMINANT = {"tiny": ["front"], "decode_gqa": ["front"], "decode_fp8": ["front"], "decode_mqa": ["front"],
            "decode_fp4": ["front"], "prefill_fp4": ["units", "tiles"],
            "prefill_shared": ["units", "tiles"], "varlen_mqa": ["units", "tiles"],
            "dense_causal": ["tiles"], "kv_store_fp8": ["store"], "select_decode": ["select"],
            "select_prefill": ["select"]}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def accounting(wl):
    """Algorithmic work of one batch: unique KV bytes, effective flops, Q/O bytes."""
    sel = wl.selected.astype(np.int64)
    Tq, Hkv, K = sel.shape
    cu = wl.cu_seqlens_q.astype(np.int64)
    used = wl.used_kv_lens.astype(np.int64)
    seq = np.full(Tq, -1, dtype=np.int64)
    for s in range(wl.B):
        seq[cu[s]:cu[s + 1]] = s
    has = seq >= 0
    s_ = np.where(has, seq, 0)
    L = np.where(has, used[s_], 0)
    pos = L - (cu[s_ + 1] - cu[s_]) + (np.arange(Tq) - cu[s_])
    nblk = (L + 127) // 128
    valid = has[:, None, None] & (sel >= 0) & (sel < nblk[:, None, None])
    hi = np.minimum(128 * sel + 128, L[:, None, None])
    if wl.causal:
        valid &= 128 * sel <= pos[:, None, None]
        hi = np.minimum(hi, pos[:, None, None] + 1)
    nkeys = np.where(valid, hi - 128 * sel, 0)
    flops = 4.0 * 128 * wl.G * float(nkeys.sum())
    nbmax = int(nblk.max()) + 1 if Tq else 1
    g = np.broadcast_to(np.arange(Hkv)[None, :, None], sel.shape)
    key = (np.broadcast_to(s_[:, None, None], sel.shape) * Hkv + g) * nbmax + sel
    uk = np.unique(key[valid])
    ub = uk % nbmax
    us = uk // nbmax // Hkv
    # bytes of one K (or V) row: 128 values, or MXFP4's 64 code and 4 scale bytes
    row_bytes = 64 + 4 if wl.mxfp4 else 128 * wl.k_vals.element_size()
    block_tokens = np.minimum(128 * ub + 128, used[us]) - 128 * ub
    unique_kv = float(block_tokens.sum()) * 2 * row_bytes
    q_elem = wl.q.element_size()
    qo = float(Tq * wl.Hq) * (128 * q_elem * 2 + 4)
    return dict(unique_kv_bytes=unique_kv, effective_flops=flops, qo_bytes=qo)


# the source file each kernel family is compiled from
KERNEL_SOURCES = {"front": "msa_forward.hip", "classify": "msa_forward.hip", "units": "msa_tiles.hip",
                  "tiles": "msa_tiles.hip", "index": "msa_index.hip", "emit": "msa_index.hip",
                  "store": "msa_store.hip", "select": "msa_select.hip"}


def kernel_sources_sha256(workload):
    """Digest of the sources behind a workload's dominant kernels: their own
    .hip files, every shared header and the host file that sizes and launches
    them. A change to any of these voids the workload's recorded counters."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_sparse_attention_selection_amd", "csrc")
    own = {KERNEL_SOURCES[k] for k in DOMINANT[workload]} | {"msa_api.hip"}
    for name in sorted(os.listdir(csrc)):
        if name.endswith(".hpp") or name in own:
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload, kernels):
    """HBM bytes per launch of `kernels` from the recorded counter runs, or None.

    profiles/traffic_<workload>.txt holds a JSON object written from two
    rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch, per
    kernel) and the same counters for a plain 1 GiB copy (bench.py
    --calibrate-copy), which give the KiB-to-bytes factors. The figure is
    reported only while the kernel sources are the ones it was taken on.
    """
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != kernel_sources_sha256(workload):
        return None
    try:
        ff, fw = rec["fetch_factor"], rec["write_factor"]
        return int(sum(rec["kernels"][k]["fetch_kib"] * ff + rec["kernels"][k]["write_kib"] * fw
                       for k in kernels))
    except (KeyError, TypeError):
        return None


# rocprofv3 runs whose outputs write_profile_summaries() turns into the
# text summaries under profiles/ ($ROOT: the repository root on the GPU machine)
PROF_TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d $ROOT/gpurun_out/prof/{w} -o run "
                  "-- python3 $ROOT/bench.py --workload {w} --steps 20 --warmup 5 --no-cpu-baseline")
PROF_PMC_CMD = ("rocprofv3 --pmc {c} --output-format csv -d $ROOT/gpurun_out/traffic/{w}_{c} -o run "
                "-- python3 $ROOT/bench.py --workload {w} --steps 3 --warmup 1 --no-cpu-baseline")
PROF_COPY_CMD = ("rocprofv3 --pmc {c} --output-format csv -d $ROOT/gpurun_out/traffic/copy_{c} -o run "
                 "-- python3 $ROOT/bench.py --calibrate-copy")
KERNEL_KEYS = {"front": "k_front", "units": "k_units", "tiles": "k_tiles", "classify": "k_classify_waves",
               "index": "k_index", "emit": "k_emit", "store": "k_store_kv", "select": "k_select"}
# SQ counter passes (each within one pass's hardware limits: at most 8 SQ
# and 2 GRBM counters), one rocprofv3 run each
COUNTER_SETS = {
    "issue": ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU",
              "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR"],
    "busy": ["GRBM_GUI_ACTIVE", "SQ_BUSY_CU_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU",
             "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "SQ_LDS_BANK_CONFLICT"],
}
PROF_SET_CMD = ("rocprofv3 --pmc {counters} --output-format csv -d $ROOT/gpurun_out/counters/{w}_{s} -o run "
                "-- python3 $ROOT/bench.py --workload {w} --steps 3 --warmup 1 --no-cpu-baseline")


def write_profile_summaries(src):
    """profiles/kernels_<w>.md and profiles/traffic_<w>.txt from rocprofv3 outputs under src.

    src/prof/<w>/**/run_kernel_stats.csv: the kernel-trace statistics of
    PROF_TRACE_CMD; src/traffic/{copy,<w>}_{FETCH_SIZE,WRITE_SIZE}/**/
    run_counter_collection.csv: the counter runs of PROF_PMC_CMD and
    PROF_COPY_CMD. FETCH_SIZE and WRITE_SIZE are KiB-like units per dispatch;
    the plain 1 GiB copy gives the factors to bytes.
    """
    import csv
    import glob
    from collections import defaultdict

    def one(pattern):
        f = sorted(glob.glob(os.path.join(src, pattern), recursive=True))
        return f[0] if f else None

    def counters(d):
        f = one(os.path.join("traffic", d, "**", "*counter_collection.csv"))
        acc = defaultdict(list)
        if f:
            for r in csv.DictReader(open(f)):
                acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}

    factors = None
    cf, cw = counters("copy_FETCH_SIZE"), counters("copy_WRITE_SIZE")
    if cf and cw:
        (f_kib, _), f_name = max((v, k) for k, v in cf.items() if "copy" in k.lower())
        (w_kib, _), _ = max((v, k) for k, v in cw.items() if "copy" in k.lower())
        factors = ((1 << 30) / f_kib, (1 << 30) / w_kib, f_kib, w_kib, f_name)
    def counter_sets(w):
        """{kernel short name: {counter: average per dispatch}} over the counter passes of w"""
        acc = defaultdict(lambda: defaultdict(list))
        for sname in COUNTER_SETS:
            f = one(os.path.join("counters", f"{w}_{sname}", "**", "*counter_collection.csv"))
            if not f:
                continue
            for r in csv.DictReader(open(f)):
                for short, pat in KERNEL_KEYS.items():
                    if pat in r["Kernel_Name"]:
                        acc[short][r["Counter_Name"]].append(float(r["Counter_Value"]))
        return {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in acc.items()}

    for w in DESCRIPTIONS:
        cs = counter_sets(w)
        if cs:
            sha = kernel_sources_sha256(w)
            lines = [f"# {w}: SQ counters per dispatch", "", f"Workload: {DESCRIPTIONS[w]}.", "",
                     "Commands (from the repository root on an MI355X; `$ROOT` is that root), one per pass:", "",
                     "```"]
            lines += [PROF_SET_CMD.format(counters=" ".join(c), w=w, s=n) for n, c in COUNTER_SETS.items()]
            lines += ["```", "", f"Kernel sources: sha256 {sha}.", "",
                      "Averages per dispatch, summed over the chip. Derived: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES "
                      "/ (GRBM_GUI_ACTIVE / 8 XCDs x 256 CUs x 4 SIMDs); per-MFMA ratios divide instruction "
                      "counts by SQ_INSTS_MFMA (wave-level instructions).", ""]
            names = sorted({c for d in cs.values() for c in d})
            kern = [k for k in ("tiles", "units", "front", "classify", "index", "emit", "select", "store") if k in cs]
            lines += ["| Counter | " + " | ".join(f"`{KERNEL_KEYS[k]}`" for k in kern) + " |",
                      "|---|" + "---|" * len(kern)]
            for c in names:
                lines.append(f"| {c} | " + " | ".join(f"{cs[k].get(c, float('nan')):.4g}" for k in kern) + " |")

            def ratio(k, a, b):
                x, y = cs[k].get(a), cs[k].get(b)
                return f"{x / y:.3g}" if x is not None and y else "-"
            lines += ["", "| Derived | " + " | ".join(f"`{KERNEL_KEYS[k]}`" for k in kern) + " |",
                      "|---|" + "---|" * len(kern)]
            for label, a, b in [("VALU instructions per MFMA", "SQ_INSTS_VALU", "SQ_INSTS_MFMA"),
                                ("fp32 transcendentals per MFMA", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_MFMA"),
                                ("LDS instructions per MFMA", "SQ_INSTS_LDS", "SQ_INSTS_MFMA"),
                                ("SALU instructions per MFMA", "SQ_INSTS_SALU", "SQ_INSTS_MFMA"),
                                ("waiting share of wave time", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES")]:
                lines.append(f"| {label} | " + " | ".join(ratio(k, a, b) for k in kern) + " |")
            util = []
            for k in kern:
                g, m = cs[k].get("GRBM_GUI_ACTIVE"), cs[k].get("SQ_VALU_MFMA_BUSY_CYCLES")
                util.append(f"{m / (g / 8 * 256 * 4):.3f}" if g and m is not None else "-")
            lines.append("| MFMA busy (fraction of SIMD cycles) | " + " | ".join(util) + " |")
            with open(os.path.join(ROOT, "profiles", f"counters_{w}.md"), "w") as f:
                f.write("\n".join(lines) + "\n")
            print("wrote", f"profiles/counters_{w}.md")

    for w in DESCRIPTIONS:
        sha = kernel_sources_sha256(w)
        stats = one(os.path.join("prof", w, "**", "*kernel_stats.csv"))
        if stats:
            rows = [r for r in csv.DictReader(open(stats)) if "msa" in r["Name"]]
            lines = [f"# {w}: rocprofv3 kernel statistics", "",
                     f"Workload: {DESCRIPTIONS[w]}.", "",
                     "Command (from the repository root on an MI355X; `$ROOT` is that root):", "",
                     "```", PROF_TRACE_CMD.format(w=w), "```", "",
                     f"Kernel sources: sha256 {sha}.", "",
                     "| Kernel | Calls | Average (us) | Min (us) | Max (us) | Share of GPU time |",
                     "|---|---|---|---|---|---|"]
            for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
                lines.append(f"| `{r['Name'][:70]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                             f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                             f"{float(r['Percentage']):.1f}% |")
            lines += ["", "The benchmark's own input generation kernels (torch fills, copies) are omitted; "
                      "their share is part of the last column's remainder."]
            with open(os.path.join(ROOT, "profiles", f"kernels_{w}.md"), "w") as f:
                f.write("\n".join(lines) + "\n")
            print("wrote", f"profiles/kernels_{w}.md")
        fk, wk = counters(f"{w}_FETCH_SIZE"), counters(f"{w}_WRITE_SIZE")
        if factors and fk and wk:
            ff, fw, f_kib, w_kib, f_name = factors
            rec = {"workload": w, "sources_sha256": sha, "fetch_factor": ff, "write_factor": fw,
                   "copy_reference": {"bytes": 1 << 30, "fetch_size": f_kib, "write_size": w_kib,
                                      "kernel": f_name[:120]},
                   "commands": [PROF_COPY_CMD.format(c="FETCH_SIZE"), PROF_COPY_CMD.format(c="WRITE_SIZE"),
                                PROF_PMC_CMD.format(w=w, c="FETCH_SIZE"), PROF_PMC_CMD.format(w=w, c="WRITE_SIZE")],
                   "kernels": {}}
            for short, pat in KERNEL_KEYS.items():
                # every kernel of the family (e.g. the selection's score and list
                # launches), each launched once per call: their per-dispatch
                # averages add up to one call's traffic
                a = [v for k, v in fk.items() if pat in k]
                b = [v for k, v in wk.items() if pat in k]
                if a and b:
                    f_sum, w_sum = sum(x[0] for x in a), sum(x[0] for x in b)
                    rec["kernels"][short] = {"fetch_kib": f_sum, "write_kib": w_sum, "dispatches": a[0][1],
                                             "kernels_in_family": len(a), "hbm_bytes": f_sum * ff + w_sum * fw}
            with open(os.path.join(ROOT, "profiles", f"traffic_{w}.txt"), "w") as f:
                json.dump(rec, f, indent=1)
            print("wrote", f"profiles/traffic_{w}.txt",
                  {k: round(v["hbm_bytes"] / 1e6, 1) for k, v in rec["kernels"].items()}, "MB per launch")


def bench_store(args, torch, msa):
    """The paged K/V store benchmark: one step is one msa_store_kv call."""
    from oracle import store_ref  # the CPU baseline leg only

    dev = torch.device("cuda:0")
    N, Hkv, P = 32768, 8, 64
    NP = N // P + 64
    sets = []
    for i in range(2):
        g = torch.Generator().manual_seed(4242 + i)
        k = torch.randn((N, Hkv, 128), generator=g).to(torch.bfloat16)
        v = torch.randn((N, Hkv, 128), generator=g).to(torch.bfloat16)
        loc = torch.randperm(NP * P, generator=g)[:N].to(torch.int64)
        sets.append(dict(k=k.to(dev), v=v.to(dev), loc=loc.to(dev), k_cpu=k, v_cpu=v, loc_cpu=loc))
    kc = torch.zeros((NP, Hkv, P, 128), dtype=torch.uint8, device=dev).view(torch.float8_e4m3fn)
    vc = torch.zeros_like(kc)
    moved = N * Hkv * 128 * 2 * (2 + 1) + N * 8  # read K and V (16-bit) and the slots, write K and V (fp8)

    def step(i):
        d = sets[i % 2]
        msa.store_kv(d["k"], d["v"], d["loc"], kc, vc, page_size=P)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        step(i)
    stop.record(stream)
    stop.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    msa.profile_enable(["store"])
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    k_ms, k_n = msa.profile_collect("store")
    msa.profile_enable([])
    k_avg = k_ms / max(k_n, 1)
    achieved = moved / (k_avg * 1e-3) / 1e9
    roof = dict(bound="hbm", achieved=round(achieved, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(achieved / HBM_PEAK_GBS, 4), traffic=measured_traffic(args.workload, ["store"]),
                kernel="store", kernel_avg_us=round(k_avg * 1e3, 2), launches=k_n)
    cpu = None
    if not args.no_cpu_baseline:
        d = sets[0]
        n_s = 2048
        kh = np.zeros((NP, Hkv, P, 128), np.uint8)
        vh = np.zeros((NP, Hkv, P, 128), np.uint8)
        kf, vf, lf = d["k_cpu"][:n_s].float().numpy(), d["v_cpu"][:n_s].float().numpy(), d["loc_cpu"][:n_s].numpy()
        t0 = time.time()
        reps = 0
        while time.time() - t0 < 5.0:
            store_ref.store_kv(kf, vf, lf, kh, vh, P)
            reps += 1
        el = time.time() - t0
        cpu = {"value": round(moved * n_s / N * reps / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{n_s} of {N} new tokens, repeated {reps}x ({el:.1f} s of oracle time); "
                         f"bytes scaled by the sampled fraction"}
    res = {"metric": STORE_METRIC, "value": round(moved / (ms_step * 1e-3) / 1e9, 2), "unit": "GB/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16->fp8",
           "data": "synthetic",
           "config": {"workload": f"{args.workload}: {DESCRIPTIONS[args.workload]}", "new_tokens": N,
                      "bytes_per_step": moved, "parallelism": "single GPU", "input_sets": 2},
           "roofline": roof, "cpu_baseline": cpu}
    print(json.dumps(res), flush=True)


def bench_select(args, torch, msa):
    """The block-selection benchmark: one step is one msa_select_blocks call."""
    import workloads as W
    from oracle import decode as odecode  # the CPU baseline leg only
    from oracle import select_ref

    dev = torch.device("cuda:0")
    seed0 = W.SELECT_CONFIGS[args.workload]["seed"]
    sets = []
    for i in range(2):
        si = W.SELECT_MAKERS[args.workload](seed=seed0 + 1000 * i, poison=False)
        sets.append(dict(si=si, q=si.q_idx.to(dev), k=si.k_idx.to(dev),
                         bt=torch.from_numpy(si.block_tables).to(dev),
                         cu=torch.from_numpy(si.cu_seqlens_q).to(dev),
                         used=torch.from_numpy(si.used_kv_lens).to(dev)))
    si0 = sets[0]["si"]
    kelem = si0.k_idx.element_size()
    # algorithmic work of one step (set 0; set 1 is drawn the same way):
    # every visible index key is read once per (sequence, KV head) and
    # multiplied with each query token of the sequence that sees it
    seq, pos = select_ref._positions(si0.cu_seqlens_q, si0.used_kv_lens, si0.Tq, si0.causal)
    keys_read = sum(int(L) for s, L in enumerate(si0.used_kv_lens) if np.any(seq == s)) * si0.Hkv
    pairs = int(np.sum(np.where(seq >= 0, pos + 1, 0))) * si0.Hkv
    bytes_step = keys_read * 128 * kelem + si0.Tq * si0.Hkv * (256 + 4 * si0.topk)
    flops_step = 2 * 128 * pairs
    sel = torch.empty((si0.Tq, si0.Hkv, si0.topk), dtype=torch.int32, device=dev)

    def step(i):
        d = sets[i % 2]
        msa.select_blocks(d["q"], d["k"], d["bt"], cu_seqlens_q=d["cu"], used_kv_lens=d["used"],
                          page_size=si0.page_size, topk=si0.topk, causal=si0.causal, selected=sel)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        step(i)
    stop.record(stream)
    stop.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    msa.profile_enable(["select"])
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    k_ms, k_n = msa.profile_collect("select")
    msa.profile_enable([])
    k_avg = k_ms / max(k_n, 1)
    decode = args.workload == "select_decode"
    if decode:
        achieved, peak, unit, bound = bytes_step / (k_avg * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", "hbm"
        value = bytes_step / (ms_step * 1e-3) / 1e9
    else:
        achieved, peak, unit, bound = flops_step / (k_avg * 1e-3) / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", "mfma"
        value = flops_step / (ms_step * 1e-3) / 1e12
    roof = dict(bound=bound, achieved=round(achieved, 2), peak=peak, unit=unit, frac=round(achieved / peak, 4),
                traffic=measured_traffic(args.workload, ["select"]), kernel="select",
                kernel_avg_us=round(k_avg * 1e3, 2), launches=k_n)
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle on whole (token, KV head) rows of set 0, one sequence's
        # pages de-paged per row, until 5 s have passed
        rng = np.random.default_rng(11)
        t_start, done_bytes, done_flops, n_rows = time.time(), 0, 0, 0
        while time.time() - t_start < 5.0:
            t = int(rng.integers(si0.Tq))
            g = int(rng.integers(si0.Hkv))
            s = int(seq[t])
            L = int(si0.used_kv_lens[s])
            n = -(-L // si0.page_size)
            pages = torch.from_numpy(si0.block_tables[s, :n].astype(np.int64))
            a = int(si0.cu_seqlens_q[s])
            sub_k = odecode(si0.k_idx[pages][:, g:g + 1])
            sub_q = odecode(si0.q_idx[a:int(si0.cu_seqlens_q[s + 1]), g:g + 1])
            sc = select_ref.block_scores(sub_q, sub_k, np.arange(n, dtype=np.int32)[None, :], [0, sub_q.shape[0]],
                                         [L], si0.page_size, si0.causal, tokens=[t - a])
            select_ref.select_topk(sc[t - a:t - a + 1], si0.topk, [0, 1], [L], False, True)
            done_bytes += L * 128 * kelem
            done_flops += 2 * 128 * (int(pos[t]) + 1)
            n_rows += 1
        el = time.time() - t_start
        cpu_val = done_bytes / el / 1e9 if decode else done_flops / el / 1e12
        cpu = {"value": round(cpu_val, 5), "unit": unit, "cores": 1, "kind": "oracle",
               "sample": f"{n_rows} random (token, KV head) rows of one input set, each scored over its "
                         f"sequence's keys ({el:.1f} s of oracle time)"}
    res = {"metric": SELECT_METRIC[args.workload][0], "value": round(value, 2), "unit": unit,
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16 x " + ("fp8" if kelem == 1 else "bf16") + " -> fp32", "data": "synthetic",
           "config": {"workload": f"{args.workload}: {DESCRIPTIONS[args.workload]}", "query_tokens": si0.Tq,
                      "index_key_bytes_per_step": bytes_step, "flops_per_step": flops_step,
                      "parallelism": "single GPU", "input_sets": 2},
           "roofline": roof, "cpu_baseline": cpu}
    print(json.dumps(res), flush=True)


def _decoded(wl, g):
    """The MXFP4 workload's slices of KV head g as exact fp32 values, decoded
    by the oracle (its caches are then those the oracle's attention reads)."""
    import dataclasses

    import torch
    from oracle import mxfp4

    keep = wl.slice_head == g
    idx = torch.from_numpy(np.nonzero(keep)[0])

    def dec(codes, scales):
        return torch.from_numpy(mxfp4.dequantize(codes[idx].numpy(), scales[idx].numpy())).float()

    return dataclasses.replace(wl, kv_dtype=torch.float32, slice_page=wl.slice_page[keep],
                               slice_head=wl.slice_head[keep], k_vals=dec(wl.k_vals, wl.k_scales),
                               v_vals=dec(wl.v_vals, wl.v_scales), k_scales=None, v_scales=None)


def cpu_baseline(wl, acct, budget_pairs=None, min_seconds=5.0):
    """Time the fp64 oracle over a bounded sample of (token, KV head) pairs.

    The sample is repeated until at least ``min_seconds`` of oracle time has
    accumulated; the rate is unique-KV bytes of the sample per second.
    """
    import oracle
    import workloads as W

    tot = wl.Tq * wl.Hkv
    n = tot if budget_pairs is None else min(tot, budget_pairs)
    rng = np.random.default_rng(0)
    pairs = np.sort(rng.choice(tot, size=n, replace=False)) if n < tot else np.arange(tot)
    G = wl.G
    groups = []
    for g in np.unique(pairs % wl.Hkv):
        toks = pairs[pairs % wl.Hkv == g] // wl.Hkv
        k, v, bt = W.compact_cache(_decoded(wl, int(g)) if wl.mxfp4 else wl, heads=[int(g)])
        q = wl.q[:, g * G:(g + 1) * G, :].contiguous()
        sel = np.ascontiguousarray(wl.selected[:, g:g + 1, :])
        groups.append((q, k, v, sel, bt, toks))
    secs, reps = 0.0, 0
    while secs < min_seconds or reps == 0:
        for q, k, v, sel, bt, toks in groups:
            t0 = time.perf_counter()
            oracle.attention(q, k, v, sel, bt, wl.cu_seqlens_q, wl.used_kv_lens, wl.causal, pairs=toks)
            secs += time.perf_counter() - t0
        reps += 1
    frac = n / tot
    cores = oracle.max_threads()
    # one thread: growing slices of the same pairs until min_seconds / 2
    done, secs1 = 0, 0.0
    m = max(1, n // 64)
    while secs1 < min_seconds / 2:
        for q, k, v, sel, bt, toks in groups:
            part = toks[:m]
            t0 = time.perf_counter()
            oracle.attention(q, k, v, sel, bt, wl.cu_seqlens_q, wl.used_kv_lens, wl.causal, pairs=part, threads=1)
            secs1 += time.perf_counter() - t0
            done += part.size
            if secs1 >= min_seconds / 2:
                break
        m = min(2 * m, n)
    return dict(
        value=round(acct["unique_kv_bytes"] * frac * reps / secs / 1e9, 4),
        unit="GB/s",
        cores=cores,
        kind="oracle",
        sample=f"{n} of {tot} (token, kv-head) pairs of one batch ({100 * frac:.0f}%), repeated {reps}x "
               f"({secs:.1f} s of fp64 oracle time); unique-KV bytes scaled by the sampled fraction",
        single_thread_value=round(acct["unique_kv_bytes"] * done / tot / secs1 / 1e9, 4),
        single_thread_sample=f"{done} pairs of the same sample on one thread ({secs1:.1f} s)",
    )


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_gqa", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-pairs", type=int, default=None, help="oracle sample size in (token, kv-head) pairs")
    ap.add_argument("--profile-summaries", metavar="DIR", default=None,
                    help="only write profiles/kernels_<w>.md and profiles/traffic_<w>.txt from the rocprofv3 "
                         "outputs under DIR (see PROF_TRACE_CMD, PROF_PMC_CMD, PROF_COPY_CMD); needs no GPU")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (reference kernel for the "
                         "FETCH_SIZE / WRITE_SIZE counters) and print its size")
    ap.add_argument("--micro", nargs="*", metavar="WHAT", default=None,
                    help="only run the rate measurements of lib/msa_rates (hbm, launch, lds, mix, chain; "
                         "default all): device rates the kernels' designs rest on")
    args = ap.parse_args()

    if args.profile_summaries:
        write_profile_summaries(args.profile_summaries)
        return
    if args.micro is not None:
        # a child process of its own: this one never touches the GPU
        from block_sparse_attention_selection_amd.build import RATES
        if not os.path.exists(RATES):
            print(f"{RATES} is not built (python -m block_sparse_attention_selection_amd.build)", file=sys.stderr)
            sys.exit(1)
        sys.exit(subprocess.call([RATES, *args.micro]))
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_sparse_attention_selection_amd as msa
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}), flush=True)
        return
    msa.load()
    if args.workload == "kv_store_fp8":
        bench_store(args, torch, msa)
        return
    if args.workload in SELECT_METRIC:
        bench_select(args, torch, msa)
        return
    seed0 = W.CONFIGS[args.workload]["seed"]

    batches = []
    for i in range(2):
        t0 = time.time()
        wl = W.make(args.workload, seed=seed0 + 1000 * i, poison=False)
        if wl.mxfp4:
            k, ks, v, vs = W.mxfp4_pool(wl, device=dev)
        else:
            (k, v), ks, vs = W.kv_pool(wl, device=dev), None, None
        d = dict(q=wl.q.to(dev), k=k, v=v, ks=ks, vs=vs, sel=torch.from_numpy(wl.selected).to(dev),
                 bt=torch.from_numpy(wl.block_tables).to(dev),
                 cu=torch.from_numpy(wl.cu_seqlens_q).to(dev), used=torch.from_numpy(wl.used_kv_lens).to(dev))
        d["out"] = torch.empty_like(d["q"])
        d["lse"] = torch.empty((wl.Hq, wl.Tq), dtype=torch.float32, device=dev)
        acct = accounting(wl)
        batches.append((wl, d, acct))
        log(f"batch {i}: {args.workload} generated in {time.time() - t0:.1f}s, "
            f"unique KV {acct['unique_kv_bytes'] / 1e6:.1f} MB, {acct['effective_flops'] / 1e9:.2f} GFLOP")

    def step(i):
        wl, d, _ = batches[i % 2]
        if wl.mxfp4:
            msa.kvouter_attention_mxfp4(d["q"], d["k"], d["ks"], d["v"], d["vs"], d["sel"], d["bt"],
                                        cu_seqlens_q=d["cu"], used_kv_lens=d["used"], page_size=wl.page_size,
                                        causal=wl.causal, return_lse=True, out=d["out"], lse=d["lse"])
        else:
            msa.kvouter_attention(d["q"], d["k"], d["v"], d["sel"], d["bt"], cu_seqlens_q=d["cu"],
                                  used_kv_lens=d["used"], page_size=wl.page_size, causal=wl.causal,
                                  return_lse=True, out=d["out"], lse=d["lse"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    dom = DOMINANT[args.workload]
    stream = torch.cuda.current_stream(dev)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)

    # timed region: whole calls, no instrumentation inside
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(i)
    stop.record(stream)
    stop.synchronize()
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps

    # the distribution of single steps: the same steps with one event
    # between consecutive calls (an event adds a little time, so the mean
    # step above is taken without them)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        step(i)
        evs[i + 1].record(stream)
    evs[-1].synchronize()
    per_step_us = np.array([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(args.steps)])

    # same steps again, timing the dominant kernels: their dispatches record
    # HIP events at the kernels' start and end (msa_profile_enable), so the
    # kernel time excludes everything between launches
    msa.profile_enable(dom)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    per_kernel = {}
    for kname in dom:
        ms_k, n_k = msa.profile_collect(kname)
        per_kernel[kname] = (ms_k, n_k)
    msa.profile_enable([])
    k_ms = sum(v[0] for v in per_kernel.values())
    k_n = min(v[1] for v in per_kernel.values())

    ukv = np.mean([b[2]["unique_kv_bytes"] for b in batches])
    flops = np.mean([b[2]["effective_flops"] for b in batches])
    qo = np.mean([b[2]["qo_bytes"] for b in batches])
    value = ukv / (ms_step * 1e-3) / 1e9
    k_avg_ms = k_ms / max(k_n, 1)
    wl0 = batches[0][0]
    decode = args.workload.startswith("decode")
    if decode or args.workload == "tiny":
        alg = ukv + qo
        achieved = alg / (k_avg_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=None)
    else:
        achieved = flops / (k_avg_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), traffic=None)
    roof["traffic"] = measured_traffic(args.workload, dom)
    roof["traffic_kind"] = ("FETCH_SIZE + WRITE_SIZE per launch, scaled by a plain copy's counts: bytes between "
                            "L2 and the data fabric, MALL hits included, so an upper bound on HBM bytes")
    roof["kernel"] = "+".join(dom)
    roof["kernel_avg_us"] = round(k_avg_ms * 1e3, 2)
    roof["kernel_within_step"] = bool(k_avg_ms <= ms_step)
    roof["per_kernel_avg_us"] = {k: round(v[0] / max(v[1], 1) * 1e3, 2) for k, v in per_kernel.items()}
    roof["launches"] = k_n

    cpu = None
    if not args.no_cpu_baseline:
        try:
            cpu = cpu_baseline(wl0, batches[0][2], args.cpu_pairs)
        except Exception as e:  # the baseline is informative; never fail the bench on it
            log("cpu baseline failed:", repr(e))

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bfloat16": "bf16", "float16": "fp16"}[str(wl0.q_dtype).split(".")[-1]]
                 + ("+mxfp4kv" if wl0.mxfp4 else "+fp8kv" if wl0.kv_dtype != wl0.q_dtype else ""),
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: {DESCRIPTIONS[args.workload]}",
            "batch_sequences": wl0.B,
            "query_tokens": wl0.Tq,
            "unique_kv_bytes_per_step": int(ukv),
            "effective_flops_per_step": int(flops),
            "decode_step_us": round(ms_step * 1e3, 2),
            "step_us_median": round(float(np.median(per_step_us)), 2),
            "step_us_p10": round(float(np.percentile(per_step_us, 10)), 2),
            "step_us_p90": round(float(np.percentile(per_step_us, 90)), 2),
            "effective_tflops": round(flops / (ms_step * 1e-3) / 1e12, 3),
            "hbm_frac_of_peak": round(value / HBM_PEAK_GBS, 4),
            "parallelism": "single GPU",
            "input_sets": 2,
        },
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
