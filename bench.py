"""Benchmark of the DSA hot path on one MI355X.

One step = one decode step of the whole path on one batch of synthetic
queries, launched as a serving loop issues it: the three C-ABI calls on the
stream, call 1 (append the new key, quantise q, lightning-indexer score),
call 2 (causal top-2048), call 3 (sparse absorbed MLA), with argument
structs built once per cache replica outside the timed region. The same
steps replayed as one captured HIP graph per step are reported beside it. The default workload
is decode at L = 16384 (B = 1), the configuration the headline metric is
quoted on; --workload selects another one (batch32, decode128k).

Inputs are resident in HBM before the timed region. Every step reads its
caches from one of R replicas (R * footprint >= 1 GiB and R * bytes touched
per step >= 1 GiB) so the 256 MiB Infinity Cache cannot serve them;
scores/idx/out buffers are reused like a serving loop's workspace. HIP events on the launch stream bracket the timed
region. Each call's device time is then measured the same way over a graph
that runs that call once per replica, back to back; the call with the
largest average is the "dominant kernel" of the roofline object. The
batched decode (32 rows) and the long-context decode (4 rows at L = 131072)
are measured the same way under "other_workloads".

Prints ONE JSON line. `cpu_baseline` is the CPU oracle (oracle/) timed on
the host's cores on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode16k",
                    choices=["decode16k", "batch32", "decode128k"])
    ap.add_argument("--replica-bytes", type=float, default=float(1 << 30),
                    help="minimum total bytes of rotated cache replicas")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the batched and long-context decode workloads")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the paged-cache / Hadamard / cache-append measurements")
    ap.add_argument("--only-prefill", action="store_true",
                    help="run only the prefill leg and print its JSON object (for profiling)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill leg (T = 4096 causal queries, per-call TFLOP/s)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time for the oracle sample")
    ap.add_argument("--sweep", action="store_true",
                    help="add the supplementary batch sweep (B = 1..64 rows at L = 16384)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 512 MiB device-to-device copy five times (the "
                         "reference kernel for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="turn four rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE and "
                         "WRITE_SIZE of this benchmark, then of --calibrate-copy) into "
                         "profiles/counters.json and exit")
    return ap.parse_args()


# kernels launched by each call of the path (substrings of rocprofv3 kernel names)
KERNELS_OF_CALL = {
    "indexer": ["decode_score_kernel"],
    "topk": ["topk_select_kernel"],
    "sparse_mla": ["sparse_mla_kernel", "sparse_mla_pair_kernel", "sparse_mla_ring_kernel",
                   "merge_few_kernel", "combine_regs_kernel", "combine_kernel"],
}


def summarize_counters(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, workload):
    """HBM bytes per call launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by the ratio of the true bytes of a 512 MiB device
    copy to what the same counter reads for that copy."""
    import csv
    from collections import defaultdict

    def per_kernel(path, counter):
        d = defaultdict(list)
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    d[r["Kernel_Name"]].append(float(r["Counter_Value"]) * 1024.0)
        return d

    def name_matches(k, sub):
        # the kernel's own name (before its template arguments) is `sub`
        base = k.split("(")[0].split("<")[0]
        return base.endswith("::" + sub) or base == sub

    def mean_of(d, sub, required=True):
        """Bytes per launch of the kernels named `sub`: the mean over the
        dispatches of each instantiation, summed over the instantiations (a
        call may launch several, e.g. the two levels of a long-row top-k)."""
        names = [k for k in d if name_matches(k, sub)]
        if not names:
            if not required:
                return None, 0
            raise SystemExit(f"no dispatch of a kernel named like {sub!r}")
        return (sum(sum(d[k]) / len(d[k]) for k in names),
                min(len(d[k]) for k in names))

    copy_bytes = float(512 << 20)
    def copy_mean(d):
        vals = [v for k, vs in d.items() if "copyBuffer" in k for v in vs]
        if not vals:
            raise SystemExit("no dispatch of the device copy")
        return sum(vals) / len(vals)

    f_scale = copy_bytes / copy_mean(per_kernel(copy_fetch_csv, "FETCH_SIZE"))
    w_scale = copy_bytes / copy_mean(per_kernel(copy_write_csv, "WRITE_SIZE"))
    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    out = os.path.join(ROOT, "profiles", "counters.json")
    srch = source_hash()
    try:
        allrec = json.load(open(out))
    except (OSError, ValueError):
        allrec = {}
    if allrec.get("source_hash") != srch or "workloads" not in allrec:
        allrec = {"source_hash": srch, "workloads": {}}
    rec = {"fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)}
    for call, subs in KERNELS_OF_CALL.items():
        ent = {"kernels": {}}
        tf = tw = 0.0
        for sub in subs:
            fb, n = mean_of(fetch, sub, required=False)       # a call's kernels vary with its shape
            if fb is None:
                continue
            wb, _ = mean_of(write, sub)
            ent["kernels"][sub] = {"fetch_bytes": round(fb * f_scale), "write_bytes": round(wb * w_scale),
                                   "dispatches": n}
            tf += fb * f_scale
            tw += wb * w_scale
        if not ent["kernels"]:
            raise SystemExit(f"no dispatch of a kernel of call {call!r}")
        ent.update(fetch_bytes=round(tf), write_bytes=round(tw), bytes_per_launch=round(tf + tw))
        rec[call] = ent
    allrec["workloads"][workload] = rec
    with open(out, "w") as fh:
        json.dump(allrec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec))


def calibrate_copy():
    import torch
    n = 512 << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n,
                      "launches": 5}), flush=True)


# ------------------------------------------------------------ byte model --

def algorithmic_bytes(wl, n_valid, keff):
    """Bytes the method itself must move per call, summed over the batch:
    per row, the indexer reads n_valid FP8 keys and scales, the query and
    weights and appends one key; top-k reads n_valid scores and writes
    k_eff indices; the attention reads k_eff indices, gathers k_eff latent
    and rotary rows and reads the query and writes the output."""
    n_valid = np.asarray(n_valid, np.int64)
    keff = np.asarray(keff, np.int64)
    H, Hq = wl.H, wl.Hq
    act = 2
    indexer = int(np.sum(n_valid * (128 + 4) + H * 128 * act + H * 4 + (128 * act + 128 + 4)))
    topk = int(np.sum(4 * n_valid + 4 * keff))
    mla = int(np.sum(4 * keff + 1152 * keff + Hq * 576 * 2 + Hq * 512 * 2))
    # step total: the scores round trip (write by call 1, read by call 2) is
    # a cost of the three-call split, not of the method
    step = indexer + int(np.sum(4 * keff)) + int(np.sum(1152 * keff + Hq * 576 * 2 + Hq * 512 * 2))
    return dict(indexer=indexer, topk=topk, sparse_mla=mla, step=step)


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_attention_index_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel_call, srchash, workload):
    """HBM traffic per launch of a call on a workload from the committed
    rocprofv3 counter summary, if it was taken on the current kernel
    sources."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != srchash:
        return None
    ent = rec.get("workloads", {}).get(workload, {}).get(kernel_call)
    return ent.get("bytes_per_launch") if ent else None


# ----------------------------------------------------------------- setup --

def setup(wl, replica_bytes):
    import torch

    import sparse_attention_index_amd as dsa
    import synth

    x = synth.make_inputs(wl)
    dev = torch.device("cuda")
    B, S, L = wl.B, wl.S, wl.Lmax
    cos, sin = dsa.rope_table(L, yarn=wl.yarn)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    k_all = torch.from_numpy(x["k_raw"]).to(dev).to(torch.bfloat16)
    kc = torch.zeros((B, L, 128), dtype=torch.uint8, device=dev)
    ks = torch.zeros((B, L), dtype=torch.float32, device=dev)
    dsa.indexer_append(k_all, torch.arange(L, dtype=torch.int32, device=dev)[None].expand(B, L)
                       .contiguous(), cos, sin, kc, ks)
    latent, kpe = bf16(x["latent"]), bf16(x["kpe"])
    pos_np = x["pos"]
    pos = torch.from_numpy(pos_np).to(dev)
    k_new = torch.stack([k_all[b, pos_np[b]] for b in range(B)]).contiguous()   # [B,S,128]
    q_raw = torch.from_numpy(x["q_raw"]).to(dev).to(torch.bfloat16)
    w = torch.from_numpy(x["w"]).to(dev)
    q_mla = bf16(x["q_mla"])
    del k_all
    per_replica = kc.numel() + ks.numel() * 4 + latent.numel() * 2 + kpe.numel() * 2
    # replicas: R * footprint >= replica_bytes, and also R * (bytes one step
    # touches) >= replica_bytes, so that the rotation's touched set alone is
    # several times the Infinity Cache
    n_valid = [int(p) + 1 for p in pos_np.reshape(-1)]
    touched = algorithmic_bytes(wl, n_valid, [min(wl.K, n) for n in n_valid])["step"]
    R = max(2, int(np.ceil(replica_bytes / per_replica)), int(np.ceil(replica_bytes / touched)))
    reps = [dict(kc=kc, ks=ks, latent=latent, kpe=kpe)]
    for _ in range(R - 1):
        reps.append(dict(kc=kc.clone(), ks=ks.clone(), latent=latent.clone(), kpe=kpe.clone()))
    scores = torch.empty((B, S, L), dtype=torch.float32, device=dev)
    idx = torch.empty((B, S, wl.K), dtype=torch.int32, device=dev)
    out = torch.empty((B, S, wl.Hq, 512), dtype=torch.bfloat16, device=dev)
    q8 = torch.empty((B, S, wl.H, 128), dtype=torch.uint8, device=dev)
    qs = torch.empty((B, S, wl.H), dtype=torch.float32, device=dev)
    # workspaces sized once, outside the timed region
    mla_ws_args = dsa.mla_args(q_mla, latent, kpe, idx, wl.softmax_scale, out)
    mla_ws = torch.empty(max(1, dsa.sparse_mla_workspace_bytes(mla_ws_args)), dtype=torch.uint8,
                         device=dev)
    topk_ws = dsa.topk_workspace(scores, pos, wl.K)
    torch.cuda.synchronize()
    return dict(x=x, cos=cos, sin=sin, pos=pos, k_new=k_new, q_raw=q_raw, w=w, q_mla=q_mla,
                reps=reps, R=R, per_replica=per_replica, scores=scores, idx=idx, out=out, q8=q8,
                qs=qs, mla_ws=mla_ws, topk_ws=topk_ws)


def make_calls(wl, st):
    """The three calls of one step, bound to replica r."""
    import sparse_attention_index_amd as dsa

    def indexer(r):
        rep = st["reps"][r % st["R"]]
        dsa.indexer(st["q_raw"], st["w"], st["pos"], st["cos"], st["sin"], rep["kc"], rep["ks"],
                    st["scores"], k_raw=st["k_new"], q_fp8=st["q8"], q_scale=st["qs"])

    def topk(r):
        dsa.topk(st["scores"], st["pos"], wl.K, idx=st["idx"], workspace=st["topk_ws"])

    def sparse_mla(r):
        rep = st["reps"][r % st["R"]]
        dsa.sparse_mla(st["q_mla"], rep["latent"], rep["kpe"], st["idx"], wl.softmax_scale,
                       out=st["out"], workspace=st["mla_ws"])

    return {"indexer": indexer, "topk": topk, "sparse_mla": sparse_mla}


def capture(fn):
    """Record fn() into a HIP graph (launches on torch's capture stream)."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


# ------------------------------------------------------------- timing --

def eager_stepper(wl, st):
    """The step as a serving loop issues it: the three C-ABI calls launched on
    the stream, argument structs built once per replica outside the timed
    region. Returns steps(first, n), which enqueues steps first..first+n-1."""
    import ctypes

    import torch

    import sparse_attention_index_amd as dsa

    L = dsa.lib()
    ia = [dsa.indexer_args(st["q_raw"], st["w"], st["pos"], st["cos"], st["sin"], rep["kc"],
                           rep["ks"], st["scores"], k_raw=st["k_new"], q_fp8=st["q8"],
                           q_scale=st["qs"]) for rep in st["reps"]]
    ma = [dsa.mla_args(st["q_mla"], rep["latent"], rep["kpe"], st["idx"], wl.softmax_scale,
                       st["out"], workspace=st["mla_ws"]) for rep in st["reps"]]
    ta = dsa.topk_args(st["scores"], st["pos"], wl.K, st["idx"], workspace=st["topk_ws"])
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    byref = ctypes.byref
    R = st["R"]
    st["eager_args"] = (ia, ta, ma)               # kept alive with the state

    def steps(first, n):
        for i in range(first, first + n):
            r = i % R
            c1 = L.dsa_indexer(byref(ia[r]), sp)
            c2 = L.dsa_topk(byref(ta), sp)
            c3 = L.dsa_sparse_mla(byref(ma[r]), sp)
            if c1 or c2 or c3:
                raise RuntimeError(f"step {i}: status {c1} {c2} {c3}")

    return steps


def measure(wl, st, steps, warmup):
    """Time `steps` steps launched eagerly (three C-ABI calls per step, the
    replicas in rotation), the same steps replayed as one captured graph per
    step, and each call's average device time; returns the figures of the
    bench record."""
    import torch

    calls = make_calls(wl, st)
    st["calls"] = calls
    R = st["R"]

    def step(r):
        for c in ("indexer", "topk", "sparse_mla"):
            calls[c](r)

    # eager warm-up (one-time kernel attribute set-up happens here), then one
    # graph per replica for the step and one graph per call covering all
    # replicas back to back
    for r in range(min(R, 3)):
        step(r)
    torch.cuda.synchronize()
    run = eager_stepper(wl, st)
    run(0, warmup)
    torch.cuda.synchronize()

    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    run(warmup, steps)
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)

    # distribution of single steps: a second pass with an event between steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        run(i, 1)
        evs[i + 1].record()
    torch.cuda.synchronize()
    per_step_us = np.array([evs[i].elapsed_time(evs[i + 1]) * 1000.0 for i in range(steps)])
    quantiles = {k: round(float(np.percentile(per_step_us, q)), 2)
                 for k, q in (("p10", 10), ("p50", 50), ("p90", 90))}

    # the same steps as one captured graph per step, replayed in rotation
    step_graphs = [capture(lambda r=r: step(r)) for r in range(R)]
    for i in range(min(warmup, R)):
        step_graphs[i % R].replay()
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        step_graphs[i % R].replay()
    stop.record()
    torch.cuda.synchronize()
    graph_ms = start.elapsed_time(stop)
    del step_graphs

    # per-call device time: each call graph runs the call once per replica
    call_graphs = {c: capture(lambda c=c: [calls[c](r) for r in range(R)]) for c in calls}
    reps_call = max(1, (steps + R - 1) // R)
    avg_us = {}
    for c, g in call_graphs.items():
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps_call):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        avg_us[c] = a.elapsed_time(b) * 1000.0 / (reps_call * R)
    del call_graphs

    n_valid = [int(p) + 1 for p in st["x"]["pos"].reshape(-1)]
    keff = [min(wl.K, n) for n in n_valid]
    ab = algorithmic_bytes(wl, n_valid, keff)
    dom = max(avg_us, key=avg_us.get)
    ms_per_step = total_ms / steps
    return dict(ab=ab, dom=dom, avg_us=avg_us, ms_per_step=ms_per_step, quantiles=quantiles,
                achieved=ab[dom] / (avg_us[dom] * 1e-6) / 1e9,
                value=wl.B * wl.S * steps / (total_ms / 1000.0),
                graph_us_per_step=graph_ms * 1000.0 / steps,
                step_hbm_frac=round(ab["step"] / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))


def other_workloads_leg(args):
    """The same measurement on the batched decode (32 rows of ragged length
    2048..16384) and the long-context decode (4 rows at L = 131072)."""
    import torch

    import synth

    out = {}
    for name in ("batch32", "decode128k"):
        wl = synth.workload(name)
        st = setup(wl, args.replica_bytes)
        m = measure(wl, st, args.steps, args.warmup)
        dom = m["dom"]
        out[name] = {
            "value": round(m["value"], 1), "unit": "queries/s",
            "ms_per_step": round(m["ms_per_step"], 5),
            "graph_per_step_us": round(m["graph_us_per_step"], 2),
            "step_us_quantiles": m["quantiles"],
            "config": {"B": wl.B, "L": wl.Lmax, "topk": wl.K, "replicas": st["R"],
                       "replica_bytes": st["per_replica"]},
            "step_algorithmic_bytes": m["ab"]["step"],
            "step_hbm_frac": m["step_hbm_frac"],
            "call_avg_us": {k: round(v, 2) for k, v in m["avg_us"].items()},
            "dominant": {"kernel": dom, "achieved_gbs": round(m["achieved"], 1),
                         "frac": round(m["achieved"] / HBM_PEAK_GBS, 4),
                         "bytes_per_launch": m["ab"][dom],
                         "traffic": load_traffic(dom, source_hash(), name)},
        }
        del st, m
        torch.cuda.empty_cache()
    return out


def sweep_leg(args):
    """Supplementary: decode16k's shapes at B = 1, 4, 16, 32, 64 rows (all at
    L = 16384), to show where the single-row latency stops dominating."""
    import torch

    import synth

    out = {}
    for B in (1, 4, 16, 32, 64):
        wl = synth.sweep_workload(B)
        st = setup(wl, args.replica_bytes)
        m = measure(wl, st, args.steps, args.warmup)
        out[f"B={B}"] = {
            "value": round(m["value"], 1), "unit": "queries/s",
            "us_per_step": round(m["ms_per_step"] * 1000.0, 2),
            "step_hbm_frac": m["step_hbm_frac"],
            "call_avg_us": {k: round(v, 2) for k, v in m["avg_us"].items()},
        }
        del st, m
        torch.cuda.empty_cache()
    return out


# --------------------------------------------------------- variants leg --

def _graph_us(fn, reps):
    """Average device time of fn() over graph replays of `reps` calls."""
    import torch
    g = capture(lambda: [fn(r) for r in range(reps)])
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(3):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1000.0 / (3 * reps)


def variants_leg(wl, st, page=64):
    """The same decode step on paged caches (a random page permutation of a
    page pool per replica), the indexer call with the Hadamard rotation and
    power-of-two scales, and the MLA-side cache append."""
    import torch

    import sparse_attention_index_amd as dsa

    dev = torch.device("cuda")
    R, L = st["R"], wl.Lmax
    B = wl.B
    max_pages = (L + page - 1) // page
    num_pages = B * max_pages
    gen = torch.Generator(device="cpu")
    gen.manual_seed(7)
    table = torch.randperm(num_pages, generator=gen).to(torch.int32).reshape(B, max_pages)
    paging = dsa.Paging(table.to(dev), page, num_pages)
    flat = table.reshape(-1).long().to(dev)
    pools = []
    for rep in st["reps"]:
        kc = torch.empty((num_pages, page, 128), dtype=torch.uint8, device=dev)
        ks = torch.empty((num_pages, page), dtype=torch.float32, device=dev)
        lr = torch.empty((num_pages, page, 576), dtype=torch.bfloat16, device=dev)
        kc[flat] = rep["kc"].reshape(B * max_pages, page, 128)
        ks[flat] = rep["ks"].reshape(B * max_pages, page)
        lr[flat, :, :512] = rep["latent"].reshape(B * max_pages, page, 512)
        lr[flat, :, 512:] = rep["kpe"].reshape(B * max_pages, page, 64)
        pools.append((kc, ks, lr))
    scores_p = torch.empty((B, wl.S, paging.lmax), dtype=torch.float32, device=dev)

    def paged_step(r):
        kc, ks, lr = pools[r % R]
        dsa.indexer(st["q_raw"], st["w"], st["pos"], st["cos"], st["sin"], kc, ks, scores_p,
                    k_raw=st["k_new"], q_fp8=st["q8"], q_scale=st["qs"], paging=paging)
        dsa.topk(scores_p, st["pos"], wl.K, idx=st["idx"], workspace=st["topk_ws"])
        dsa.sparse_mla(st["q_mla"], lr[..., :512], lr[..., 512:], st["idx"], wl.softmax_scale,
                       out=st["out"], workspace=st["mla_ws"], paging=paging)

    paged_us = _graph_us(paged_step, R)

    def dense_step(r):
        for c in ("indexer", "topk", "sparse_mla"):
            st["calls"][c](r)

    chained_us = _graph_us(dense_step, R)

    def had_idx(r):
        rep = st["reps"][r % R]
        dsa.indexer(st["q_raw"], st["w"], st["pos"], st["cos"], st["sin"], rep["kc"], rep["ks"],
                    st["scores"], k_raw=st["k_new"], q_fp8=st["q8"], q_scale=st["qs"],
                    hadamard=True, pow2_scale=True)

    had_us = _graph_us(had_idx, R)

    lat_new = torch.randn((B, wl.S, 512), device=dev).to(torch.bfloat16)
    kpe_new = torch.randn((B, wl.S, 64), device=dev).to(torch.bfloat16)
    q_app = st["q_mla"].clone()

    def append(r):
        rep = st["reps"][r % R]
        dsa.mla_append(lat_new, kpe_new, st["pos"], st["cos"], st["sin"], rep["latent"],
                       rep["kpe"], q=q_app)

    app_us = _graph_us(append, R)
    for kc, ks, lr in pools:
        del kc, ks, lr
    return {
        "chained_decode": {"us_per_step": round(chained_us, 2),
                           "value": round(B * wl.S / (chained_us * 1e-6), 1),
                           "unit": "queries/s",
                           "note": "the same dense step, one graph holding one step per "
                                   "replica back to back (no per-step graph launch)"},
        "paged_decode": {"workload": f"{wl.name} on paged caches (page_size {page}, permuted "
                                    f"pool of {num_pages} pages)",
                         "value": round(B * wl.S / (paged_us * 1e-6), 1), "unit": "queries/s",
                         "us_per_step": round(paged_us, 2),
                         "note": "timed like chained_decode"},
        "indexer_hadamard_pow2": {"avg_us": round(had_us, 2),
                                  "note": "one fused launch (rotate, quantise and append the key, rotate and quantise q, score)"},
        "mla_append": {"avg_us": round(app_us, 2),
                       "bytes": int(B * wl.S * (1024 * 2 + 128 * 2 + wl.Hq * 128 * 2)),
                       "note": "latent row copy, rotary key and 128 query rope parts"},
    }


# ---------------------------------------------------------- prefill leg --

BF16_MFMA_PEAK_TFLOPS = 2500.0
FP8_MFMA_PEAK_TFLOPS = 5000.0


def prefill_leg(reps=20, cpu=False):
    """Prefill of T = 4096 causal queries at positions 0..4095 (B = 1, L = 4096,
    H_I = 64, top-2048, 128 heads): each call timed on its own over graph
    replays. Inputs: seeded N(0,1) draws made on the GPU (torch generator,
    seed 3), bf16 activations, w scaled by 64^-0.5 128^-0.5."""
    import torch

    import sparse_attention_index_amd as dsa

    T, H, Hq, K = 4096, 64, 128, 2048
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=dev)

    q_raw = randn(1, T, H, 128).to(torch.bfloat16)
    k_raw = randn(1, T, 128).to(torch.bfloat16)
    w = randn(1, T, H) * (64 ** -0.5) * (128 ** -0.5)
    q_mla = randn(1, T, Hq, 576).to(torch.bfloat16)
    latent = randn(1, T, 512).to(torch.bfloat16)
    kpe = randn(1, T, 64).to(torch.bfloat16)
    pos = torch.arange(T, dtype=torch.int32, device=dev)[None].contiguous()
    cos, sin = dsa.rope_table(T)
    kc = torch.zeros((1, T, 128), dtype=torch.uint8, device=dev)
    ks = torch.zeros((1, T), dtype=torch.float32, device=dev)
    scores = torch.empty((1, T, T), dtype=torch.float32, device=dev)
    idx = torch.empty((1, T, K), dtype=torch.int32, device=dev)
    out = torch.empty((1, T, Hq, 512), dtype=torch.bfloat16, device=dev)
    scale = 192 ** -0.5
    iargs = dsa.indexer_args(q_raw, w, pos, cos, sin, kc, ks, scores, k_raw=k_raw)
    iws = torch.empty(max(1, dsa.indexer_workspace_bytes(iargs)), dtype=torch.uint8, device=dev)
    mws = torch.empty(max(1, dsa.sparse_mla_workspace_bytes(
        dsa.mla_args(q_mla, latent, kpe, idx, scale, out))), dtype=torch.uint8, device=dev)
    tws = dsa.topk_workspace(scores, pos, K)

    # the multi-head (non-absorbed) form and the absorption products, on the
    # same latent cache and selection; wkv_b ~ N(0, 1/512)
    wkv_b = (randn(Hq, 256, 512) * (512 ** -0.5)).to(torch.bfloat16)
    q_nope = randn(1, T, Hq, 128).to(torch.bfloat16)
    q192 = torch.cat([q_nope, q_mla[..., 512:]], -1).contiguous()
    kv = torch.empty((1, T, Hq, 256), dtype=torch.bfloat16, device=dev)
    o128 = torch.empty((1, T, Hq, 128), dtype=torch.bfloat16, device=dev)
    qa = torch.empty((1, T, Hq, 576), dtype=torch.bfloat16, device=dev)
    hws = torch.empty(max(1, dsa.sparse_mha_workspace_bytes(
        dsa.mha_args(q192, kv, kpe, idx, scale, o128, pos))), dtype=torch.uint8, device=dev)

    calls = {
        "indexer": lambda: dsa.indexer(q_raw, w, pos, cos, sin, kc, ks, scores, k_raw=k_raw,
                                       workspace=iws),
        "topk": lambda: dsa.topk(scores, pos, K, idx=idx, workspace=tws),
        "sparse_mla": lambda: dsa.sparse_mla(q_mla, latent, kpe, idx, scale, out=out,
                                             workspace=mws),
        "absorb_q": lambda: dsa.mla_absorb_q(q_nope, wkv_b, out=qa[..., :512]),
        "absorb_o": lambda: dsa.mla_absorb_o(out, wkv_b, out=o128),
        "kv_up": lambda: dsa.mla_kv_up(latent, wkv_b, out=kv),
        "sparse_mha": lambda: dsa.sparse_mha(q192, kv, kpe, idx, scale, pos=pos, out=o128,
                                             workspace=hws),
    }
    for c in calls:
        calls[c]()
    torch.cuda.synchronize()
    us = {}
    for c, fn in calls.items():
        g = capture(fn)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        us[c] = a.elapsed_time(b) * 1000.0 / reps
    pairs = T * (T + 1) // 2
    sel = sum(min(K, t + 1) for t in range(T))
    idx_tflop = 2.0 * H * 128 * pairs / 1e12
    mla_tflop = 2.0 * Hq * (576 + 512) * sel / 1e12
    topk_bytes = 4 * pairs + 4 * sel
    idx_tfs = idx_tflop / (us["indexer"] * 1e-6)
    mla_tfs = mla_tflop / (us["sparse_mla"] * 1e-6)
    gemm_tflop = {"absorb_q": 2.0 * T * Hq * 128 * 512 / 1e12,
                  "absorb_o": 2.0 * T * Hq * 512 * 128 / 1e12,
                  "kv_up": 2.0 * T * 512 * Hq * 256 / 1e12}
    # algorithmic bytes: A, B and C of each product, once (bf16)
    gemm_bytes = {"absorb_q": 2 * (T * Hq * 128 + Hq * 128 * 512 + T * Hq * 512),
                  "absorb_o": 2 * (T * Hq * 512 + Hq * 128 * 512 + T * Hq * 128),
                  "kv_up": 2 * (T * 512 + Hq * 256 * 512 + T * Hq * 256)}
    mha_tflop = 2.0 * Hq * (192 + 128) * sel / 1e12
    # executed work: every listed 64-position tile of each 128-row query tile
    toff = dsa.sparse_mha_tiles_offset(1, T, T)
    nqt = T // 128
    tl = hws[toff:toff + nqt * (T // 64 + 1) * 16].view(torch.int32).view(nqt, T // 64 + 1, 4)
    ntiles = int(tl[:, 0, 0].sum().item())
    mha_exec_tflop = 2.0 * Hq * (192 + 128) * 128 * 64 * ntiles / 1e12
    mha_tfs = mha_tflop / (us["sparse_mha"] * 1e-6)
    cpu_rec = cpu_prefill_mla(q_mla, latent, kpe, idx, scale, K) if cpu else None
    cpu_mha = cpu_prefill_mha(q192, kv, kpe, idx, pos, scale, K) if cpu else None
    return {
        "workload": "prefill T=4096 (B=1, L=4096, H_I=64, top-2048, 128 heads)",
        "cpu_sparse_mla": cpu_rec,
        "cpu_sparse_mha": cpu_mha,
        "call_us": {k: round(v, 1) for k, v in us.items()},
        "indexer": {"tflops": round(idx_tfs, 1), "flop": round(idx_tflop * 1e12),
                    "frac_bf16_mfma": round(idx_tfs / BF16_MFMA_PEAK_TFLOPS, 4),
                    "frac_fp8_mfma": round(idx_tfs / FP8_MFMA_PEAK_TFLOPS, 4),
                    "note": "FP8 codes multiplied exactly on the bf16 MFMA; the call includes "
                            "the key append and query quantisation"},
        "sparse_mla": {"tflops": round(mla_tfs, 1), "flop": round(mla_tflop * 1e12),
                       "frac_bf16_mfma": round(mla_tfs / BF16_MFMA_PEAK_TFLOPS, 4)},
        "topk": {"GBps": round(topk_bytes / (us["topk"] * 1e-6) / 1e9, 1), "bytes": topk_bytes,
                 "frac_hbm": round(topk_bytes / (us["topk"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "projections": {c: {"tflops": round(f / (us[c] * 1e-6), 1), "flop": round(f * 1e12),
                            "frac_bf16_mfma": round(f / (us[c] * 1e-6) / BF16_MFMA_PEAK_TFLOPS, 4),
                            "bytes": gemm_bytes[c],
                            "frac_hbm": round(gemm_bytes[c] / (us[c] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
                        for c, f in gemm_tflop.items()},
        "sparse_mha": {"tflops": round(mha_tfs, 1), "flop": round(mha_tflop * 1e12),
                       "frac_bf16_mfma": round(mha_tfs / BF16_MFMA_PEAK_TFLOPS, 4),
                       "executed_flop": round(mha_exec_tflop * 1e12),
                       "executed_tflops": round(mha_exec_tflop / (us["sparse_mha"] * 1e-6), 1),
                       "note": "flop counts the selected (row, position) pairs; executed_flop "
                               "every 64-position tile any of 128 rows selects"},
        "forms_us": {"absorbed (absorb_q + sparse_mla + absorb_o)":
                     round(us["absorb_q"] + us["sparse_mla"] + us["absorb_o"], 1),
                     "multi-head (kv_up + sparse_mha)": round(us["kv_up"] + us["sparse_mha"], 1)},
    }


# ----------------------------------------------------------- cpu oracle --

def cpu_prefill_mha(q192, kv, kpe, idx, pos, scale, K, stride=16):
    """The oracle's multi-head prefill attention on a stratified 1/stride of
    the query rows, with the GPU run's up-projected keys/values and
    selection, rated by the selected pairs of those rows."""
    import torch

    import oracle
    T, Hq = q192.shape[1], q192.shape[2]
    rows = torch.arange(0, T, stride, device=q192.device)
    q = q192[:, rows].float().cpu().numpy().astype(np.float64)
    kvh = kv.float().cpu().numpy().astype(np.float64)
    pe = kpe.float().cpu().numpy().astype(np.float64)
    ix = idx[:, rows].cpu().numpy()
    pp = pos[:, rows].cpu().numpy()
    pairs = int(sum(min(K, int(t) + 1) for t in rows.tolist()))
    t0 = time.perf_counter()
    oracle.sparse_mha(q, kvh, pe, ix, scale, pos=pp)
    el = time.perf_counter() - t0
    flop = 2.0 * Hq * (192 + 128) * pairs
    full = 2.0 * Hq * (192 + 128) * sum(min(K, t + 1) for t in range(T))
    return {"value": round(flop / el / 1e12, 4), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": f"{rows.numel()} of {T} query rows (every {stride}th), "
            f"{pairs} selected pairs, {el:.1f} s", "projected_full_s": round(full / (flop / el), 1)}


def cpu_prefill_mla(q_mla, latent, kpe, idx, scale, K, stride=16):
    """The oracle's sparse MLA (absorbed) on a stratified 1/stride of the
    prefill's query rows (rows 0, stride, 2 stride, ...) with the GPU run's
    inputs and selection, rated by the selected pairs of those rows."""
    import torch

    import oracle
    T = q_mla.shape[1]
    rows = torch.arange(0, T, stride, device=q_mla.device)
    q = q_mla[:, rows].float().cpu().numpy().astype(np.float64)
    lat = latent.float().cpu().numpy().astype(np.float64)
    pe = kpe.float().cpu().numpy().astype(np.float64)
    ix = idx[:, rows].cpu().numpy()
    pairs = int(sum(min(K, int(t) + 1) for t in rows.tolist()))
    t0 = time.perf_counter()
    oracle.sparse_mla(q, lat, pe, ix, scale)
    el = time.perf_counter() - t0
    flop = 2.0 * q.shape[2] * (576 + 512) * pairs
    full = 2.0 * q.shape[2] * (576 + 512) * sum(min(K, t + 1) for t in range(T))
    return {"value": round(flop / el / 1e12, 4), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": f"{rows.numel()} of {T} query rows (every {stride}th), "
            f"{pairs} selected pairs, {el:.1f} s", "projected_full_s": round(full / (flop / el), 1)}


def cpu_baseline(wl, x, seconds):
    """The oracle's decode step on the host: prepare q and the new key,
    dequantise the FP8 key cache, score, top-k, sparse MLA. The key cache is
    quantised by the oracle and the latent/rope caches widened to float64
    once, outside the timed region (the oracle's resident cache form).
    Timed over whole queries until `seconds` of work have run."""
    import oracle
    import synth
    B, L = wl.B, wl.Lmax
    cos, sin = oracle.rope_table(L, yarn=wl.yarn)
    b = 0
    n = int(wl.lengths[b])
    kpos = np.arange(n, dtype=np.int32)[None]
    k8, ks, _ = oracle.indexer_prepare(x["k_raw"][b:b + 1, :n], kpos, cos, sin, True)
    lat = synth.bf16_bits_to_f32(x["latent"][b:b + 1, :n]).astype(np.float64)
    kpe = synth.bf16_bits_to_f32(x["kpe"][b:b + 1, :n]).astype(np.float64)
    qm = synth.bf16_bits_to_f32(x["q_mla"][b:b + 1]).astype(np.float64)
    pos = x["pos"][b:b + 1]
    done = 0
    t0 = time.perf_counter()
    while True:
        q8, qs, _ = oracle.indexer_prepare(x["q_raw"][b:b + 1], pos[..., None], cos, sin, True)
        kn8, kns, _ = oracle.indexer_prepare(x["k_raw"][b:b + 1, pos[0, 0]][:, None],
                                             pos, cos, sin, True)
        k8[0, pos[0, 0]] = kn8[0, 0]
        ks[0, pos[0, 0]] = kns[0, 0]
        kd = oracle.dequantize(k8, ks)
        sc = oracle.indexer_scores(oracle.dequantize(q8, qs), x["w"][b:b + 1], kd, pos + 1)
        idx = oracle.topk(sc[0], pos[0] + 1, wl.K)[None]
        oracle.sparse_mla(qm, lat, kpe, idx, wl.softmax_scale)
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds or done >= 1000:
            break
    cores = oracle.num_threads()
    rec = dict(value=done / el, unit="queries/s", cores=cores, kind="oracle",
               sample=f"{done} single-query decode steps of {wl.name} (batch row 0, "
                      f"L={n}, H=64, top-{wl.K}, 128 heads) in {el:.1f} s",
               # threads each stage of one row can use: the oracle parallelises
               # over independent rows, or over keys for a single row's scores
               stage_threads={"prepare_q": min(64, cores), "dequantise": cores,
                              "scores": cores, "topk": 1, "sparse_mla": min(128, cores)})
    # the same steps on one core, for a few seconds
    oracle.set_num_threads(1)
    try:
        done1 = 0
        t0 = time.perf_counter()
        while True:
            q8, qs, _ = oracle.indexer_prepare(x["q_raw"][b:b + 1], pos[..., None], cos, sin, True)
            kd = oracle.dequantize(k8, ks)
            sc = oracle.indexer_scores(oracle.dequantize(q8, qs), x["w"][b:b + 1], kd, pos + 1)
            idx = oracle.topk(sc[0], pos[0] + 1, wl.K)[None]
            oracle.sparse_mla(qm, lat, kpe, idx, wl.softmax_scale)
            done1 += 1
            el1 = time.perf_counter() - t0
            if el1 >= seconds / 3 or done1 >= 100:
                break
    finally:
        oracle.set_num_threads(cores)
    rec["one_core"] = {"value": done1 / el1, "sample": f"{done1} steps in {el1:.1f} s"}
    rec["host"] = {"nproc": os.cpu_count(), "cpu_model": _cpu_model()}
    return rec


def _device_record() -> dict:
    import torch
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2 ** 30, 1)}


def _cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------------ main --

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only; --gpus {args.gpus} is not supported "
              "(batch rows would shard across GPUs with no exchange, long rows over the context "
              "with one candidate all-gather and one LSE merge)",
              file=sys.stderr)
        sys.exit(2)
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, workload=args.workload)
        return
    import torch

    import synth

    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.only_prefill:
        torch.cuda.set_device(0)
        print(json.dumps(prefill_leg()), flush=True)
        return
    wl = synth.workload(args.workload)
    torch.cuda.set_device(0)
    st = setup(wl, args.replica_bytes)
    m = measure(wl, st, args.steps, args.warmup)
    x_host = st["x"]
    K = args.steps
    ab, dom, avg_us = m["ab"], m["dom"], m["avg_us"]
    achieved = m["achieved"]
    srch = source_hash()
    traffic = load_traffic(dom, srch, wl.name)
    ms_per_step = m["ms_per_step"]
    value = m["value"]

    rec = {
        "metric": "decode queries/s (indexer+top-2048+sparse MLA) at L=16K; % HBM roofline",
        "value": round(value, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3/bf16 (fp32 accumulate)",
        "data": "synthetic (seeded N(0,1) activations and caches; no trained weights)",
        "config": {"workload": wl.name, "B": wl.B, "L": wl.Lmax, "indexer_heads": wl.H,
                   "attn_heads": wl.Hq, "topk": wl.K, "replicas": st["R"],
                   "replica_bytes": st["per_replica"],
                   "launch": "eager: three C-ABI calls per step on the stream"},
        "step_us_quantiles": m["quantiles"],
        "step_algorithmic_bytes": ab["step"],
        "step_hbm_frac": m["step_hbm_frac"],
        "call_avg_us": {k: round(v, 2) for k, v in avg_us.items()},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "bytes_per_launch": ab[dom],
                     "traffic_over_algorithmic": (round(traffic / ab[dom], 2) if traffic else None),
                     "avg_launch_us": round(avg_us[dom], 3)},
        "source_hash": srch,
        "device": _device_record(),
    }
    if not args.no_variants:
        rec["variants"] = variants_leg(wl, st)
        rec["variants"]["graph_per_step"] = {
            "us_per_step": round(m["graph_us_per_step"], 2),
            "value": round(wl.B * wl.S / (m["graph_us_per_step"] * 1e-6), 1),
            "unit": "queries/s",
            "note": "the same timed steps, each replayed as one captured HIP graph"}
    del st, m
    torch.cuda.empty_cache()
    if not args.no_others:
        rec["other_workloads"] = other_workloads_leg(args)
    if args.sweep:
        rec["sweep"] = sweep_leg(args)
    if not args.no_prefill:
        rec["prefill"] = prefill_leg(cpu=not args.no_cpu_baseline)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl, x_host, args.cpu_seconds)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
