"""Benchmark of the DSA decode hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one pass of the whole path over one batch: lightning indexer -> causal top-k ->
sparse MLA (plus the split-KV merge), on the decode workload of 32 sequences with 16384-token
contexts, one new query each (indexer 32 heads x 128, top-k 2048, 64-head MQA over 576-wide
bf16 latent rows). Inputs are seeded synthetic tensors resident in HBM before timing starts.
Steps rotate over independent input sets: between two uses of one set the others touch at
least 1 GiB (four times the 256 MB Infinity Cache), so a step is not served from cached lines.

The timed steps launch their four kernels back to back on one stream; --launch graph replays
one captured HIP graph per input set instead (slower here). Prints one JSON line: metric, value
(query tokens/s), per-call times from HIP events on the launch stream around every call of a
second timed pass of the same steps, the roofline of the dominant call (its average launch
duration from K launches back to back between two events, which the rocprofv3 kernel durations
match), and the CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0        # MI355X dense fp8 MFMA
BF16_PEAK_TFLOPS = 2516.6       # MI355X dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_b32_l16k")
    ap.add_argument("--select", choices=["token", "block"], default="token",
                    help="per-position top-k (default) or block-pooled selection of "
                         "index_topk / block-size blocks")
    ap.add_argument("--block-size", type=int, default=64)
    ap.add_argument("--pool", choices=["max", "mean"], default="max")
    ap.add_argument("--index-dtype", choices=["bf16", "fp8"], default="bf16",
                    help="element type of the indexer inputs q_I / k_I (fp8: OCP e4m3fn; the "
                         "attention stays bf16)")
    ap.add_argument("--sets", type=int, default=0, help="input sets rotated (0: enough to exceed 1 GiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--launch", choices=["eager", "graph"], default="eager",
                    help="headline: one dsa_forward call per layer (default) or replayed from "
                         "one HIP graph per input set; the other mode is timed too")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph timing")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def _key_rows(case):
    """Key rows the indexer must read: per sequence, the rows its last new query sees (the
    new queries of one sequence share them)."""
    import dsa_inputs as DI
    last = {}
    for t, b, p, base in DI.query_rows(case):
        last[b] = max(last.get(b, 0), p + 1)
    return sum(last.values())


def step_bytes(case, ib=2, ab=2):
    """Algorithmic HBM bytes of one step: the key rows of the indexer cache (each once per
    sequence), the selected latent rows of every query, queries, outputs, indexer queries and
    weights (intermediates excluded); ib = bytes per indexer element (2 for bf16, 1 for fp8,
    4 for fp32), ab = bytes per attention element (2 for bf16, 4 for fp32)."""
    import dsa_inputs as DI
    tot = _key_rows(case) * case.index_head_dim * ib                        # k_I rows
    for t, b, p, base in DI.query_rows(case):
        n = p + 1
        tot += min(case.index_topk, n) * case.d_qk * ab * case.layers       # gathered rows
        tot += case.n_heads * (case.d_qk + case.d_v) * ab * case.layers     # q in, out
        tot += case.index_n_heads * (case.index_head_dim * ib + 4)          # q_I, w
    return tot


def indexer_bytes(case, ib=2):
    return (_key_rows(case) * case.index_head_dim * ib
            + case.total_q * case.index_n_heads * (case.index_head_dim * ib + 4))


def mla_bytes(case, ab=2):
    import dsa_inputs as DI
    tot = 0
    for t, b, p, base in DI.query_rows(case):
        tot += (min(case.index_topk, p + 1) * case.d_qk * ab
                + case.n_heads * (case.d_qk + case.d_v) * ab)
    return tot


def indexer_flops(case):
    """Multiply-adds of the causal score grid, counted as two FLOPs each."""
    import dsa_inputs as DI
    return sum(2 * case.index_n_heads * case.index_head_dim * (p + 1)
               for (_, _, p, _) in DI.query_rows(case))


def mla_flops(case):
    """QK^T over d_qk and P.V over d_v for every head and selected row of one layer."""
    import dsa_inputs as DI
    return sum(2 * case.n_heads * (case.d_qk + case.d_v) * min(case.index_topk, p + 1)
               for (_, _, p, _) in DI.query_rows(case))


def code_digest(path):
    """SHA-256 of a kernel source with // comments, trailing blanks and empty lines removed: a
    change of comments alone does not change the kernel the counters measured."""
    import hashlib
    import re
    lines = []
    for ln in open(path, encoding="utf-8"):
        ln = re.sub(r"//.*$", "", ln.rstrip("\n")).rstrip()
        if ln:
            lines.append(ln)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def traffic_record(workload, kernel):
    """HBM bytes per launch of `kernel` measured by rocprofv3 FETCH_SIZE / WRITE_SIZE runs,
    from the committed summary profiles/<workload>_hbm_traffic.md; None when the summary is
    missing or any kernel source's code changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    rec = None
    for ln in open(path):
        if ln.strip().startswith("traffic-record:"):
            rec = json.loads(ln.strip()[len("traffic-record:"):])
    if rec is None:
        return None
    csrc = os.path.join(ROOT, "long_context_lightning_amd", "csrc")
    shas = rec.get("code_sha256")
    # every kernel source of the tree, and only those, with the digests the counters were taken at
    if not shas or set(shas) != set(os.listdir(csrc)):
        return None
    for name, sha in shas.items():
        if code_digest(os.path.join(csrc, name)) != sha:
            return None
    key = "traffic_bytes_per_launch" if kernel == rec["kernel"] else f"{kernel}_traffic_bytes_per_launch"
    return rec.get(key)


def cpu_baseline(case, sets, budget_s):
    """The oracle as it stands, timed per query over the whole step: indexer over the query's
    visible keys, top-k, and sparse attention for every layer of the index pass. Up to 32
    queries of the workload are cycled (all of them for the long-context workloads). Host
    copies of each query's inputs, and of the latent rows its selection gathers, are made
    before the timing."""
    import torch
    import dsa_inputs as DI
    import oracle.dsa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1

    rows = DI.query_rows(case)
    d = sets[0]
    f = lambda x: x.detach().float().cpu().numpy()
    host = []
    for t, b, p, base in rows[:32]:
        qI, kI, w = f(d["q_idx"][t]), f(d["k_idx"][base:base + p + 1]), f(d["w"][t])
        sel = O.topk_row(O.indexer_scores_row(qI, kI, w), case.index_topk)
        rows_dev = base + torch.as_tensor(sel[sel >= 0], device=d["kv"][0].device)
        layers = [(f(d["q"][l][t]), f(d["kv"][l][rows_dev])) for l in range(case.layers)]
        host.append((qI, kI, w, layers))
    done, spent = 0, 0.0
    stage = [0.0, 0.0, 0.0]
    while spent < budget_s and done < 100000:
        qI, kI, w, layers = host[done % len(host)]
        t0 = time.perf_counter()
        s = O.indexer_scores_row(qI, kI, w)
        t1 = time.perf_counter()
        O.topk_row(s, case.index_topk)
        t2 = time.perf_counter()
        for q, kv_sel in layers:
            O.sparse_attention_row(q, kv_sel, case.d_v, case.softmax_scale)
        t3 = time.perf_counter()
        stage = [stage[0] + t1 - t0, stage[1] + t2 - t1, stage[2] + t3 - t2]
        spent += t3 - t0
        done += 1
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    lens = sorted({p + 1 for (_, _, p, _) in rows[:len(host)]})
    ctx = f"{lens[0]}" if len(lens) == 1 else f"{lens[0]}..{lens[-1]}"
    return {"value": done / spent, "unit": "query-tokens/s", "cores": int(threads),
            "kind": "oracle", "cpu": model, "affinity_cpus": len(os.sched_getaffinity(0)),
            "stage_seconds": {"indexer": round(stage[0], 3), "topk": round(stage[1], 3),
                              "attention": round(stage[2], 3)},
            "sample": f"{done} query steps of the same workload ({len(host)} distinct queries "
                      f"cycled, contexts {ctx}): indexer over every visible key, "
                      f"top-{case.index_topk}, {case.n_heads}-head sparse attention for each of "
                      f"{case.layers} layer(s); float64 NumPy, {spent:.1f} s of oracle time"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: libdsa runs the DSA path on one GPU; --gpus {args.gpus} is not "
              "supported (sharding decode by sequence over several GPUs is not implemented)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import dsa_inputs as DI
    import long_context_lightning_amd as dsa

    torch.cuda.set_device(0)
    case = DI.CASES[args.workload]
    # A step touches step_bytes(case) of its input set (the whole indexer key cache, only the
    # selected latent rows). Between two uses of one set the other sets touch at least 1 GiB,
    # four times the Infinity Cache, so no step is served from an earlier step's cached lines.
    fp8 = args.index_dtype == "fp8"
    f32 = case.dtype == torch.float32
    if fp8 and f32:
        sys.exit("bench.py: the fp8 indexer runs on the bf16 path; this workload is fp32")
    dt = 0 if f32 else 1                     # dsa_dtype of q, kv, out (and q_I, k_I unless fp8)
    ab = 4 if f32 else 2                     # bytes per attention element
    eb = 1 if fp8 else ab                    # bytes per indexer element
    touched = step_bytes(case, eb, ab)
    nsets = args.sets or max(2, 1 + math.ceil((1 << 30) / touched))
    sets = []
    for i in range(nsets):
        c = DI.Case(**{**case.__dict__, "seed_base": case.seed_base + 100 * i})
        d = DI.make_inputs(c, "cuda")
        if fp8:        # integer-valued indexer inputs are exact in e4m3fn
            for key in ("q_idx", "k_idx"):
                v = d[key].to(torch.float8_e4m3fn)
                assert torch.equal(v.float(), d[key].float())
                d[key] = v
        sets.append(d)
    d0 = sets[0]
    batch = dsa.Batch(d0["cu_seqlens_q"], d0["cu_seqlens_k"], max(case.seqlens_q),
                      max(case.seqlens_k), case.total_q, case.total_k)
    T = case.total_q
    ld = batch.max_seqlen_k
    scores = torch.empty((T, ld), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, case.index_topk), dtype=torch.int32, device="cuda")
    outs = [torch.empty((T, case.n_heads, case.d_v), dtype=case.dtype, device="cuda")
            for _ in range(case.layers)]
    lse = torch.empty((T, case.n_heads), dtype=torch.float32, device="cuda")
    ws_n = dsa.workspace_size(dsa.OP_SPARSE_MLA, batch, case.index_topk, case.n_heads, case.d_v)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")
    tws_n = dsa.workspace_size(dsa.OP_TOPK, batch, case.index_topk)
    tws = torch.empty(max(tws_n, 1), dtype=torch.uint8, device="cuda")
    blk = args.select == "block"
    pool_code = 1 if args.pool == "mean" else 0
    if blk:
        tws_n = int(dsa.lib().dsa_block_topk_workspace_size(batch.ptr, args.block_size))
        tws = torch.empty(max(tws_n, 1), dtype=torch.uint8, device="cuda")
    fws_n = dsa.workspace_size(dsa.OP_FORWARD, batch, case.index_topk, case.n_heads, case.d_v)
    fws = torch.empty(max(fws_n, 1), dtype=torch.uint8, device="cuda")
    L = dsa.lib()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    # arguments of the fused call, per input set and layer (built once, outside the timing)
    fargs = [[dsa._CForwardArgs(d["q_idx"].data_ptr(), d["k_idx"].data_ptr(), d["w"].data_ptr(),
                                case.index_n_heads, case.index_head_dim, case.index_topk,
                                d["q"][l].data_ptr(), d["kv"][l].data_ptr(), case.n_heads,
                                case.d_qk, case.d_v, case.softmax_scale, dt, 1 if fp8 else 0,
                                None, args.block_size if blk else 0, pool_code)
              for l in range(case.layers)] for d in sets]

    def fused_on(i, sp):
        # one dsa_forward per layer: the first runs indexer + top-k into the shared indices,
        # the other layers of the IndexShare group reuse them
        st = 0
        for l in range(case.layers):
            st |= L.dsa_forward(batch.ptr, ctypes.byref(fargs[i % nsets][l]), idx.data_ptr(),
                                1 if l == 0 else 0, outs[l].data_ptr(), lse.data_ptr(),
                                fws.data_ptr(), fws.numel(), sp)
        if st:
            raise RuntimeError(f"libdsa call failed with status {st}")

    def idx_on(d, sp):
        if fp8:
            return L.dsa_indexer_scores_fp8(batch.ptr, d["q_idx"].data_ptr(), d["k_idx"].data_ptr(),
                                            None, d["w"].data_ptr(), case.index_n_heads,
                                            case.index_head_dim, scores.data_ptr(), ld, sp)
        return L.dsa_indexer_scores(batch.ptr, d["q_idx"].data_ptr(), d["k_idx"].data_ptr(),
                                    d["w"].data_ptr(), case.index_n_heads, case.index_head_dim,
                                    dt, scores.data_ptr(), ld, sp)

    def step(i, ev=None):
        step_on(i, sp, ev)

    def step_on(i, sp, ev=None):
        d = sets[i % nsets]
        if ev is not None:
            ev[0].record(stream)
        st = idx_on(d, sp)
        if ev is not None:
            ev[1].record(stream)
        if blk:
            st |= L.dsa_block_topk(batch.ptr, scores.data_ptr(), ld, args.block_size, pool_code,
                                   case.index_topk // args.block_size, idx.data_ptr(),
                                   tws.data_ptr(), tws.numel(), sp)
        else:
            st |= L.dsa_topk(batch.ptr, scores.data_ptr(), ld, case.index_topk, idx.data_ptr(),
                             tws.data_ptr(), tws.numel(), sp)
        if ev is not None:
            ev[2].record(stream)
        for l in range(case.layers):       # IndexShare: the group's layers reuse the indices
            st |= L.dsa_sparse_mla_fwd(batch.ptr, d["q"][l].data_ptr(), d["kv"][l].data_ptr(),
                                       idx.data_ptr(), case.index_topk, case.n_heads, case.d_qk,
                                       case.d_v, case.softmax_scale, dt, outs[l].data_ptr(),
                                       lse.data_ptr(), ws.data_ptr(), ws.numel(), sp)
        if ev is not None:
            ev[3].record(stream)
        if st:
            raise RuntimeError(f"libdsa call failed with status {st}")

    def unshared_on(i, sp):
        # the same layers with IndexShare off: every layer runs its own indexer + top-k pass (on
        # the same indexer inputs, so the selection and outputs are unchanged)
        st = 0
        for l in range(case.layers):
            st |= L.dsa_forward(batch.ptr, ctypes.byref(fargs[i % nsets][l]), idx.data_ptr(),
                                1, outs[l].data_ptr(), lse.data_ptr(), fws.data_ptr(),
                                fws.numel(), sp)
        if st:
            raise RuntimeError(f"libdsa call failed with status {st}")

    fused_on(0, sp)                  # first launches (code objects load) outside any capture
    step(0)
    torch.cuda.synchronize()
    # HIP graphs: one per input set holds the step's kernels (same kernels, same arguments);
    # captured before the warm-up, so no host-side pause separates the warm-up from the timing
    graphs = []
    if args.launch == "graph" or not args.no_graph:
        for i in range(nsets):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fused_on(i, torch.cuda.current_stream().cuda_stream)
            graphs.append(g)
    # W untimed steps of every launch form timed below
    for i in range(args.warmup):
        fused_on(i, sp)
        step(i)
        if case.layers > 1:
            unshared_on(i, sp)
        if graphs:
            graphs[i % nsets].replay()
    torch.cuda.synchronize()

    def time_steps(mode):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            if mode == "graph":
                graphs[(args.warmup + i) % nsets].replay()
            elif mode == "fused":
                fused_on(args.warmup + i, sp)
            elif mode == "unshared":
                unshared_on(args.warmup + i, sp)
            else:
                step(args.warmup + i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps

    # timed region 1: the headline, K whole steps through the fused call (one dsa_forward per
    # layer), then the same K steps as three separate calls and as graph replays
    ms_eager = time_steps("fused")
    ms_separate = time_steps("separate")
    ms_graph = time_steps("graph") if graphs else None
    index_share = None
    if case.layers > 1:
        ms_unshared = time_steps("unshared")
        index_share = {"layers_per_index_pass": case.layers,
                       "shared_ms_per_step": round(ms_eager, 5),
                       "unshared_ms_per_step": round(ms_unshared, 5),
                       "speedup": round(ms_unshared / ms_eager, 3),
                       "what": "same step with every layer running its own indexer + top-k"}
    ms_step = ms_graph if args.launch == "graph" else ms_eager
    graph_info = None
    if graphs:
        # a replay must reproduce the eager step bit for bit (same kernels, same inputs)
        fused_on(0, sp)
        torch.cuda.synchronize()
        ref = [o.clone() for o in outs] + [idx.clone()]
        graphs[0].replay()
        torch.cuda.synchronize()
        same = all(torch.equal(a, b) for a, b in zip(ref, list(outs) + [idx]))
        graph_info = {"ms_per_step": round(ms_graph, 5), "value": round(T / (ms_graph * 1e-3), 1),
                      "replay_matches_eager": bool(same)}

    # timed region 2: the same K steps launched kernel by kernel, with HIP events on the launch
    # stream around every call (per-kernel durations and the roofline)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    ms_idx = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    ms_topk = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    ms_mla = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps
    per_step = sorted(e[0].elapsed_time(e[3]) for e in evs)
    ms_gpu = sum(per_step) / args.steps
    pct = lambda q: per_step[min(len(per_step) - 1, int(q * len(per_step)))]

    # timed region 3: each call's average launch duration, K launches back to back between two
    # events on the launch stream (region 2's events between the calls add their own gaps)
    def time_calls(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        st = 0
        for i in range(args.steps):
            st |= fn(args.warmup + i)
        e1.record(stream)
        torch.cuda.synchronize()
        if st:
            raise RuntimeError(f"libdsa call failed with status {st}")
        return e0.elapsed_time(e1) / args.steps

    def idx_call(i):
        return idx_on(sets[i % nsets], sp)

    def mla_call(i):
        d, l = sets[i % nsets], i % case.layers
        return L.dsa_sparse_mla_fwd(batch.ptr, d["q"][l].data_ptr(), d["kv"][l].data_ptr(),
                                    idx.data_ptr(), case.index_topk, case.n_heads, case.d_qk,
                                    case.d_v, case.softmax_scale, dt, outs[l].data_ptr(),
                                    lse.data_ptr(), ws.data_ptr(), ws.numel(), sp)

    launch_ms = {"indexer": time_calls(idx_call), "sparse_mla": time_calls(mla_call)}

    if args.calib_copy_mib:
        a = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    sb = step_bytes(case, eb, ab)
    ib, mb = indexer_bytes(case, eb), mla_bytes(case, ab)      # one call = one layer
    kern = {"indexer": (launch_ms["indexer"], ib), "sparse_mla": (launch_ms["sparse_mla"], mb)}
    dom = max(kern, key=lambda k: kern[k][0])
    dms, dbytes = kern[dom]
    # the profile whose traffic record applies: workload, indexer dtype, selection kind
    prof = (args.workload + ("_fp8" if fp8 else "")
            + (f"_block{args.block_size}_{args.pool}" if blk else ""))
    # the bound of the dominant call from its arithmetic intensity against the ridge point:
    # prefill's indexer (many queries per key row) is matrix-core bound, a few queries per
    # sequence (decode, MTP) leave both calls memory bound
    dflops = indexer_flops(case) if dom == "indexer" else mla_flops(case)
    mpeak = FP8_PEAK_TFLOPS if (dom == "indexer" and fp8) else BF16_PEAK_TFLOPS
    if case.dtype == torch.bfloat16 and dflops / dbytes > mpeak * 1e3 / HBM_PEAK_GBPS:
        achieved = dflops / (dms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                "peak": mpeak, "unit": "TFLOP/s",
                "frac": round(achieved / mpeak, 4),
                "traffic": traffic_record(prof, dom), "traffic_unit": "B/launch",
                "algorithmic_flops_per_launch": dflops, "avg_launch_ms": round(dms, 5)}
    else:
        achieved = dbytes / (dms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic_record(prof, dom), "traffic_unit": "B/launch",
                "algorithmic_bytes_per_launch": dbytes,
                "avg_launch_ms": round(dms, 5)}
    line = {
        "metric": "DSA decode query-tokens/s + achieved HBM GB/s (indexer+top-k+sparse MLA)",
        "value": round(T / (ms_step * 1e-3), 1),
        "unit": "query-tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("bf16+fp8" if fp8 else "bf16") if case.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": f"{case.name}: {case.batch} sequences, contexts "
                               f"{min(case.seqlens_k)}..{max(case.seqlens_k)}, "
                               f"{case.total_q} query tokens, indexer {case.index_n_heads}x"
                               f"{case.index_head_dim}, top-{case.index_topk}, "
                               f"{case.n_heads}-head MQA over {case.d_qk}-wide latent "
                               f"({case.d_v} value), {case.layers} layer(s) per index pass",
                   "batch": case.batch, "query_tokens": T, "input_sets_rotated": nsets,
                   "indexer_inputs": "fp8 e4m3fn" if fp8 else case.dtype.__str__()[6:],
                   "selection": (f"block-pooled ({args.pool}): top-{case.index_topk // args.block_size}"
                                 f" blocks of {args.block_size}") if blk else
                                f"per-position top-{case.index_topk}",
                   "launch": "hip_graph" if args.launch == "graph" else "eager"},
        "eager_ms_per_step": round(ms_eager, 5),
        "separate_calls_ms_per_step": round(ms_separate, 5),
        "graph": graph_info,
        "index_share": index_share,
        "achieved_hbm_gbps": round(sb / (ms_step * 1e-3) / 1e9, 1),
        "algorithmic_bytes_per_step": sb,
        "kernel_ms": {"indexer": round(ms_idx, 5), "topk": round(ms_topk, 5),
                      "sparse_mla_incl_merge": round(ms_mla, 5), "gpu_step": round(ms_gpu, 5),
                      "timing": "events between the calls of every step",
                      "gpu_step_p10_p50_p90": [round(pct(0.1), 5), round(pct(0.5), 5),
                                               round(pct(0.9), 5)]},
        "launch_ms_back_to_back": {k: round(v, 5) for k, v in launch_ms.items()},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, sets, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
