#!/usr/bin/env python3
"""Verify-step benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config dynamic]

One step = the whole verify path over one batch: spec_tree_build_mask ->
spec_kv_append -> spec_tree_attn_verify -> spec_accept_sample (or
spec_accept_topk with --acceptance topk) -> spec_kv_commit, on synthetic
inputs already resident in HBM.  Prints one JSON line:

* value: verified tree tokens/s (all verify rows, roots included) over the
  wall clock of K steps; for working sets under 1 GiB, which caches could
  hold between steps, a 1 GiB flush runs before every step and the rate
  comes from the median GPU time of a step instead;
* per-call times from HIP events on the launch stream (medians; means
  beside them), the roofline of the dominant kernel (tree attention, from
  its average launch time) and attention + acceptance against the HBM peak;
* with the default dynamic batch, a "specinfer" object: the K-schedule
  trees on the 70B-shaped layer measured in the same run (caches flushed
  before every step, medians, attention also against its ridge floor);
* beside the step (not in its time): the fused target LM head
  (spec_lm_head_accept) on the same rows with a library GEMM plus the plain
  acceptance as context (--no-lm-head skips it);
* the CPU oracle timed on a bounded sample of the same workload on this
  host, with the BLAS thread count it ran with.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published

WORKLOAD_TEXT = {
    "toy": "toy: 6-node tree root/A/B/C/D/E, B=1, 4 heads, D=64, prefix 128, fp32, vocab 1000",
    "chain8": "chain: gamma=8 (9 rows), B=1, MHA 32x128, contiguous KV 2048, bf16, vocab 32000",
    "medusa": "medusa: 3x5x7 Cartesian tree (124 rows), B=1, MHA 32x128, KV 4096, bf16, vocab 32000",
    "specinfer": "specinfer: K-schedule (3,2,2,1,1) trees (46 rows) x B=8, GQA 64/8, D=128, "
                 "contiguous KV 8192, bf16, vocab 128256",
    "dynamic": "dynamic: EAGLE-2 top-5 trees under ECHO budget Kmax=1024 rows, B=64, "
               "paged KV (block 16) prefixes U[512,16384], GQA 32/8, D=128, bf16, vocab 128256",
    "lookahead": "lookahead: W=5 N=4 G=5 pass (30 rows, two causal branches, caller mask), B=1, "
                 "MHA 32x128, contiguous KV 2048, bf16, vocab 32000",
}


def algorithmic(w, topk=False):
    """Algorithmic bytes / flops of one step.  The acceptance figure returned
    here counts every target row once, and the draft rows of nodes with
    children unless the children are deterministic (topk): the reading of the
    statistics step in which every row's log-sum-exp is formed.  What the
    method must read is less (accept_bytes)."""
    import numpy as np
    e = 2 if w.dtype == "bf16" else 4
    words = (w.max_rows + 63) // 64
    a_attn = 0
    f_attn = 0
    a_acc = 0
    for b in range(w.B):
        o, n = int(w.row_offsets[b]), w.rows(b)
        L = int(w.prefix_len[b])
        a_attn += w.Hkv * (L + n) * w.D * 2 * e + 2 * n * w.Hq * w.D * e + n * words * 8
        if getattr(w, "visibility", None) is not None:
            seen = np.asarray(w.visibility[b], dtype=bool).sum(axis=1)   # new rows each row sees
        else:
            par = w.parents[o:o + n]
            depth = np.zeros(n, dtype=np.int64)
            for i in range(1, n):
                depth[i] = depth[par[i]] + 1
            seen = depth + 1
        f_attn += w.Hq * w.D * 4 * int(np.sum(L + seen))
        a_acc += n * w.V * 4 + (0 if topk else int(w.nonleaf[o:o + n].sum()) * w.V * 4)
    return a_attn, f_attn, a_acc


def attn_plus_accept(a_attn, a_acc, a_all, t_attn, t_acc, rows):
    """(A_attn + A_acc) / (t_attn + t_acc) against the HBM peak, with A_acc
    the bytes the acceptance must read; beside it the same with every target
    row counted (a rate, not a traffic: the rows of leaves where no walk ends
    are not read)."""
    t = t_attn + t_acc
    return {"bytes": a_attn + a_acc, "ms": t * 1e3, "tree_tokens_per_s": rows / t,
            "gbs": (a_attn + a_acc) / t / 1e9,
            "hbm_frac": (a_attn + a_acc) / t / 1e9 / HBM_PEAK_GBS,
            "accept_bytes": a_acc, "accept_gbs": a_acc / t_acc / 1e9,
            "bytes_every_target_row": a_attn + a_all,
            "hbm_frac_every_target_row": (a_attn + a_all) / t / 1e9 / HBM_PEAK_GBS}


def accept_bytes(w, topk, path, accept_len):
    """Bytes the acceptance must read: the target rows of nodes with children
    (every child probability needs its parent's log-sum-exp), their draft rows
    (sampled children), and the target row of each leaf where a walk ends
    (the bonus draw).  Target rows of the other leaves are needed by nothing:
    no child probability and no draw uses them."""
    import numpy as np
    path = path.cpu().numpy()
    alen = accept_len.cpu().numpy()
    rows = 0
    for b in range(w.B):
        o, n = int(w.row_offsets[b]), w.rows(b)
        nonleaf = int(w.nonleaf[o:o + n].sum())
        rows += nonleaf * (1 if topk else 2)
        a = int(alen[b])
        if a >= 0 and not bool(w.nonleaf[o + int(path[b, a])]):
            rows += 1
    return rows * w.V * 4


def measured_traffic(config):
    """HBM bytes per attention call from the committed counter summary.

    profiles/attn_<config>_traffic.json holds FETCH_SIZE + WRITE_SIZE of the
    attention kernels (two rocprofv3 --pmc runs, calibrated against a 1 GiB
    device copy) and the sha256 of the sources they were built from.  When
    those sources have changed since, the counters describe another kernel
    and the traffic is reported as null.
    """
    import hashlib
    path = os.path.join(ROOT, "profiles", f"attn_{config}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return rec["traffic_bytes_per_call"]


def blas_threads():
    """Threads the oracle's numpy actually runs with: the BLAS thread pools'
    own counts (threadpoolctl), else OMP_NUM_THREADS, else the affinity mask."""
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return max(n)
    except ImportError:
        pass
    threads = os.environ.get("OMP_NUM_THREADS")
    return int(threads) if threads else len(os.sched_getaffinity(0))


def cpu_baseline(w, budget_s, topk=False):
    """Time the oracle on the requests of the workload, in order (and again
    from the first request when one pass over the batch takes less than the
    budget), until about budget_s seconds of CPU time are spent."""
    import numpy as np
    import torch
    from oracle import accept as OA
    from oracle import attention as OAt
    from oracle import kv as OK
    from oracle import tree as OT
    inputs = {}

    def host_inputs(b):
        if b not in inputs:
            o, n = int(w.row_offsets[b]), w.rows(b)
            kp, vp = w.prefix_kv(b)
            f64 = lambda t: t[o:o + n].to("cpu", torch.float64).numpy()   # noqa: E731
            inputs[b] = (kp, vp, f64(w.q), f64(w.k_new), f64(w.v_new), f64(w.p_logits),
                         f64(w.q_logits))
        return inputs[b]

    rows = 0
    spent = 0.0
    done = 0
    while spent < budget_s:
        b = done % w.B
        o, n = int(w.row_offsets[b]), w.rows(b)
        L = int(w.prefix_len[b])
        kp, vp, q, kt, vt, pl, ql = host_inputs(b)      # inputs to host first (not timed)
        par = w.parents[o:o + n]
        t0 = time.perf_counter()
        OT.pack_words(OT.ancestor_mask(par), (w.max_rows + 63) // 64)
        OAt.tree_attention(q, kp, vp, kt, vt, par, scale=1.0 / np.sqrt(w.D))
        if topk:
            r = OA.accept_request_topk(par, w.tokens[o:o + n], pl, w.temperature, w.seed,
                                       w.step, b)
        else:
            r = OA.accept_request(par, w.tokens[o:o + n], pl, ql, w.temperature, w.seed,
                                  w.step, b)
        for h in range(w.Hkv):
            OK.commit(np.concatenate([kp[h], kt[:, h]]), L, r["path"])
            OK.commit(np.concatenate([vp[h], vt[:, h]]), L, r["path"])
        spent += time.perf_counter() - t0
        rows += n
        done += 1
    return {"value": rows / spent, "unit": "tree tokens/s", "cores": blas_threads(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS"), "kind": "oracle",
            "sample": f"{done} request-steps ({rows} verify rows; requests taken in order, "
                      f"cycling over the batch of {w.B}) of the same workload: mask + attention "
                      f"(all heads, one layer) + acceptance + commit, numpy fp64; "
                      f"{spent:.1f} s of CPU time"}


class TreeBuilder:
    """The dynamic workload's trees built on the device: B requests, top-5
    expansion for 8 rounds (depth <= 8), checkpoints at depths 3 and 6, a
    budget of 1024 rows, at most 64 rows per request.  Drafter candidates are
    synthetic (workloads.drafts) and resident on the device; each run ends by
    copying the B + 1 row offsets to the host, as a caller must to plan the
    verify calls."""

    def __init__(self, w_batch, K=5, rounds=8, capacity=256, budget=1024, max_rows=64,
                 gates=((3, 0.02), (6, 0.002))):
        import torch
        import workloads as W
        from tree_attention_verification_02_amd import _lib as L
        self.L, self.B, self.budget, self.max_rows, self.gates = L, w_batch, budget, max_rows, gates
        self.toks, self.probs = W.drafts.candidates(rounds, w_batch, K, 128256, seed=0,
                                                    device="cuda")
        self.tree = L.DraftTree(w_batch, K, capacity, "cuda")
        self.roots = torch.arange(w_batch, dtype=torch.int32, device="cuda")
        cap = min(budget, w_batch * max_rows)
        self.ro = torch.empty(w_batch + 1, dtype=torch.int32, device="cuda")
        self.par = torch.empty(cap, dtype=torch.int32, device="cuda")
        self.tok = torch.empty(cap, dtype=torch.int32, device="cuda")
        self.ws = torch.empty(L.spec_draft_select_workspace_bytes(w_batch, max_rows),
                              dtype=torch.uint8, device="cuda")
        self.ro_h = torch.empty(w_batch + 1, dtype=torch.int32, pin_memory=True)

    def run(self, sync=True):
        L = self.L
        L.spec_draft_begin(self.tree, self.roots)
        for r in range(self.toks.shape[0]):
            L.spec_draft_expand(self.tree, self.toks[r], self.probs[r], self.gates)
        L.spec_draft_select(self.tree, self.budget, self.max_rows, self.ro, self.par, self.tok,
                            self.ws)
        self.ro_h.copy_(self.ro, non_blocking=True)
        if sync:
            import torch
            torch.cuda.current_stream().synchronize()
        return self.ro_h.numpy()

    def host_tree(self):
        ro = self.run().copy()
        return ro, self.par[:ro[-1]].cpu().numpy(), self.tok[:ro[-1]].cpu().numpy()


FLUSH_BELOW_BYTES = 1 << 30      # flush caches between steps for working sets below this


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def make_flush(nbytes=1 << 30):
    """A device write of 1 GiB: evicts the L2s and the 256 MB Infinity Cache."""
    import torch
    buf = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    return lambda: buf.fill_(1.0)


def time_steps(calls, steps, flush=None):
    """Run `steps` steps of `calls` with a HIP event between consecutive calls
    (all on the stream the library launches on); returns (wall seconds of
    the whole loop, per-step lists of per-call milliseconds)."""
    import torch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        if flush is not None:
            flush()
        ev[s][0].record()
        for i, fn in enumerate(calls):
            fn()
            ev[s][i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [[ev[s][i].elapsed_time(ev[s][i + 1]) for i in range(len(calls))]
                  for s in range(steps)]


def measure_config(name, acceptance, steps, warmup=5):
    """A second target workload measured in the same run: every call timed
    with HIP events, caches flushed before every step (outside the timed
    calls), medians.  Attention is reported against both HBM and the
    ridge-bound floor max(bytes / 8 TB/s, flops / 2.5 PFLOP/s)."""
    import torch
    import workloads as W
    from tree_attention_verification_02_amd.pipeline import VerifyStep
    topk = acceptance == "topk"
    w = W.make(name, device="cuda", **({"draft": "topk"} if topk else {}))
    vs = VerifyStep(w, acceptance=acceptance)
    a_attn, f_attn, a_acc = algorithmic(w, topk)
    names = ["mask", "append", "attention", "accept", "commit"]
    calls = [vs.build_mask, vs.append, vs.attention, vs.accept, vs.commit]
    flush = make_flush()
    for _ in range(warmup):
        for fn in calls:
            fn()
    _, steps_ms = time_steps(calls, steps, flush)
    per = {n: median([st[i] for st in steps_ms]) for i, n in enumerate(names)}
    t_attn, t_acc = per["attention"] * 1e-3, per["accept"] * 1e-3
    a_all = a_acc
    a_acc = accept_bytes(w, topk, vs.acc.path, vs.acc.accept_len)
    floor = max(a_attn / (HBM_PEAK_GBS * 1e9), f_attn / (BF16_PEAK_TFLOPS * 1e12))
    out = {"workload": WORKLOAD_TEXT[name], "batch": w.B, "verify_rows": w.R, "steps": steps,
           "timing": "HIP events per call, caches flushed before every step, medians",
           "per_call_ms": per,
           "attention": {"algorithmic_bytes": a_attn, "flops": f_attn,
                         "gbs": a_attn / t_attn / 1e9, "hbm_frac": a_attn / t_attn / 1e9 / HBM_PEAK_GBS,
                         "tflops": f_attn / t_attn / 1e12,
                         "mfma_frac": f_attn / t_attn / 1e12 / BF16_PEAK_TFLOPS,
                         "ridge_floor_ms": floor * 1e3, "frac_of_ridge_floor": floor / t_attn},
           "attn_plus_accept": attn_plus_accept(a_attn, a_acc, a_all, t_attn, t_acc, w.R),
           "step_gpu_ms": median([sum(st) for st in steps_ms]),
           "mean_accepted_drafts": float(vs.acc.accept_len.float().mean())}
    del vs, w
    torch.cuda.empty_cache()
    return out


def measure_lm_head(w, acceptance, accept_ms, reps=15):
    """The fused target LM head (spec_lm_head_accept) on the same workload:
    hidden states [R][Hq*D] and a [V][Hq*D] head, bf16.  Reported beside the
    step, with a library GEMM (torch.mm, hipBLASLt, fp32 output) followed by
    the plain acceptance as context."""
    import torch
    import workloads as W
    from tree_attention_verification_02_amd.pipeline import VerifyStep
    hidden, weight = W.heads.head_inputs(w)
    H = int(hidden.shape[1])
    flops = 2.0 * w.R * H * w.V

    def med(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ts.sort()
        return ts[len(ts) // 2]

    hs = VerifyStep(w, acceptance=acceptance, head=(hidden, weight))
    t_head = med(hs.accept)
    hg = VerifyStep(w, acceptance=acceptance, temperature=0.0, head=(hidden, weight))
    t_greedy = med(hg.accept)
    try:
        t_lib = med(lambda: torch.mm(hidden, weight.t(), out_dtype=torch.float32))
        lib_kind = "torch.mm bf16 -> fp32 (hipBLASLt)"
    except (RuntimeError, TypeError):
        t_lib = med(lambda: torch.mm(hidden, weight.t()).float())
        lib_kind = "torch.mm bf16 -> bf16, then to fp32"
    mean_acc = float(hs.acc.accept_len.float().mean())
    del hs, hg, hidden, weight
    torch.cuda.empty_cache()
    return {"call": "spec_lm_head_accept (head GEMM with the acceptance statistics in its "
                    "epilogue, then the walk)",
            "hidden": H, "flops": flops, "temperature": float(w.temperature),
            "ms": t_head, "ms_greedy": t_greedy,
            "tflops_greedy": flops / (t_greedy * 1e-3) / 1e12,
            "mfma_frac_greedy": flops / (t_greedy * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "library_gemm": lib_kind, "library_gemm_ms": t_lib,
            "library_gemm_plus_accept_ms": t_lib + accept_ms,
            "mean_accepted_drafts": mean_acc}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="dynamic", choices=list(WORKLOAD_TEXT))
    ap.add_argument("--acceptance", default="sample", choices=["sample", "topk"],
                    help="children drawn from the draft rows (spec_accept_sample) or the "
                         "drafter's top-k tokens (spec_accept_topk)")
    ap.add_argument("--tree-builder", action="store_true",
                    help="dynamic config only: build the trees on the device each step "
                         "(spec_draft_begin, 8 rounds of spec_draft_expand, spec_draft_select, "
                         "row offsets back to the host) before the verify calls")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-copy-probe", action="store_true",
                    help="skip the device-copy bandwidth probe printed as context")
    ap.add_argument("--no-lm-head", action="store_true",
                    help="skip the fused target LM head measurement (spec_lm_head_accept)")
    ap.add_argument("--no-specinfer", action="store_true",
                    help="skip the second target workload (K-schedule trees, 70B-shaped layer) "
                         "measured beside the dynamic batch")
    ap.add_argument("--calib-copy-gib", type=float, default=0.0,
                    help="also run one device copy of this many GiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              f"(requests are independent, see the sharding notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    from tree_attention_verification_02_amd.pipeline import VerifyStep

    topk = args.acceptance == "topk"
    builder = None
    over = {"draft": "topk"} if topk else {}
    if args.tree_builder:
        if args.config != "dynamic":
            print("bench.py: --tree-builder applies to --config dynamic", file=sys.stderr)
            sys.exit(2)
        builder = TreeBuilder(w_batch=W.CONFIGS["dynamic"]["B"])
        ro, par, tok = builder.host_tree()
        # same prefix lengths as the generated dynamic workload, so the verify
        # calls do the same attention work
        over.update(tree=("given", [par[ro[b]:ro[b + 1]] for b in range(builder.B)]),
                    given_tokens=tok, L=W.gen.prefix_lengths("dynamic"))
    w = W.make(args.config, device="cuda", **over)
    vs = VerifyStep(w, acceptance=args.acceptance)
    a_attn, f_attn, a_acc = algorithmic(w, topk)
    names = ["mask", "append", "attention", "accept", "commit"]
    calls = [vs.build_mask, vs.append, vs.attention, vs.accept, vs.commit]
    if builder is not None:
        names = ["draft_build"] + names
        calls = [builder.run] + calls
    # Working sets that an L2 + Infinity Cache (256 MB) could hold between
    # steps are measured with a cache flush before every step, outside the
    # timed calls; the headline dynamic batch (~3 GB) needs none.
    flush = make_flush() if a_attn + a_acc < FLUSH_BELOW_BYTES else None
    for _ in range(args.warmup):
        for fn in calls:
            fn()
    torch.cuda.synchronize()
    wall, steps_ms = time_steps(calls, args.steps, flush)
    per = {n: median([st[i] for st in steps_ms]) for i, n in enumerate(names)}   # ms per call
    per_mean = {n: sum(st[i] for st in steps_ms) / len(steps_ms) for i, n in enumerate(names)}
    gpu_ms = median([sum(st) for st in steps_ms])
    if flush is not None:
        # the wall clock would include the flushes: rate from the GPU time
        value = w.R / (gpu_ms * 1e-3)
        value_basis = "median GPU time of one step (caches flushed before every step)"
    else:
        value = w.R * args.steps / wall
        value_basis = "wall clock of the timed steps"

    # context: a plain device copy (read + write) on the same GPU
    copy_gbs = None
    if not args.no_copy_probe:
        n = (1 << 30) // 4
        src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        copy_gbs = 5 * 2 * n * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del src, dst

    if args.calib_copy_gib > 0:
        n = int(args.calib_copy_gib * (1 << 30)) // 4
        src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    R = w.R
    ms_step = wall / args.steps * 1e3 if flush is None else gpu_ms
    t_attn = per["attention"] * 1e-3
    t_acc = per["accept"] * 1e-3
    # the roofline uses the average launch duration (what a rocprofv3 kernel
    # trace of the same command reports); everything else uses medians
    achieved = a_attn / (per_mean["attention"] * 1e-3) / 1e9
    out = {
        "metric": "verified tree tokens/s (1 GPU); achieved HBM GB/s as % of peak",
        "value": value,
        "unit": "tree tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.config], "name": args.config,
                   "batch": w.B, "verify_rows": R, "draft_tokens": R - w.B,
                   "kv_tokens": int(w.prefix_len.sum()) + R, "vocab": w.V,
                   "acceptance": args.acceptance, "tree_builder": bool(args.tree_builder),
                   "value_basis": value_basis},
        "roofline": {"bound": "hbm", "kernel": "spec_tree_attn_verify (split-KV main + combine)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(args.config),
                     "traffic_unit": "HBM bytes per call (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated)",
                     "algorithmic_bytes": a_attn, "avg_launch_ms": per_mean["attention"],
                     "median_launch_ms": per["attention"],
                     "mfma_tflops": f_attn / t_attn / 1e12,
                     "mfma_frac": f_attn / t_attn / 1e12 / BF16_PEAK_TFLOPS},
        "attn_plus_accept": attn_plus_accept(a_attn, accept_bytes(w, topk, vs.acc.path,
                                                                   vs.acc.accept_len),
                                             a_acc, t_attn, t_acc, R),
        "per_call_ms": per,
        "per_call_ms_mean": per_mean,
        "timing": "HIP events on the launch stream around every call; per-call figures are "
                  "medians over the timed steps",
        "stream_copy_gbs": copy_gbs,
        "gpu_ms_per_step": gpu_ms,
        "mean_accepted_drafts": float(vs.acc.accept_len.float().mean()),
    }
    if not args.no_lm_head and builder is None:
        out["lm_head"] = measure_lm_head(w, args.acceptance, per["accept"])
    if args.config == "dynamic" and builder is None and not args.no_specinfer:
        del vs
        torch.cuda.empty_cache()
        out["specinfer"] = measure_config("specinfer", args.acceptance, max(args.steps, 20))
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, topk)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
