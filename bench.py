"""Benchmark of the tree-verify hot path on one MI355X.

One step = one verification pass over one batch: tv_build_mask, tv_attention
(one attention layer) and tv_accept (greedy, or stochastic for the MTP chain
workload). Inputs are seeded synthetic tensors of the workload's shapes,
resident in HBM before timing starts. Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 4] [--calls 200]

The headline workload is --config 4 (32K-token context, B4, 32/8 heads, D128,
64-node dynamic trees). `value` is verified tree tokens per second of one
attention layer: B*N over the mean tv_attention duration, from a block of
--calls back-to-back calls timed with HIP events on the launch stream. The
K whole steps are timed as well (ms_per_step, step_tokens_per_s). The other
workloads (--extra-configs) are measured the same way afterwards and reported
under "other_configs", each with its own roofline (MFMA-bound above the bf16
ridge point, HBM-bound below it). --accept stochastic runs a greedy workload's
tree with sampled acceptance instead. Only one GPU is supported.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published peak
BF16_DENSE_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published peak


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=4, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--calls", type=int, default=200,
                    help="back-to-back calls per timed block of each kernel call (at least 100)")
    ap.add_argument("--extra-configs", default="1,2,3,5",
                    help="other workloads measured after the headline one and reported as extra keys "
                         "(comma-separated config numbers; empty for none)")
    ap.add_argument("--accept", default="default", choices=["default", "stochastic"],
                    help="stochastic: run the workload's tree with sampled acceptance (T = 1, draft rows and "
                         "uniforms from the same seeded streams, each node's token drawn from its draft row)")
    ap.add_argument("--nodes", type=int, default=0,
                    help="tree node slots per sequence (up to 128) instead of the workload's own N")
    ap.add_argument("--ragged", action="store_true",
                    help="give each sequence a seeded node count in [N/2, N] (tree_sizes)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--step-only", action="store_true",
                    help="stop after the timed region (steps and call blocks; no mask-cost, decode, cold-cache, "
                         "builder, commit or other-workload timings), so that a trace sees the step's kernels only")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target wall time of the oracle sample")
    ap.add_argument("--power-seconds", type=int, default=3,
                    help="seconds of back-to-back tv_attention calls during which amd-smi samples package power and "
                         "clocks (0 to skip)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the timed steps, run one device-to-device copy of this many MiB (an HBM counter "
                         "calibration point for rocprofv3 --pmc runs)")
    return ap.parse_args()


def workload_name(w, c, sizes=None):
    L = f"L~U[{c['L'][0]},{c['L'][1]}]" if isinstance(c["L"], tuple) else f"L{c['L']}"
    n = f"N{w.N}" if sizes is None else f"N{w.N} ragged (node counts in [{int(sizes.min())}, {int(sizes.max())}])"
    return (f"cfg{w.cfg} {c['name']}: B{w.B} Hq{w.Hq}/Hkv{w.Hkv} D{w.D} {L} {n} tree={c['tree']} "
            f"V{w.V} {w.mode}")


def present(w, sizes):
    """Node count of every sequence."""
    return np.full(w.B, w.N, np.int64) if sizes is None else sizes.astype(np.int64)


def attention_bytes(w, sizes=None):
    """Algorithmic HBM bytes of one tv_attention call: every visible K/V row
    once, Q once, the output once, masks, page-table entries, prefix lengths
    (present nodes only)."""
    n = present(w, sizes)
    W = (w.N + 63) // 64
    toks = int((w.prefix_lens.astype(np.int64) + n).sum())
    kv = toks * w.Hkv * w.D * 2 * 2
    rows = int(n.sum()) * w.Hq
    q, out = rows * w.D * 2, rows * w.D * 4
    pages = int(((w.prefix_lens.astype(np.int64) + n + 15) // 16).sum()) * 4
    return kv + q + out + int(n.sum()) * 8 * W + pages + w.B * 4 * (2 if sizes is not None else 1)


def attention_flops(w, depth, sizes=None):
    """4*D flops (QK^T and PV) per visible (query row, key) pair."""
    n = present(w, sizes)
    live = np.arange(w.N)[None, :] < n[:, None]
    vis = ((w.prefix_lens.astype(np.int64)[:, None] + depth + 1) * live).sum()  # keys seen by each node
    return 4 * w.D * w.Hq * int(vis)


def accept_bytes(w, sizes=None):
    n = int(present(w, sizes).sum())
    if w.mode == "greedy":
        return n * w.V * 4 + n * 4 * 3
    # target rows, draft rows 1..n-1, and one re-read of a target and a draft row for the final draw
    return (2 * n - w.B) * w.V * 4 + 2 * w.B * w.V * 4 + n * 4 * 3


KERNEL_SOURCES = {"tv_attention": "attention.hip", "tv_accept": "accept.hip", "tv_build_mask": "mask.hip"}
CALL_KERNELS = {"tv_attention": "attn_mfma_kernel (+ attn_combine_kernel when the keys are split)",
                "tv_accept": "argmax_chunk_kernel + greedy_path_kernel (greedy; argmax_path_kernel alone for "
                             "grids of at most 256 workgroups) or softmax_chunk_kernel + stochastic_path_kernel "
                             "(stochastic)",
                "tv_build_mask": "build_mask_kernel",
                "tv_commit": "commit_kernel"}


def measured_traffic(call, key):
    """HBM bytes per call from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summaries (already scaled by the copy-kernel calibration), used only while
    the source hash recorded with them matches the current kernel source."""
    import glob
    import hashlib

    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[call], "tv_internal.h"):
        with open(os.path.join(ROOT, "tree_verify_attention_attn_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    src = h.hexdigest()[:16]
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "hbm_traffic_*.txt"))):
        with open(path) as fh:
            for line in fh:
                parts = line.split()
                if len(parts) == 6 and parts[0] == "traffic" and parts[1] == call:
                    kv = dict(p.split("=", 1) for p in parts[2:])
                    if kv["config"] == str(key) and kv["src"] == src:
                        return int(kv["read_bytes"]) + int(kv["write_bytes"])
    return None


def cpu_baseline(w, depth, target_s, threads, sizes=None):
    """Times the fp64 oracle (attention for every head of the sampled nodes,
    then their acceptance) on the host, on whole sequences, growing the
    sample until it takes about `target_s` seconds or covers the batch; a
    shorter sample is repeated until about `target_s` seconds are spent and
    its median run is reported."""
    import oracle

    n = present(w, sizes)
    omask, _ = oracle.build_mask(w.parents, tree_sizes=sizes)

    def run(nseq):
        rows = np.array([[b, i, h] for b in range(nseq) for i in range(int(n[b])) for h in range(w.Hq)], np.int32)
        ts = None if sizes is None else sizes[:nseq]
        oracle.attention(w, omask, rows=rows, nthreads=threads, tree_sizes=sizes)
        if w.mode == "greedy":
            oracle.accept_greedy(w.target_logits[:nseq], w.draft_tokens[:nseq], w.parents[:nseq], nthreads=threads,
                                 tree_sizes=ts)
        else:
            oracle.accept_stochastic(w.target_logits[:nseq], w.draft_logits[:nseq], w.draft_tokens[:nseq],
                                     w.parents[:nseq], w.uniforms[:nseq], w.temperature, nthreads=threads,
                                     tree_sizes=ts)

    nseq, elapsed, done = 1, 0.0, 0
    while True:
        t0 = time.perf_counter()
        run(nseq)
        elapsed = time.perf_counter() - t0
        done = nseq
        if elapsed >= target_s or nseq >= w.B:
            break
        nseq = min(w.B, max(nseq + 1, int(nseq * min(8.0, 1.2 * target_s / max(elapsed, 1e-3)))))
    # a sample shorter than the target (the whole batch took less) is run
    # again until about target_s of CPU work is spent; the median run counts
    runs = [elapsed]
    while sum(runs) < target_s and len(runs) < 10000:
        t0 = time.perf_counter()
        run(done)
        runs.append(time.perf_counter() - t0)
    elapsed = float(np.median(runs))
    toks = int(n[:done].sum())
    return dict(value=toks / elapsed, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{done} of {w.B} sequences ({toks} tree tokens, {toks * w.Hq} attention rows "
                       f"+ acceptance), {elapsed:.3g} s wall"
                       f"{f' (median of {len(runs)} runs)' if len(runs) > 1 else ''}, fp64 C oracle, "
                       f"{threads} threads", host_cores=os.cpu_count())


def copy_for_calibration(torch, dev, mib):
    """One device-to-device copy of `mib` MiB, whose counter readings calibrate
    rocprofv3's FETCH_SIZE and WRITE_SIZE against known bytes."""
    src = torch.empty(mib << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def commit_moves(w, path, lens):
    """Rows (per KV head) a commit moves: path entries after the identity run."""
    rows = 0
    for b in range(w.B):
        p = path[b, :lens[b]]
        rows += int((p != np.arange(len(p))).sum())
    return rows


def commit_bytes(w, path, lens):
    """Algorithmic bytes of one tv_commit: every moved K and V row read and
    written once, plus per-sequence metadata (prefix length, accepted length,
    bonus, the accepted path, two page-table entries per path node) read and
    the outputs (new length, next root, emitted row) written."""
    kv = commit_moves(w, path, lens) * w.Hkv * w.D * 2 * 2 * 2
    n = int(np.sum(lens))
    return kv + w.B * 12 + n * 4 * 3 + w.B * (w.N + 2) * 4


def device_time(torch, call, n=50):
    """Mean device time (us) of `call` over n back-to-back calls. A call can be
    shorter than its host-side launch, so the stream is held by a bounded spin
    kernel while the host queues all n; the events then time the calls back
    to back on the device. Returns (us, whether the spin outlasted the
    queueing)."""
    for _ in range(5):
        call()
    es, e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    torch.cuda.synchronize()
    es.record()
    torch.cuda._sleep(5_000_000)
    e0.record()
    h0 = time.perf_counter()
    for _ in range(n):
        call()
    host_ms = (time.perf_counter() - h0) * 1e3
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n * 1e3, bool(host_ms < es.elapsed_time(e0))


def build_tree_timing(tv, torch, d, w, c):
    """Times tv_build_tree on this workload's tree shape, fed the proposal
    rows the input generator draws for its trees (threshold 0, as there)."""
    import tvgen

    B, N, k = w.B, w.N, c["topk"]
    toks, probs = np.zeros((B, N, k), np.int32), np.zeros((B, N, k), np.float32)
    roots = np.zeros(B, np.int32)
    for b in range(B):
        rec = {}
        _, t = tvgen.dynamic_tree(w.seed, (tvgen.TID_TREE << 16) + b, N, c["max_depth"], k, w.V, record=rec)
        roots[b] = t[0]
        for node, (tk, sc) in rec.items():
            if node < N:
                toks[b, node], probs[b, node] = tk, sc
    dr, dt, dp = d(roots), d(toks), d(probs)
    out = tv.tv_build_tree(dr, dt, dp, k, 0.0, c["max_depth"])
    # the generator multiplies fp64 probabilities, the builder their fp32
    # roundings: a near tie can order two nodes differently
    same = float((out["parents"].cpu().numpy() == w.parents).all(1).mean())
    us, ok = device_time(torch, lambda: tv.tv_build_tree(dr, dt, dp, k, 0.0, c["max_depth"], outputs=out))
    return {"avg_us": us, "queued_within_spin": ok, "trees": B, "nodes_per_tree": N, "proposals_per_node": k,
            "same_trees_as_workload": same,
            "nodes_per_s": B * N / us * 1e6,
            "note": "tv_build_tree (not part of the step) rebuilding this workload's trees from the proposal rows "
                    "the input generator drew; one wavefront per tree, sequential best-first pops: latency-bound"}


def commit_timing(tv, torch, dev, w, depth, d, kp, vp, table, plens, tokens, outs):
    """Times tv_commit (after acceptance; it rewrites the pools, so it runs
    after every other GPU measurement) on two sets of paths: the last timed
    step's own acceptance, and each sequence's deepest root-to-leaf path (the
    most rows its tree can move)."""
    deep_path = np.full((w.B, w.N), -1, np.int32)
    deep_len = np.zeros(w.B, np.int32)
    for b in range(w.B):
        c, p = int(np.argmax(depth[b])), []
        while c >= 0:
            p.append(c)
            c = int(w.parents[b, c])
        deep_path[b, :len(p)] = p[::-1]
        deep_len[b] = len(p)
    bonus = d(np.arange(w.B, dtype=np.int32))
    co = dict(new_prefix_lens=torch.empty(w.B, dtype=torch.int32, device=dev),
              next_root=torch.empty(w.B, dtype=torch.int32, device=dev),
              emitted=torch.empty((w.B, w.N), dtype=torch.int32, device=dev))
    step_path, step_len = outs["path"].cpu().numpy(), outs["accept_len"].cpu().numpy()
    res = {}
    for name, pth, ln, bn in (("step_paths", outs["path"], outs["accept_len"], outs["bonus"]),
                              ("deepest_paths", d(deep_path), d(deep_len), bonus)):
        hp, hl = (step_path, step_len) if name == "step_paths" else (deep_path, deep_len)
        def call():
            tv.tv_commit(kp, vp, table, plens, w.max_prefix_len, tokens, pth, ln, bn, outputs=co)
        us, queued = device_time(torch, call)
        nbytes = commit_bytes(w, hp, hl)
        res[name] = {"avg_us": us, "queued_within_spin": queued,
                     "rows_moved_per_kv_head": commit_moves(w, hp, hl),
                     "mean_accept_len": float(np.mean(hl)), "bytes": nbytes, "gbs": nbytes / us / 1e3}
    assert tv.tv_device_error(dev) == 0
    res["note"] = ("tv_commit after acceptance (not part of the step); one workgroup per (sequence, KV head), "
                   "a single dependent read-then-write round trip: latency-bound, not bandwidth-bound")
    return res


RIDGE_FLOP_PER_BYTE = BF16_DENSE_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)  # 312.5: above it the MFMA peak binds


def usable_cores():
    """Host cores this process may use: its CPU affinity, capped by a cgroup
    CPU quota and by OMP_NUM_THREADS when either is set (the share a shared
    host grants one job)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    try:
        with open("/sys/fs/cgroup/cpu.max") as fh:
            quota, period = fh.read().split()[:2]
            if quota != "max":
                n = min(n, max(1, int(-(-int(quota) // int(period)))))
    except (OSError, ValueError):
        pass
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(n, 1)


def block_us(torch, call, n):
    """Mean device time (us) of `call` over a block of n back-to-back calls,
    with HIP events recorded on the launch stream around the whole block."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n):
        call()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n * 1e3


def roofline_entry(name, us, nbytes, flops, traffic=None, kernel=None):
    """The roofline of one call: HBM when its arithmetic intensity is below
    the bf16 ridge point, MFMA above it."""
    if flops and flops / nbytes > RIDGE_FLOP_PER_BYTE:
        ach = flops / us / 1e6  # TFLOP/s
        r = {"bound": "mfma", "achieved": ach, "peak": BF16_DENSE_TFLOPS, "unit": "TFLOP/s",
             "frac": ach / BF16_DENSE_TFLOPS, "algorithmic_flops": flops,
             "hbm_gbs": nbytes / us / 1e3, "hbm_frac": nbytes / us / 1e3 / HBM_PEAK_GBS}
    else:
        ach = nbytes / us / 1e3  # GB/s
        r = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS}
        if flops:
            r["mfma_frac"] = flops / us / 1e6 / BF16_DENSE_TFLOPS
    r["traffic"] = traffic
    r["algorithmic_bytes"] = nbytes
    r["call_us"] = us
    if kernel:
        r["kernel"] = kernel
    return r


class Setup:
    """One workload's inputs and outputs resident on the GPU, and its calls."""

    def __init__(self, torch, tv, cfg, stochastic=False, nodes=0, ragged=False):
        import tvgen

        self.torch, self.tv, self.cfg = torch, tv, cfg
        dev = self.dev = torch.device("cuda:0")
        self.c = c = tvgen.CONFIGS[cfg]
        over = {}
        if stochastic:
            over["mode"] = "stochastic"
        if nodes:
            over["N"] = nodes
        self.w = w = tvgen.make_workload(cfg, overrides=over or None)
        self.key = str(cfg) + ("-stochastic" if stochastic else "") + (f"-N{nodes}" if nodes else "") + \
            ("-ragged" if ragged else "")
        self.depth = np.stack([tvgen.tree_depths(p) for p in w.parents])
        self.sizes = None
        if ragged:
            st = tvgen.Stream(w.seed, 41)
            self.sizes = np.array([w.N - w.N // 2 + st.randint(w.N // 2 + 1) for _ in range(w.B)], np.int32)
        self.n_present = present(w, self.sizes)
        self.tokens = int(self.n_present.sum())
        d = self.d
        self.parents, self.tokens_d = d(w.parents), d(w.draft_tokens)
        self.q, self.kp, self.vp = d(w.q, torch.bfloat16), d(w.k_pages, torch.bfloat16), d(w.v_pages, torch.bfloat16)
        self.table, self.plens = d(w.page_table), d(w.prefix_lens)
        self.tl = d(w.target_logits)
        self.dl = d(w.draft_logits) if w.draft_logits is not None else None
        self.un = d(w.uniforms) if w.uniforms is not None else None
        self.mode = tv.GREEDY if w.mode == "greedy" else tv.STOCHASTIC
        self.mask = torch.empty((w.B, w.N, (w.N + 63) // 64), dtype=torch.int64, device=dev)
        self.ts = d(self.sizes) if self.sizes is not None else None
        self.dep = torch.empty((w.B, w.N), dtype=torch.int32, device=dev)
        self.out = torch.empty((w.B, w.N, w.Hq, w.D), dtype=torch.float32, device=dev)
        aws = tv.tv_attention_workspace_bytes(dev, w.B, w.N, w.Hq, w.Hkv, w.D, w.max_prefix_len)
        self.attn_ws = torch.empty(max(aws, 1), dtype=torch.uint8, device=dev)
        self.acc_ws = torch.empty(max(tv.tv_accept_workspace_bytes(w.B, w.N, w.V, self.mode), 1), dtype=torch.uint8,
                                  device=dev)
        self.outs = dict(accept_len=torch.empty(w.B, dtype=torch.int32, device=dev),
                         path=torch.empty((w.B, w.N), dtype=torch.int32, device=dev),
                         bonus=torch.empty(w.B, dtype=torch.int32, device=dev))
        self.a_bytes = attention_bytes(w, self.sizes)
        self.a_flops = attention_flops(w, self.depth, self.sizes)
        self.c_bytes = accept_bytes(w, self.sizes)
        tv.tv_build_mask(self.parents, self.mask, self.dep, tree_sizes=self.ts)

    def d(self, a, dtype=None):
        t = self.torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(dtype) if dtype is not None else t).to(self.dev)

    def build_mask(self):
        self.tv.tv_build_mask(self.parents, self.mask, self.dep, tree_sizes=self.ts)

    def attention(self, mask="tree"):
        w = self.w
        self.tv.tv_attention(self.q, self.kp, self.vp, self.table, self.plens, w.max_prefix_len,
                             self.mask if mask == "tree" else None, float(w.sm_scale), out=self.out,
                             workspace=self.attn_ws, tree_sizes=self.ts)

    def accept(self):
        w = self.w
        self.tv.tv_accept(self.tl, self.tokens_d, self.parents, mode=self.mode, draft_logits=self.dl,
                          uniforms=self.un, temperature=w.temperature, outputs=self.outs, workspace=self.acc_ws,
                          tree_sizes=self.ts)

    def step(self):
        self.build_mask()
        self.attention()
        self.accept()

    def name(self):
        return workload_name(self.w, self.c, self.sizes)

    def calls(self, n):
        """tv_attention, tv_accept and tv_build_mask, each timed over a block
        of n back-to-back calls."""
        torch = self.torch
        for _ in range(3):
            self.step()
        t_attn = block_us(torch, self.attention, n)
        t_acc = block_us(torch, self.accept, n)
        t_mask = block_us(torch, self.build_mask, n)
        return t_attn, t_acc, t_mask

    def mask_cost(self):
        """tv_attention with the tree mask against the same call with
        tree_mask = NULL (every tree key visible), interleaved in blocks of 20
        calls, the order of the two blocks alternating from round to round so
        that clock drift and position affect both alike; medians of 6 blocks."""
        masked, unmasked = [], []
        for r in range(6):
            for m in (("tree", None) if r % 2 == 0 else (None, "tree")):
                (masked if m else unmasked).append(block_us(self.torch, lambda: self.attention(m), 20))
        t_m, t_u = float(np.median(masked)), float(np.median(unmasked))
        return {"masked_us": t_m, "unmasked_us": t_u, "overhead": t_m / t_u - 1.0,
                "note": "tv_attention with the tree mask vs tree_mask=NULL on the same KV"}


ATTN_KERNEL = "tv_attention: attn_mfma_kernel (+ attn_combine_kernel when the keys are split)"


def power_sample(torch, call, seconds):
    """Runs `call` back to back for about `seconds` + 2 s while amd-smi samples
    the package power and the graphics clock of every XCD once a second
    (`amd-smi metric -p -c`), and reads the board's power cap (`rocm-smi
    --showmaxpower`). Returns None when the tools are missing."""
    import shutil
    import subprocess

    if shutil.which("amd-smi") is None:
        return None
    smp = subprocess.Popen(["amd-smi", "metric", "-p", "-c", "--csv", "-w", "1", "-W", str(int(seconds))],
                           stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds + 2.0:
        for _ in range(50):
            call()
        n += 50
    torch.cuda.synchronize()
    try:
        out = smp.communicate(timeout=30)[0]
    except subprocess.TimeoutExpired:
        smp.kill()
        return None
    hdr, rows = None, []
    for line in out.splitlines():
        f = [x.strip() for x in line.split(",")]
        if "socket_power" in f:
            hdr = f
        elif hdr and len(f) == len(hdr):
            r = dict(zip(hdr, f))
            try:
                clk = [float(r[f"gfx_{i}_clk"]) for i in range(8) if f"gfx_{i}_clk" in r and r[f"gfx_{i}_clk"] != "N/A"]
                rows.append((float(r["socket_power"]), sum(clk) / len(clk) if clk else None))
            except (KeyError, ValueError):
                pass
    if len(rows) < 2:
        return None
    rows = rows[1:]  # the first sample can precede the load
    cap = None
    if shutil.which("rocm-smi"):
        txt = subprocess.run(["rocm-smi", "--showmaxpower"], capture_output=True, text=True).stdout
        for line in txt.splitlines():
            if "Max Graphics Package Power" in line:
                try:
                    cap = float(line.rsplit(":", 1)[1])
                except ValueError:
                    pass
    return {"socket_power_w": [p for p, _ in rows], "gfx_clock_mhz": [c for _, c in rows],
            "power_cap_w": cap, "calls": n,
            "note": "amd-smi metric -p -c once a second while the call runs back to back (the first sample "
                    "dropped); gfx_clock_mhz = mean over the XCDs of each sample"}


def extra_config(torch, tv, cfg, n):
    """Attention and acceptance of another workload, as extra keys of the line."""
    s = Setup(torch, tv, cfg)
    t_attn, t_acc, t_mask = s.calls(n)
    assert tv.tv_device_error(s.dev) == 0
    res = {"workload": s.name(), "tree_tokens": s.tokens,
           "tokens_per_s": s.tokens / t_attn * 1e6,
           "roofline": roofline_entry("tv_attention", t_attn, s.a_bytes, s.a_flops,
                                      measured_traffic("tv_attention", s.key), ATTN_KERNEL),
           "tv_accept": {"avg_us": t_acc, "bytes": s.c_bytes, "gbs": s.c_bytes / t_acc / 1e3,
                         "hbm_frac": s.c_bytes / t_acc / 1e3 / HBM_PEAK_GBS,
                         "traffic": measured_traffic("tv_accept", s.key)},
           "tv_build_mask_us": t_mask,
           "mask_overhead": s.mask_cost(),
           "calls_per_block": n}
    if cfg == 1:
        res["note"] = "launch-bound: 60 KB per call"
    del s
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import tree_verify_attention_attn_amd as tv

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    s = Setup(torch, tv, args.config, stochastic=args.accept == "stochastic" and
              tvgen_mode(args.config) != "stochastic", nodes=args.nodes, ragged=args.ragged)
    w, dev = s.w, s.dev
    ncalls = max(args.calls, 100)

    for _ in range(args.warmup):
        s.step()
    torch.cuda.synchronize()
    tv.tv_tau_reset(dev)
    if tv.tv_device_error(dev) != 0:
        raise RuntimeError("device error during warm-up")

    # the timed region: K whole steps (mask, attention, accept), then a block
    # of back-to-back calls of each kernel call, with HIP events on the launch
    # stream around each block
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        s.step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tau, cycles = tv.tv_tau(dev)
    t_attn, t_acc, t_mask = s.calls(ncalls)
    assert tv.tv_device_error(dev) == 0

    ms_per_step = wall / args.steps * 1e3
    tokens = s.tokens
    kernels = {
        "tv_build_mask": dict(avg_us=t_mask),
        "tv_attention": dict(avg_us=t_attn, bytes=s.a_bytes, flops=s.a_flops, gbs=s.a_bytes / t_attn / 1e3,
                             hbm_frac=s.a_bytes / t_attn / 1e3 / HBM_PEAK_GBS,
                             mfma_frac=s.a_flops / t_attn / 1e6 / BF16_DENSE_TFLOPS,
                             tokens_per_s=tokens / t_attn * 1e6),
        "tv_accept": dict(avg_us=t_acc, bytes=s.c_bytes, gbs=s.c_bytes / t_acc / 1e3,
                          hbm_frac=s.c_bytes / t_acc / 1e3 / HBM_PEAK_GBS,
                          traffic=measured_traffic("tv_accept", s.key)),
        "calls_per_block": ncalls,
    }
    roof = roofline_entry("tv_attention", t_attn, s.a_bytes, s.a_flops, measured_traffic("tv_attention", s.key),
                          ATTN_KERNEL)
    roof["note"] = ("achieved = algorithmic bytes (or flops) per tv_attention call / its mean duration over a block "
                    "of back-to-back calls (HIP events on the launch stream around the block); traffic = calibrated "
                    "rocprofv3 FETCH_SIZE + WRITE_SIZE bytes per call, null when not measured for this source")
    result = {
        "metric": "verified tree tokens/sec per attention layer; achieved HBM GB/s vs peak",
        "value": tokens / t_attn * 1e6,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": s.name(), "batch": w.B, "tree_nodes": w.N,
                   "tree_tokens_per_step": tokens, "q_heads": w.Hq,
                   "kv_heads": w.Hkv, "head_dim": w.D, "max_prefix_len": w.max_prefix_len, "vocab": w.V,
                   "accept": w.mode, "page_size": 16, "parallelism": "single-gpu"},
        "value_note": ("value = B*N tree tokens / mean tv_attention duration (one attention layer) over a block of "
                       "back-to-back calls; step_tokens_per_s = the same tokens / the whole step (mask + attention + "
                       "acceptance), from the wall clock around the K timed steps"),
        "step_tokens_per_s": tokens * args.steps / wall,
        "roofline": roof,
        "kernels": kernels,
        "tau": tau,
        "tau_cycles": cycles,
    }
    if args.step_only:
        if args.copy_mib > 0:
            copy_for_calibration(torch, dev, args.copy_mib)
        print(json.dumps(result), flush=True)
        return
    result["mask_overhead"] = s.mask_cost()
    # the package power and clock while tv_attention runs back to back
    if args.power_seconds > 0:
        result["power"] = power_sample(torch, s.attention, args.power_seconds)
    # verify premium: the same call for the root row only (N = 1, a plain
    # decode step) over the same KV, blocks of 20 calls, medians of 5 blocks
    q1 = s.q[:, :1].contiguous()
    out1 = torch.empty((w.B, 1, w.Hq, w.D), dtype=torch.float32, device=dev)
    ws1 = torch.empty(max(tv.tv_attention_workspace_bytes(dev, w.B, 1, w.Hq, w.Hkv, w.D, w.max_prefix_len), 1),
                      dtype=torch.uint8, device=dev)

    def decode():
        tv.tv_attention(q1, s.kp, s.vp, s.table, s.plens, w.max_prefix_len, None, float(w.sm_scale), out=out1,
                        workspace=ws1)
    t_dec = float(np.median([block_us(torch, decode, 20) for _ in range(5)]))
    t_m = result["mask_overhead"]["masked_us"]
    result["verify_premium"] = {"decode_us": t_dec, "verify_us": t_m, "premium": t_m / t_dec,
                                "tree_tokens_per_decode_token": tokens / w.B,
                                "note": "tv_attention over the same KV for the root row only (N = 1, no mask) "
                                        "against the tree-verify call"}
    # cold caches: before each timed call a 1 GiB buffer is written, which
    # evicts the 4 MB L2s and the 256 MB MALL; 10 calls of each
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def cold(call, nbytes):
        ts_ = []
        for r in range(10):
            flush.fill_(r & 0xFF)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            call()
            e1.record()
            torch.cuda.synchronize()
            ts_.append(e0.elapsed_time(e1) * 1e3)
        med = float(np.median(ts_))
        return dict(median_us=med, p10_us=float(np.percentile(ts_, 10)), p90_us=float(np.percentile(ts_, 90)),
                    gbs=nbytes / med / 1e3, hbm_frac=nbytes / med / 1e3 / HBM_PEAK_GBS)
    result["cold_cache"] = {
        "tv_attention": cold(s.attention, s.a_bytes),
        "tv_accept": cold(s.accept, s.c_bytes),
        "note": "one call after writing a 1 GiB buffer (L2 and MALL evicted); the block figures above are warm"}
    # a measured stream copy on this machine: 1 GiB device to device (2 GiB moved),
    # median of 5; the kernels' bandwidth is also reported as a fraction of it
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(3)
    cps = []
    for _ in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        flush.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        cps.append(e0.elapsed_time(e1) * 1e-3)
    copy_gbs = 2 * (1 << 30) / float(np.median(cps[1:])) / 1e9
    result["stream_copy"] = {"gbs": copy_gbs, "frac_of_peak": copy_gbs / HBM_PEAK_GBS,
                             "tv_attention_frac_of_copy": kernels["tv_attention"]["gbs"] / copy_gbs,
                             "tv_accept_frac_of_copy": kernels["tv_accept"]["gbs"] / copy_gbs,
                             "note": "1 GiB device-to-device copy (read + write), median of 5 after one warm-up"}
    del flush, src
    if s.c["tree"] == "dynamic" and s.sizes is None:
        result["build_tree"] = build_tree_timing(tv, torch, s.d, w, s.c)
    depth_present = np.where(np.arange(w.N)[None, :] < s.n_present[:, None], s.depth, -1)
    result["commit"] = commit_timing(tv, torch, dev, w, depth_present, s.d, s.kp, s.vp, s.table, s.plens,
                                     s.d(w.draft_tokens), s.outs)
    if args.copy_mib > 0:
        copy_for_calibration(torch, dev, args.copy_mib)
    # the other workloads: attention and acceptance of each, as extra keys
    extras = [int(x) for x in args.extra_configs.split(",") if x.strip()] if args.extra_configs else []
    extras = [x for x in extras if x != args.config]
    depth, sizes = s.depth, s.sizes  # host arrays, kept for the CPU baseline
    if extras:
        del s
        torch.cuda.empty_cache()
        result["other_configs"] = {f"cfg{x}": extra_config(torch, tv, x, ncalls) for x in extras}
    if not args.no_cpu_baseline:
        threads = usable_cores()
        result["cpu_baseline"] = cpu_baseline(w, depth, args.cpu_seconds, threads, sizes)
        result["cpu_baseline"]["cpu_model"] = cpu_model()
        if args.config in (1, 2):  # the single-thread figure on the two small workloads
            one = cpu_baseline(w, depth, min(args.cpu_seconds, 5.0), 1, sizes)
            result["cpu_baseline"]["one_thread"] = {"value": one["value"], "sample": one["sample"]}
    print(json.dumps(result), flush=True)


def tvgen_mode(cfg):
    import tvgen
    return tvgen.CONFIGS[cfg]["mode"]


if __name__ == "__main__":
    main()
