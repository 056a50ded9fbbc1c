"""CSA2 decode benchmark: layer-steps/s of one decode group (Full + Reindex + Reuse) at 1M
context on one MI355X, with the scan kernel's HBM roofline and the CPU oracle beside it.

A step is one decode group over the whole batch: for every layer the current token's window
row is appended, the Full layer also appends its global-KV row and runs the full indexer
(one fused call),
Reindex rescores the pool, Reuse keeps the previous top-k, and every layer runs sparse
attention.  Inputs are seeded synthetic tensors resident in HBM before timing starts.  Each
step uses the next of R cache replicas so the 256 MB Infinity Cache cannot hold the
working set; the group is replayed from a HIP graph (one per replica).

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, os.path.join(ROOT, "tests")):
    if p not in sys.path:
        sys.path.insert(0, p)

import numpy as np  # noqa: E402
import torch  # noqa: E402

METRIC = "CSA2 decode layer-steps/s at 1M ctx (Full+Reindex+Reuse); % HBM roofline"
HBM_PEAK_GBS = 8000.0
SCAN_KERNEL = "k_scan"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="long_1m")
    ap.add_argument("--replicas", type=int, default=0, help="0 = enough for >= 1 GiB")
    ap.add_argument("--scan-reps", type=int, default=40)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="no HIP graph")
    ap.add_argument("--counters", action="store_true",
                    help="for rocprofv3 --pmc: a few eager launches of the dominant kernel, then a "
                         "device-to-device copy of --calib-mb MiB (counter calibration); no timing")
    ap.add_argument("--calib-mb", type=int, default=512)
    ap.add_argument("--counter-summary", metavar="DIR",
                    help="no GPU: write profiles/<kernel counters>.json from the FETCH_SIZE and "
                         "WRITE_SIZE csv files that two rocprofv3 --pmc runs of --counters left in "
                         "DIR (file prefix dec_ for decode, pf_ for --workload prefill, sp_ for "
                         "--workload spec_1m)")
    return ap.parse_args()


class Bench:
    """One decode group over the whole batch, as a model runs it layer after layer: every
    index layer quantises its fp32 indexer query (MXFP4), the Full layer appends the token's
    global-KV row inside its index call, Reindex rescores the pool, Reuse keeps the previous
    top-k, and every layer appends its window row inside its attention call.  Each layer
    keeps its own outputs (top-k, attention output and log-sum-exp), so that one replay can
    be checked layer by layer."""

    def __init__(self, wl, replicas):
        import kv_cache_decode_csa2_amd as k
        import synth_inputs as si
        from gpu_harness import GpuState, dev
        from harness import make_table

        self.k, self.wl = k, wl
        table, nblk = make_table(wl.ctx, seed=wl.seed, permute=False)
        self.table_np, self.n_blocks = table, nblk
        t0 = time.time()
        g = GpuState(wl, table, nblk, with_latent=True)
        log(f"caches built in {time.time() - t0:.1f}s")
        self.g = g
        self.cfg = g.cfg
        layout = k.csa2_layout(self.cfg)
        self.ab = algorithmic_bytes(wl, layout)
        # replicas rotate so that the other replicas' group bytes (>= 512 MB) pass between
        # two uses of one replica: the 256 MB Infinity Cache cannot hold a replica's bytes
        R = replicas or 1 + int(np.ceil((512 << 20) / self.ab["total"]))
        self.kv = [g.kv] + [g.kv.clone() for _ in range(R - 1)]
        self.idx = [g.idx] + [g.idx.clone() for _ in range(R - 1)]
        self.R = R
        B, maxb = table.shape
        self.maxb = maxb
        i32 = dict(dtype=torch.int32, device="cuda")
        self.layers = []
        src = -1
        for li, mode in enumerate(wl.layers):
            lay = dict(mode=mode, q=g.attn_q(li), swa=g.layer_swa(li),
                       swa_row=dev(np.stack([si.layer_swa_rows(wl, li, b, min(wl.ctx[b], wl.W))[-1]
                                             for b in range(B)])),
                       out=torch.empty((B, wl.H_q, wl.D), dtype=torch.float32, device="cuda"),
                       lse=torch.empty((B, wl.H_q), dtype=torch.float32, device="cuda"))
            if mode in "FR":
                lay["qf"] = dev(si.layer_idx_q(wl, li).reshape(B, wl.H_I * wl.d_I))
                lay["w"] = dev(si.layer_idx_w(wl, li))
                lay["qc"] = torch.empty((B, wl.H_I * wl.d_I // 2), dtype=torch.uint8, device="cuda")
                lay["qs"] = torch.empty((B, wl.H_I * wl.d_I // 32), dtype=torch.uint8, device="cuda")
                lay["topk"] = torch.empty((B, wl.k), **i32)
                lay["topk_len"] = torch.empty(B, **i32)
                k.csa2_quantize_mxfp4(lay["qf"], lay["qc"], lay["qs"])  # (for scan() alone)
                src = li
            lay["src"] = src  # the layer whose top-k this layer attends
            self.layers.append(lay)
        # the current token's global row (position L-1), appended by the Full layer
        self.tok_lat = dev(np.stack([si.latent_rows(wl, b, wl.ctx[b])[-1] for b in range(B)]))
        self.tok_key = dev(np.stack([si.idx_keys(wl, b)[-1] for b in range(B)]))
        self.ws = [torch.zeros(k.csa2_workspace_bytes(self.cfg, k.CSA2_OP_INDEX_FULL, B, maxb),
                               dtype=torch.uint8, device="cuda") for _ in range(R)]
        self.ws_attn = torch.zeros(k.csa2_workspace_bytes(self.cfg, k.CSA2_OP_SPARSE_ATTN, B, maxb),
                                   dtype=torch.uint8, device="cuda")
        self.pool = torch.empty((B, wl.K_blk), **i32)
        self.pool_len = torch.empty(B, **i32)
        torch.cuda.synchronize()

    def step(self, r, only=None):
        """One decode group on replica r (only: just that layer, for the per-mode times):
        one fused layer call per layer (the indexer query's quantise, the token's appends,
        the index step of the layer's mode and its attention)."""
        k, g, c = self.k, self.g, self.cfg
        kv, idx, ws = self.kv[r], self.idx[r], self.ws[r]
        for li, lay in enumerate(self.layers):
            if only is not None and li != only:
                continue
            if lay["mode"] == "F":
                k.csa2_decode_full_layer(c, lay["qf"], lay["w"], self.tok_lat, self.tok_key,
                                         lay["swa_row"], lay["q"], kv, idx, g.n_blocks, g.table,
                                         lay["swa"], g.C, g.ctx, self.pool, self.pool_len,
                                         lay["topk"], lay["topk_len"], lay["out"], lay["lse"], ws,
                                         self.ws_attn)
            elif lay["mode"] == "R":
                k.csa2_decode_reindex_layer(c, lay["qf"], lay["w"], lay["swa_row"], lay["q"], kv,
                                            idx, g.n_blocks, g.table, lay["swa"], g.C, g.ctx,
                                            self.pool, self.pool_len, lay["topk"],
                                            lay["topk_len"], lay["out"], lay["lse"], ws,
                                            self.ws_attn)
            else:
                s = self.layers[lay["src"]]
                k.csa2_decode_reuse_layer(c, lay["swa_row"], lay["q"], kv, g.n_blocks, g.table,
                                          lay["swa"], g.C, g.ctx, s["topk"], s["topk_len"],
                                          lay["out"], lay["lse"], self.ws_attn)

    def scribble(self, r):
        """Overwrite what the group appends (position L-1 of the global caches of replica r
        and of every window ring) with other values, so that a replay that follows must
        write them itself."""
        import synth_inputs as si
        from gpu_harness import dev
        k, g, wl = self.k, self.g, self.wl
        B = wl.B
        pos = dev((np.asarray(wl.ctx, np.int64) - 1).astype(np.int32))
        k.csa2_append_global(self.cfg, dev(si.normal(wl.seed, 4001, (B, wl.D))),
                             dev(si.normal(wl.seed, 4002, (B, wl.H_I * wl.d_I))), g.table,
                             g.n_blocks, pos, 1, self.kv[r], self.idx[r])
        for li, lay in enumerate(self.layers):
            k.csa2_append_swa(self.cfg, dev(si.normal(wl.seed, 4003 + li, (B, wl.D))), pos, 1,
                              lay["swa"], g.C)
        torch.cuda.synchronize()

    def results(self):
        """Per-layer outputs of the last step (host arrays): the pool of the Full layer, and
        per layer the attended top-k, its length, the attention output and log-sum-exp."""
        res = []
        for lay in self.layers:
            s = self.layers[lay["src"]]
            res.append(dict(mode=lay["mode"], topk=s["topk"].cpu().numpy(),
                            topk_len=s["topk_len"].cpu().numpy(), out=lay["out"].cpu().numpy(),
                            lse=lay["lse"].cpu().numpy()))
        return dict(pool=self.pool.cpu().numpy(), pool_len=self.pool_len.cpu().numpy(),
                    layers=res)

    def scan(self, r):
        lay = self.layers[0]
        self.k.csa2_index_full_scan(self.cfg, lay["qc"], lay["qs"], lay["w"], self.idx[r],
                                    self.g.n_blocks, self.g.table, self.g.ctx, self.ws[r])


def kernels_per_mode(wl):
    """Kernel launches of one layer of each mode in the step (the fused layer calls): Full =
    scan (with the query quantise and global append) + selection + attention, plus a global
    append of its own for 8 x 128-style layouts (four 32-groups per head, two or more heads)
    and for the shared-key variant; Reindex = rescoring scan + selection + attention; Reuse =
    attention."""
    own_append = (wl.d_I // 32 > 2 and wl.H_I > 1) or wl.shared_key
    return {"F": 4 if own_append else 3, "R": 3, "U": 1}


def oracle_group(wl, o):
    """The decode group computed by the oracle on its own caches (which hold every position
    up to L-1, i.e. the state after the group's appends): per-layer pool, top-k and
    attention, in the layout of Bench.results()."""
    import oracle
    import synth_inputs as si
    pool = topk = None
    res = []
    for li, mode in enumerate(wl.layers):
        if mode in "FR":
            q = si.layer_idx_q(wl, li).reshape(wl.B, wl.H_I * wl.d_I)
            qc, qs = oracle.quantize_mxfp4(q)
            w = si.layer_idx_w(wl, li)
        if mode == "F":
            p, pl, t, tl = oracle.index_full(o.cfg, qc, qs, w, o.idx, o.table, o.ctx)
            pool, topk = (p, pl), (t, tl)
        elif mode == "R":
            topk = oracle.index_reindex(o.cfg, qc, qs, w, o.idx, o.table, o.ctx, *pool)
        out, lse = oracle.sparse_attn(o.cfg, si.layer_attn_q(wl, li), o.kv, o.table,
                                      o.layer_swa(li), o.C, o.ctx, *topk)
        res.append(dict(mode=mode, topk=topk[0], topk_len=topk[1], out=out, lse=lse))
    return dict(pool=pool[0], pool_len=pool[1], layers=res)


def compare_group(got, ref, tol=2e-3):
    """Index sets bit-exact and attention within tol per (sequence, head) row; returns a
    summary dict whose "ok" says whether everything matched."""
    from gpu_harness import attn_close
    sets = bool(np.array_equal(got["pool"], ref["pool"]) and
                np.array_equal(got["pool_len"], ref["pool_len"]))
    rel_max = lse_max = 0.0
    attn_ok = True
    for g_, r_ in zip(got["layers"], ref["layers"]):
        sets = sets and bool(np.array_equal(g_["topk"], r_["topk"]) and
                             np.array_equal(g_["topk_len"], r_["topk_len"]))
        ok, rel, lerr = attn_close(g_["out"], g_["lse"], r_["out"], r_["lse"], tol)
        attn_ok = attn_ok and ok
        rel_max, lse_max = max(rel_max, rel), max(lse_max, lerr)
    return dict(index_sets_bit_exact=sets, attn_max_rel_err=float(f"{rel_max:.3g}"),
                lse_max_err=float(f"{lse_max:.3g}"), tolerance=tol, ok=bool(sets and attn_ok))


class PrefillBench:
    """The prefill-chunk workload: n_q query tokens at the end of one sequence run the
    prefill indexer (matrix-core scoring + per-query selection) and the per-query sparse
    attention over their top-k and window.  Speculative verification (1 + 5 draft tokens)
    is the same step with n_q = 6.  The indexer cache is replicated (replicas rotate between
    steps) so that the replicas together exceed the 256 MB Infinity Cache."""

    def __init__(self, wl, replicas=0):
        import kv_cache_decode_csa2_amd as k
        import synth_inputs as si
        from gpu_harness import GpuState, dev, prefill_q
        from harness import make_table

        self.k, self.wl = k, wl
        table, nblk = make_table(wl.ctx, seed=wl.seed, permute=False)
        t0 = time.time()
        g = GpuState(wl, table, nblk, with_latent=True)
        log(f"caches built in {time.time() - t0:.1f}s")
        self.g, self.cfg = g, g.cfg
        self.R = replicas or max(1, -(-(1 << 30) // g.idx.numel()))
        self.idx = [g.idx] + [g.idx.clone() for _ in range(self.R - 1)]
        self.n_q = wl.n_q
        self.q_pos0 = wl.ctx[0] - wl.n_q
        self.row = g.table[0].contiguous()
        self.maxb = self.row.numel()
        self.qc, self.qs, self.w = prefill_q(wl, 0, self.n_q)
        self.C = self.n_q + wl.W
        first = max(0, self.q_pos0 - wl.W + 1)
        rows = si.layer_swa_rows(wl, 0, 0, self.q_pos0 + self.n_q - first)
        self.ring = torch.zeros((1, self.C, g.lay.swa_row_bytes), dtype=torch.uint8, device="cuda")
        k.csa2_append_swa(self.cfg, dev(rows), dev(np.array([first], np.int32)), rows.shape[0],
                          self.ring, self.C)
        self.qa = dev(si.prefill_attn_q(wl, 0, self.n_q).view(np.int16))
        n = self.n_q
        self.ws = torch.zeros(k.csa2_workspace_bytes(self.cfg, k.CSA2_OP_INDEX_PREFILL, n, self.maxb),
                              dtype=torch.uint8, device="cuda")
        self.ws_attn = torch.zeros(k.csa2_workspace_bytes(self.cfg, k.CSA2_OP_SPARSE_ATTN, n, self.maxb),
                                   dtype=torch.uint8, device="cuda")
        i32 = dict(dtype=torch.int32, device="cuda")
        self.pool = torch.empty((n, wl.K_blk), **i32)
        self.pool_len = torch.empty(n, **i32)
        self.topk = torch.empty((n, wl.k), **i32)
        self.topk_len = torch.empty(n, **i32)
        self.out = torch.empty((n, wl.H_q, wl.D), dtype=torch.float32, device="cuda")
        self.lse = torch.empty((n, wl.H_q), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()

    def step(self, r=0):
        k, g, c = self.k, self.g, self.cfg
        k.csa2_index_prefill(c, self.qc, self.qs, self.w, self.q_pos0, self.idx[r], g.n_blocks, self.row,
                             self.pool, self.pool_len, self.topk, self.topk_len, self.ws)
        k.csa2_sparse_attn_prefill(c, self.qa, g.kv, g.n_blocks, self.row, self.ring, self.C,
                                   self.q_pos0, self.topk, self.topk_len, self.out, self.lse,
                                   self.ws_attn)

    def scan(self, r=0):
        self.k.csa2_index_prefill_scan(self.cfg, self.qc, self.qs, self.w, self.q_pos0, self.idx[r],
                                       self.g.n_blocks, self.row, self.ws)

    def index(self, r=0):
        k, g, c = self.k, self.g, self.cfg
        k.csa2_index_prefill(c, self.qc, self.qs, self.w, self.q_pos0, self.idx[r], g.n_blocks, self.row,
                             self.pool, self.pool_len, self.topk, self.topk_len, self.ws)


def prefill_work(wl, layout):
    """Algorithmic work of the prefill indexer's scoring: causal (query, position) pairs, the
    FP4 flops of their scores, and the bytes the method must move -- every key once plus the
    selection outputs (pool and top-k of every query).  The kernels' own intermediate writes
    are a design choice, counted apart as `design_bytes`: one pass writes an exact score per
    causal pair (at most 16 queries), or the maxima pass writes block and group maxima and the
    rescoring pass the scores of about k flagged blocks per query (8 scores each)."""
    n_q, L = wl.n_q, wl.ctx[0]
    t = np.arange(L - n_q, L, dtype=np.int64)
    pairs = int((t + 1).sum())
    blocks = int(((t + 8) // 8).sum())
    flops = 2 * pairs * wl.H_I * wl.d_I
    alu = 2 * pairs * wl.H_I  # ReLU + fma per (pair, head)
    keys = L * (layout.idx_block_bytes // 8)
    outputs = n_q * (wl.K_blk + wl.k + 2) * 4
    maxima = 4 * blocks + 4 * ((blocks + 7) // 8)
    design = 4 * pairs + maxima if n_q <= 16 else maxima + n_q * wl.k * 8 * 4
    return dict(pairs=pairs, flops=flops, alu=alu, bytes=keys + outputs, key_bytes=keys,
                output_bytes=outputs, design_bytes=design)


MFMA_FP4_PEAK_TFLOPS = 10100.0
ALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12  # fp32 lane-instructions/s without packed math


def calibration_copy(mb):
    """A plain device copy of known size (mb MiB read, mb MiB written) for counter scaling."""
    src = torch.ones(mb << 18, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"calibration copy: {mb} MiB")


def main_prefill(a, wl):
    bench = PrefillBench(wl, a.replicas)
    R = bench.R
    if a.counters:
        for i in range(3):
            bench.step(i % R)
        torch.cuda.synchronize()
        calibration_copy(a.calib_mb)
        return
    spec = wl.name.startswith("spec")
    layout = bench.k.csa2_layout(bench.cfg)
    pw = prefill_work(wl, layout)
    if a.eager:
        step = lambda i: bench.step(i % R)  # noqa: E731
    else:
        graphs = [capture(lambda r=r: bench.step(r)) for r in range(R)]
        step = lambda i: graphs[i % R].replay()  # noqa: E731
    warm = a.warmup if spec else max(1, a.warmup // 4)
    timed(step, warm)
    steps = a.steps if spec else max(1, a.steps // 20)
    ms = timed(step, steps)
    value = (1.0 if spec else bench.n_q) / (ms / 1e3)
    log(f"{wl.name} step {ms:.4f} ms -> {value:.0f} {'verify-steps' if spec else 'query-tokens'}/s"
        f" ({R} replicas)")
    import hashlib
    src = open(os.path.join(ROOT, "kv_cache_decode_csa2_amd", "csrc", "csa2_prefill.hip"), "rb").read()
    traffic = traffic_for(hashlib.sha256(src).hexdigest(), COUNTER_RUNS[counter_kind(wl)][3], wl.name)
    reps = 40 if spec else 5
    sg = capture(lambda: [bench.scan(i % R) for i in range(reps)])
    timed(lambda i: sg.replay(), 1)
    scan_ms = timed(lambda i: sg.replay(), 3) / reps
    sec = scan_ms / 1e3
    # the whole indexer call (the scoring pass, the pool selection, for more than 16 queries the
    # rescoring of the flagged blocks, the top-k selection)
    ig = capture(lambda: [bench.index(i % R) for i in range(reps)])
    timed(lambda i: ig.replay(), 1)
    index_ms = timed(lambda i: ig.replay(), 3) / reps
    fr = {"hbm": pw["bytes"] / sec / 1e9 / HBM_PEAK_GBS,
          "mfma": pw["flops"] / sec / 1e12 / MFMA_FP4_PEAK_TFLOPS,
          "alu": pw["alu"] / sec / 1e12 / ALU_PEAK_TOPS}
    log(f"prefill scoring {scan_ms:.3f} ms: hbm {fr['hbm']:.3f}, mfma {fr['mfma']:.3f}, "
        f"alu {fr['alu']:.3f} of peak")
    # the chunk's scores are a dense FP4 contraction (matrix-core bound by arithmetic
    # intensity); a verification step's 6 queries read every key for few flops (HBM bound)
    bound = "hbm" if spec else "mfma"
    ach = {"hbm": pw["bytes"] / sec / 1e9, "mfma": pw["flops"] / sec / 1e12,
           "alu": pw["alu"] / sec / 1e12}[bound]
    peak = {"hbm": HBM_PEAK_GBS, "mfma": MFMA_FP4_PEAK_TFLOPS, "alu": ALU_PEAK_TOPS}[bound]
    unit = {"hbm": "GB/s", "mfma": "TFLOP/s", "alu": "Tops/s"}[bound]
    metric = ("CSA2 speculative-verification steps/s at 1M ctx (1 + 5 draft queries: prefill "
              "indexer + sparse attention)" if spec else
              "CSA2 prefill-chunk query-tokens/s (prefill indexer + sparse attention)")
    result = {
        "metric": metric,
        "value": round(value, 1), "unit": "verify-steps/s" if spec else "query-tokens/s",
        "n_gpus": 1, "steps": steps,
        "warmup": warm, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "mxfp4", "data": "synthetic",
        "config": {"workload": wl.name, "queries": wl.n_q, "context": wl.ctx[0],
                   "indexer": f"{wl.H_I}x{wl.d_I} fp4", "pool_blocks": wl.K_blk, "topk": wl.k,
                   "q_heads": wl.H_q, "window": wl.W, "replicas": R, "graph": not a.eager},
        "roofline": {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
                     "frac": round(fr[bound], 4), "traffic": traffic,
                     "traffic_over_algorithmic": (round(traffic / pw["bytes"], 2)
                                                  if traffic else None),
                     "algorithmic_bytes": pw["bytes"],
                     "kernel": "k_prefill" if spec else "k_prefill maxima pass",
                     "kernel_us": round(scan_ms * 1e3, 2),
                     "index_us": round(index_ms * 1e3, 2),
                     "index_frac": round({"hbm": pw["bytes"] / (index_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                                          "mfma": pw["flops"] / (index_ms / 1e3) / 1e12 / MFMA_FP4_PEAK_TFLOPS}[bound], 4),
                     "fractions": {k_: round(v, 4) for k_, v in fr.items()}, "work": pw},
        "cpu_baseline": None,
    }
    if not a.no_cpu_baseline:
        result["cpu_baseline"] = (cpu_baseline_spec(wl, a.cpu_seconds) if spec else
                                  cpu_baseline_prefill(wl, a.cpu_seconds))
    print(json.dumps(result), flush=True)


def cpu_baseline_prefill(wl, seconds):
    """The oracle on a bounded sample of the prefill chunk: its queries taken one at a time
    from the end of the chunk backwards (each the Full steps on its causal prefix, then its
    attention over its top-k and window), for about `seconds`; query-tokens/s."""
    import oracle
    import synth_inputs as si
    from harness import OracleState, make_table
    table, nblk = make_table(wl.ctx, seed=wl.seed, permute=False)
    t0 = time.time()
    o = OracleState(wl, table, nblk, with_latent=True)
    log(f"oracle caches built in {time.time() - t0:.1f}s")
    n_q = wl.n_q
    q_pos0 = wl.ctx[0] - n_q
    qc, qs = oracle.quantize_mxfp4(si.prefill_idx_q(wl, 0, n_q).reshape(n_q, -1))
    w = si.prefill_idx_w(wl, 0, n_q)
    C = n_q + wl.W
    first = max(0, q_pos0 - wl.W + 1)
    rows = si.layer_swa_rows(wl, 0, 0, q_pos0 + n_q - first)
    ring = oracle.alloc_swa(o.cfg, 1, C)
    oracle.append_swa(o.cfg, rows[None], np.array([first], np.int32), ring, C)
    qa = si.prefill_attn_q(wl, 0, n_q)
    n = 0
    t0 = time.time()
    while n < n_q:
        i = n_q - 1 - n
        _, _, t, tl = oracle.index_prefill(o.cfg, qc[i:i + 1], qs[i:i + 1], w[i:i + 1],
                                           q_pos0 + i, o.idx, o.table[0])
        oracle.sparse_attn_prefill(o.cfg, qa[i:i + 1], o.kv, o.table[0], ring[0], C, q_pos0 + i,
                                   t, tl)
        n += 1
        el = time.time() - t0
        if el >= seconds:
            break
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    cores = int(os.environ.get("OMP_NUM_THREADS", cores))
    return dict(value=n / el, unit="query-tokens/s", cores=cores, kind="oracle",
                sample=f"the last {n} of the {n_q} queries of the {wl.name} workload, each "
                       f"indexed over its whole causal prefix (~{wl.ctx[0]} positions) and "
                       f"attended, {el:.1f} s wall")


def capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # one eager run on the side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    return graph


def timed(fn, n):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(n):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def algorithmic_bytes(wl, layout):
    """Bytes the method must move per group (see the measurement notes of the design)."""
    B = wl.B
    idx_pos = layout.idx_block_bytes // 8
    L = np.asarray(wl.ctx, np.int64)
    scan = int(L.sum()) * idx_pos
    pool_pos = int(np.minimum(L, wl.K_blk * 8).sum())
    reindex = pool_pos * idx_pos
    rows_main = int(np.minimum(L, wl.k).sum()) * layout.kv_row_bytes
    rows_win = int(np.minimum(L, wl.W).sum()) * layout.swa_row_bytes
    qio = B * wl.H_q * (wl.D * 2 + wl.D * 4 + 4)
    attn = rows_main + rows_win + qio
    n_r = wl.layers.count("R")
    total = scan + n_r * reindex + len(wl.layers) * attn
    return dict(scan=scan, reindex=reindex, attn=attn, total=total)


def cpu_baseline(wl, seconds, gpu_first=None):
    """The oracle on whole decode groups of the workload for about `seconds` (its first
    group is also the reference the GPU's first replay is compared with)."""
    from harness import OracleState, make_table
    table, nblk = make_table(wl.ctx, seed=wl.seed, permute=False)
    t0 = time.time()
    o = OracleState(wl, table, nblk, with_latent=True)
    log(f"oracle caches built in {time.time() - t0:.1f}s")
    groups = 0
    first = None
    t0 = time.time()
    while True:
        res = oracle_group(wl, o)
        first = first or res
        groups += 1
        el = time.time() - t0
        if el >= seconds:
            break
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    cores = int(os.environ.get("OMP_NUM_THREADS", cores))
    base = dict(value=groups * len(wl.layers) / el, unit="layer-steps/s", cores=cores,
                kind="oracle",
                sample=f"{groups} full {''.join(wl.layers)} groups of the {wl.name} workload "
                       f"(all {sum(wl.ctx)} positions scanned per Full layer), {el:.1f} s wall")
    parity = None
    if gpu_first is not None:
        parity = dict(checked="first replay of the group graph (replica 0) against the oracle's "
                              "first group", **compare_group(gpu_first, first))
    return base, parity


def cpu_baseline_spec(wl, seconds):
    """The oracle on the verification step: the prefill indexer over the n_q queries (each
    the Full steps on its causal prefix) and their sparse attention, repeated for about
    `seconds`."""
    import oracle
    import synth_inputs as si
    from harness import OracleState, make_table
    table, nblk = make_table(wl.ctx, seed=wl.seed, permute=False)
    t0 = time.time()
    o = OracleState(wl, table, nblk, with_latent=True)
    log(f"oracle caches built in {time.time() - t0:.1f}s")
    n_q = wl.n_q
    q_pos0 = wl.ctx[0] - n_q
    qc, qs = oracle.quantize_mxfp4(si.prefill_idx_q(wl, 0, n_q).reshape(n_q, -1))
    w = si.prefill_idx_w(wl, 0, n_q)
    C = n_q + wl.W
    first = max(0, q_pos0 - wl.W + 1)
    rows = si.layer_swa_rows(wl, 0, 0, q_pos0 + n_q - first)
    ring = oracle.alloc_swa(o.cfg, 1, C)
    oracle.append_swa(o.cfg, rows[None], np.array([first], np.int32), ring, C)
    qa = si.prefill_attn_q(wl, 0, n_q)
    n = 0
    t0 = time.time()
    while True:
        _, _, t, tl = oracle.index_prefill(o.cfg, qc, qs, w, q_pos0, o.idx, o.table[0])
        oracle.sparse_attn_prefill(o.cfg, qa, o.kv, o.table[0], ring[0], C, q_pos0, t, tl)
        n += 1
        el = time.time() - t0
        if el >= seconds:
            break
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    cores = int(os.environ.get("OMP_NUM_THREADS", cores))
    return dict(value=n / el, unit="verify-steps/s", cores=cores, kind="oracle",
                sample=f"{n} whole verification steps of the {wl.name} workload ({n_q} queries, "
                       f"all {wl.ctx[0]} positions scored per query), {el:.1f} s wall")


def traffic_for(kernel_src_hash, name="scan_long_1m_counters.json", workload="long_1m"):
    """HBM bytes per launch measured by the counter runs recorded in profiles/<name>, if they
    were taken on the current kernel source and on this workload (else None)."""
    path = os.path.join(ROOT, "profiles", name)
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_sha256") != kernel_src_hash or not d.get("workload", "").startswith(workload + ":"):
        return None
    return d.get("bytes_per_launch")


COUNTER_RUNS = {  # workload kind -> (file prefix, kernel, kernel source, profile name, workload)
    "decode": ("dec", "k_scan<", "csa2_index.hip", "scan_long_1m_counters.json",
               "long_1m: B=1, L=1,048,576, indexer 4x64 FP4"),
    "prefill": ("pf", "k_prefill<", "csa2_prefill.hip", "prefill_counters.json",
                "prefill: 4096 queries at 258048..262143, L=262,144, indexer 8x128 FP4"),
    "spec": ("sp", "k_prefill<", "csa2_prefill.hip", "spec_1m_counters.json",
             "spec_1m: 6 queries at 1048570..1048575, L=1,048,576, indexer 4x64 FP4"),
}


def counter_kind(wl):
    return "spec" if wl.name.startswith("spec") else ("prefill" if wl.n_q else "decode")


def _targs(kname, name):
    """Template arguments of a kernel name that starts with kname ('k_scan<', 'k_prefill<')."""
    return name.split(kname, 1)[1].split(">", 1)[0] if kname in name else ""


def _counted(kind, kname, name):
    """The dispatches a counter summary covers: the Full-mode scan (not the Reindex rescoring,
    k_scan<H, G, true, ...>); the prefill chunk's maxima pass (k_prefill<H, G, false, 1>); the
    verification step's one-pass kernel (k_prefill<H, G, true, 0>)."""
    if kname not in name:
        return False
    t = _targs(kname, name)
    if kind == "decode":
        return ", true," not in t[:12]
    if kind == "prefill":
        return t.endswith("false, 1")
    return t.endswith("true, 0")


def counter_summary(a, wl):
    """HBM bytes per launch of the dominant kernel from two rocprofv3 --pmc runs (FETCH_SIZE,
    WRITE_SIZE; KiB per dispatch), each scaled by what the same counter reads for the
    calibration copy of a.calib_mb MiB that --counters runs after the kernel."""
    import csv
    import hashlib
    kind = counter_kind(wl)
    prefix, kname, src_name, out_name, wl_text = COUNTER_RUNS[kind]
    raw = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        with open(os.path.join(a.counter_summary, f"{prefix}_{ctr}_counter_collection.csv")) as f:
            rows = [r for r in csv.DictReader(f) if r["Counter_Name"] == ctr]
        kern = [float(r["Counter_Value"]) for r in rows if _counted(kind, kname, r["Kernel_Name"])]
        if kind == "prefill":
            resc = [float(r["Counter_Value"]) for r in rows if "k_prefill_rescore<" in r["Kernel_Name"]]
            raw["rescore_" + ctr] = sum(resc) / max(1, len(resc))
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        if not kern or not copies:
            raise SystemExit(f"{ctr}: no {kname} or copy dispatches in {a.counter_summary}")
        raw[ctr] = (sum(kern) / len(kern), len(kern), max(copies))
    calib = a.calib_mb << 20
    # the copy reads and writes calib bytes; FETCH_SIZE counts half of them on this machine
    ff = calib / (raw["FETCH_SIZE"][2] * 1024.0)
    wf = calib / (raw["WRITE_SIZE"][2] * 1024.0)
    fetch = raw["FETCH_SIZE"][0] * 1024.0 * ff
    write = raw["WRITE_SIZE"][0] * 1024.0 * wf
    src_path = os.path.join(ROOT, "kv_cache_decode_csa2_amd", "csrc", src_name)
    if kind != "decode":
        alg = prefill_work(wl, _layout_of(wl))["bytes"]
    else:
        alg = wl.max_ctx * (wl.H_I * (wl.d_I // 2 + wl.d_I // 32))
    wl_flag = f" --workload {wl.name}" if kind != "decode" else ""
    d = {
        "kernel": kname, "dispatches": raw["FETCH_SIZE"][1],
        "fetch_kib_raw": round(raw["FETCH_SIZE"][0], 1), "write_kib_raw": round(raw["WRITE_SIZE"][0], 1),
        "calibration": {"copy_mib": a.calib_mb, "fetch_kib_raw": raw["FETCH_SIZE"][2],
                        "write_kib_raw": raw["WRITE_SIZE"][2], "fetch_factor": round(ff, 4),
                        "write_factor": round(wf, 4)},
        "fetch_bytes": int(fetch), "write_bytes": int(write), "bytes_per_launch": int(fetch + write),
        **({"rescoring_pass": {"kernel": "k_prefill_rescore<H, G>",
                               "fetch_bytes": int(raw["rescore_FETCH_SIZE"] * 1024.0 * ff),
                               "write_bytes": int(raw["rescore_WRITE_SIZE"] * 1024.0 * wf)}}
           if kind == "prefill" else {}),
        "algorithmic_bytes": int(alg),
        "source_sha256": hashlib.sha256(open(src_path, "rb").read()).hexdigest(),
        "source": f"kv_cache_decode_csa2_amd/csrc/{src_name}",
        "command": [f"rocprofv3 --pmc {c} --kernel-include-regex '{kname.rstrip('<')}|copyBuffer|copy' "
                    f"--output-format csv -d {a.counter_summary} -o {prefix}_{c} -- python3 bench.py"
                    f"{wl_flag} --counters" for c in ("FETCH_SIZE", "WRITE_SIZE")]
                   + [f"python3 bench.py{wl_flag} --counter-summary {a.counter_summary}"],
        "workload": wl_text,
    }
    with open(os.path.join(ROOT, "profiles", out_name), "w") as f:
        json.dump(d, f, indent=1)
        f.write("\n")
    log(f"wrote profiles/{out_name}: {d['bytes_per_launch'] / 1e6:.1f} MB per launch "
        f"(algorithmic {alg / 1e6:.1f} MB)")


def _layout_of(wl):
    class L:  # the index-cache block size, as csa2_layout states it
        idx_block_bytes = 8 * wl.H_I * (wl.d_I // 2 + wl.d_I // 32)
    return L


PCIE_PEAK_GBS = 63.0  # PCIe 5.0 x16, one direction (32 GT/s x 16 lanes, 128b/130b)


def main_tier(a):
    """The persistent global-KV tier at 1M context: both FP4 block caches of the long_1m
    sequence (indexer keys and main latent rows of 1,048,576 positions) leave through
    csa2_blocks_gather into pinned host memory and come back through csa2_blocks_scatter into
    another physical placement.  One step = save (gather + device-to-host) and restore
    (host-to-device + scatter) of both caches."""
    import kv_cache_decode_csa2_amd as k
    import synth_inputs as si
    from gpu_harness import GpuState, dev
    from harness import make_table
    wl = si.workload("long_1m")
    table, nblk = make_table(wl.ctx, seed=wl.seed, permute=False)
    t0 = time.time()
    g = GpuState(wl, table, nblk, with_latent=True)
    log(f"caches built in {time.time() - t0:.1f}s")
    valid = table >= 0
    new_table, _ = make_table(wl.ctx, seed=wl.seed + 1, permute=True)
    src = dev(table[valid].astype(np.int32))
    dst = dev(new_table[valid].astype(np.int32))
    caches = [g.idx, g.kv]
    rows = [torch.empty((src.numel(), c.shape[1]), dtype=torch.uint8, device="cuda") for c in caches]
    host = [torch.empty(r.shape, dtype=torch.uint8, pin_memory=True) for r in rows]
    total = sum(r.numel() for r in rows)

    def save():
        for c, r, h in zip(caches, rows, host):
            k.csa2_blocks_gather(c, src, r)
            h.copy_(r, non_blocking=True)

    def restore():
        for c, r, h in zip(caches, rows, host):
            r.copy_(h, non_blocking=True)
            k.csa2_blocks_scatter(r, dst, c)

    steps = max(1, a.steps // 20)
    save(), restore()
    t_save = timed(lambda i: save(), steps)
    t_restore = timed(lambda i: restore(), steps)
    t_gather = timed(lambda i: [k.csa2_blocks_gather(c, src, r) for c, r in zip(caches, rows)], steps)
    t_scatter = timed(lambda i: [k.csa2_blocks_scatter(r, dst, c) for c, r in zip(caches, rows)], steps)
    ms = t_save + t_restore
    value = 2 * total / (ms / 1e3) / 1e9
    log(f"tier: {total / 1e6:.1f} MB each way, save {t_save:.2f} ms, restore {t_restore:.2f} ms, "
        f"device gather {t_gather:.3f} ms, scatter {t_scatter:.3f} ms")
    kern_ms = (t_gather + t_scatter) / 2
    ach = 2 * total / (kern_ms / 1e3) / 1e9  # each copy kernel reads and writes the bytes
    result = {
        "metric": "CSA2 global-KV tier round trip GB/s at 1M ctx (save + restore of both FP4 "
                  "block caches through pinned host memory)",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": 1,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": "tier_1m", "context": wl.ctx[0], "indexer": f"{wl.H_I}x{wl.d_I} fp4",
                   "bytes_each_way": total, "pinned_host": True},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "k_blocks_copy", "kernel_us": round(kern_ms * 1e3, 2)},
        "pcie": {"save_ms": round(t_save, 3), "restore_ms": round(t_restore, 3),
                 "save_gbs": round(total / t_save / 1e6, 2),
                 "restore_gbs": round(total / t_restore / 1e6, 2), "peak_per_direction": PCIE_PEAK_GBS},
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


def main():
    a = parse()
    if a.counter_summary:
        import synth_inputs as si
        return counter_summary(a, si.workload(a.workload))
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 (multi-GPU "
                                   "sharding is a design note, not implemented)"}))
        sys.exit(2)
    import hashlib

    import synth_inputs as si
    torch.cuda.set_device(0)
    if a.workload == "tier_1m":
        return main_tier(a)
    wl = si.workload(a.workload)
    if wl.n_q:
        return main_prefill(a, wl)
    bench = Bench(wl, a.replicas)
    if a.counters:
        for i in range(3):
            bench.scan(i % bench.R)
        torch.cuda.synchronize()
        calibration_copy(a.calib_mb)
        return
    ab = bench.ab
    R = bench.R
    log(f"workload {wl.name}: {R} replicas, algorithmic bytes/group {ab['total'] / 1e6:.1f} MB")

    if a.eager:
        step = lambda i: bench.step(i % R)  # noqa: E731
    else:
        graphs = [capture(lambda r=r: bench.step(r)) for r in range(R)]
        step = lambda i: graphs[i % R].replay()  # noqa: E731
    # the first replay's per-layer results, compared with the oracle in the CPU leg
    step(0)
    torch.cuda.synchronize()
    first = bench.results()
    timed(step, a.warmup)
    ms = timed(step, a.steps)
    n_layers = len(wl.layers)
    value = n_layers / (ms / 1e3)
    log(f"group {ms * 1e3:.1f} us -> {value:.0f} layer-steps/s")
    # per-mode times: each layer of the group replayed alone (its inputs -- the pool and
    # top-k of the earlier layers -- are those the group left in place)
    modes = {}
    if not a.eager:
        for li, mode in enumerate(wl.layers):
            lg = [capture(lambda r=r: bench.step(r, only=li)) for r in range(R)]
            timed(lambda i: lg[i % R].replay(), max(1, a.warmup // 2))
            modes.setdefault(mode, round(timed(lambda i: lg[i % R].replay(), max(1, a.steps // 2)) * 1e3, 2))
        log(f"per-mode us: {modes}")

    # scan kernel alone: a graph of back-to-back scans over rotating replicas
    reps = a.scan_reps
    sg = capture(lambda: [bench.scan(i % R) for i in range(reps)])
    timed(lambda i: sg.replay(), 2)
    scan_ms = timed(lambda i: sg.replay(), 5) / reps
    achieved = ab["scan"] / (scan_ms / 1e3) / 1e9
    src = open(os.path.join(ROOT, "kv_cache_decode_csa2_amd", "csrc", "csa2_index.hip"), "rb").read()
    traffic = traffic_for(hashlib.sha256(src).hexdigest(), workload=wl.name)
    log(f"scan {scan_ms * 1e3:.2f} us -> {achieved:.0f} GB/s")

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "layer-steps/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "context": wl.max_ctx,
                   "context_min": int(min(wl.ctx)), "context_total": int(sum(wl.ctx)),
                   "indexer": f"{wl.H_I}x{wl.d_I} fp4" + (" (one shared key per position)"
                                                            if wl.shared_key else ""),
                   "pool_blocks": wl.K_blk, "topk": wl.k,
                   "q_heads": wl.H_q, "window": wl.W, "layers": wl.layers,
                   "replicas": R, "graph": not a.eager},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": SCAN_KERNEL + ("_shared" if wl.shared_key else ""),
                     "kernel_us": round(scan_ms * 1e3, 3), "algorithmic_bytes": ab["scan"]},
        "group": {"algorithmic_bytes": ab["total"],
                  "kernels_per_mode": kernels_per_mode(wl),
                  "pages_kernels_per_reuse_layer": {"decode": 11, "prefill": 15},
                  "hbm_frac": round(ab["total"] / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                  "us_per_mode": modes,
                  "sequence_layer_steps_per_s": round(value * wl.B, 1)},
        "cpu_baseline": None,
    }
    if not a.no_cpu_baseline:
        result["cpu_baseline"], result["parity"] = cpu_baseline(wl, a.cpu_seconds, first)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
