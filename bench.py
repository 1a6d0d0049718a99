#!/usr/bin/env python3
"""Indexer throughput on one MI355X: HISA against the flat DSA indexer.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line on stdout.  The default workload is the 32K decode
batch: 16 sequences of 32768 keys (d = 64, bf16, mixture-of-Gaussians keys),
B = 128, m = 64, k = 2048.  One step is one decode step of the whole path:
each sequence appends its newest key (position 32767, with the in-place
update of that block's representative) and its query at 32767 is indexed.
The flat indexer runs the same steps on the same bytes.

Inputs are resident in HBM before the timed region.  To keep the 256 MB
last-level cache from serving repeated steps, the step rotates over
`--replicas` copies of the key cache and representatives (cold-cache
numbers); `--replicas 1` gives the warm-cache figure.

On the 32K decode batch the JSON line also carries an "attention" object:
the sparse attention that consumes the indices (one head of dimension 128,
bf16 queries, keys and values drawn i.i.d. N(0, 1)), timed alone and as
index + attention steps over HISA's and over the flat indexer's output.

The timed region replays one captured HIP graph per step (per replica):
the step's kernels without host work in between.  Per-kernel durations come
from HIP start / stop events attached to the kernel dispatches of a
separate run of eager steps (queued behind a sleep kernel so they run back
to back); the roofline object is computed from the kernel with the largest
average duration.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix peak of one MI355X
# where the library switches to its MFMA kernels (queries per call)
TOKEN_TILES_FROM = 512          # token scores in 16-query MFMA tiles
BLOCK_TILES_FROM = 256          # block scores in 16-query MFMA tiles
FLAT_MFMA_FROM = 32             # flat scores in 16-query MFMA tiles

WORKLOADS = ("decode_32k_x16", "chunked_prefill_32k", "long_context_128k", "long_decode_1m",
             "tiny_prefill_4k", "decode_32k_x64", "decode_32k_x256", "decode_varlen_x64")
# decode batches of more sequences: the same step at larger batch, to show
# where the decode path reaches its steady-state HBM fraction
DECODE_BATCH = {"decode_32k_x16": 16, "decode_32k_x64": 64, "decode_32k_x256": 256}

ATTN_WORKLOADS = ("decode_32k_x16",)
# LSA-Flat leg: workload -> (p buckets searched, k keys); p = k / 8 (8 keys per bucket on average)
LSA_WORKLOADS = {"decode_32k_x16": (256, 2048), "decode_32k_x64": (256, 2048), "decode_varlen_x64": (256, 2048)}
ATTN_SEED = 56

STAGES_HISA = ("block_stage", "token_scores", "token_topk")
STAGES_FLAT = ("flat_scores", "flat_topk")
SPLIT_BELOW = 512               # fewer queries: the token stage splits each query over workgroups
FUSED_MAX_BLOCKS = 2048         # ... and with at most this many blocks stage 1 joins it in one kernel


def hisa_stage_names(nq, max_len, B):
    """Stage index -> name for one HISA call (the library's stage events)."""
    if nq < SPLIT_BELOW and (max_len + B - 1) // B <= FUSED_MAX_BLOCKS:
        return {1: "select_and_scores", 2: "token_topk"}
    return dict(enumerate(STAGES_HISA))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---- algorithmic traffic per stage ------------------------------------------------

def hisa_stage_bytes(q_pos, B, m, k):
    """Algorithmic HBM bytes of the two HISA stages for queries at q_pos
    (d = 64: a key or representative row is 128 bytes).  Block stage: the
    query, its causal representatives, the kept-block list out.  Token
    stage: the query, the kept list, the candidate keys, int32 indices out."""
    q_pos = np.asarray(q_pos, np.int64)
    nb = q_pos // B + 1                                  # causal blocks
    kept = np.minimum(nb, m)
    cand = np.minimum(kept * B, q_pos + 1)                # <= m*B candidate tokens
    return {
        "block_stage": float((128 + nb * 128 + 2 * m * 4).sum()),
        # few queries: scores go to a workspace row, then the top-k reads it
        "token_scores": float((128 + m * 4 + cand * 128 + m * B * 4).sum()),
        "token_topk": float(len(q_pos) * (m * B * 4 + m * 4 + k * 4)),
        # stage 1 and the token scores as one kernel (few queries)
        "select_and_scores": float((128 + nb * 128 + 2 * m * 4).sum() + (128 + m * 4 + cand * 128 + m * B * 4).sum()),
        # the token stage without the workspace round trip: query, kept
        # list and candidate keys in, indices out
        "token_ideal": float((128 + m * 4 + cand * 128 + k * 4).sum()),
    }


def stage_flops(q_pos, B, m):
    """Algorithmic flops of the contractions: 2*64 per (query, row) pair
    over the causal representatives (block stage), the kept candidates
    (token stage) and every visible key (flat scores)."""
    q_pos = np.asarray(q_pos, np.int64)
    nb = q_pos // B + 1
    cand = np.minimum(np.minimum(nb, m) * B, q_pos + 1)
    return {"block_stage": float(128 * nb.sum()), "token_scores": float(128 * cand.sum()),
            "flat_scores": float(128 * (q_pos + 1).sum())}


def stage_roofline(name, ms, nq, flops, nbytes):
    """(bound, achieved, peak, unit, work per launch) of one stage: the
    MFMA-tiled stages against the bf16 matrix peak, the rest against HBM."""
    st = name.split("/")[-1]
    mfma = ((st == "token_scores" and nq >= TOKEN_TILES_FROM) or (st == "block_stage" and nq >= BLOCK_TILES_FROM)
            or (st == "flat_scores" and nq >= FLAT_MFMA_FROM))
    if mfma:
        return "mfma", flops / (ms * 1e-3) / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", flops
    return "hbm", nbytes / (ms * 1e-3) / 1e9, HBM_PEAK_GBPS, "GB/s", nbytes


def flat_stage_bytes(q_pos, k):
    """Flat: the scores stage reads every visible key and writes its score;
    the top-k stage reads the scores and writes int32 indices."""
    q_pos = np.asarray(q_pos, np.int64)
    n = q_pos + 1
    return {
        "flat_scores": float((n * 128 + 128 + n * 4).sum()),
        "flat_topk": float((n * 4).sum() + len(n) * k * 4),
    }


# ---- measured HBM traffic ----------------------------------------------------------

# kernel symbol that carries each stage
STAGE_KERNEL = {"block_stage": ("stage1_select_kernel", "stage1_tile_kernel", "block_score"),
                "token_scores": ("select_score_kernel", "stage2_tile_kernel"),
                "token_topk": ("topk_rows_kernel",),
                "select_and_scores": ("decode_fused_kernel", "decode_step_kernel"),
                "flat_scores": ("flat_score_kernel", "flat_score_mfma_kernel")}


def kernel_source_hash(root):
    import glob
    import hashlib
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(root, "long_context_sparse_hisa_amd", "csrc", "*"))):
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(root, workload, stage, fused_step=False):
    """HBM bytes per dispatch of a stage's kernel from the PMC summary under
    profiles/ (FETCH_SIZE and WRITE_SIZE scaled by a known-size copy), or
    None when there is none or the kernel sources changed since.
    fused_step: the step runs hisa_decode_step, whose selection-and-scores
    kernel is decode_step_kernel rather than decode_fused_kernel."""
    import glob
    sym = STAGE_KERNEL.get(stage.split("/")[-1])
    if sym is None:
        return None
    if fused_step:
        sym = tuple(sorted(sym, key=lambda x: x != "decode_step_kernel"))
    for path in glob.glob(os.path.join(root, "profiles", "*_hbm_traffic.md")):
        lines = open(path).read().splitlines()
        sha = [l.split("=", 1)[1].strip() for l in lines if l.startswith("source_sha256")]
        if not sha or sha[0] != kernel_source_hash(root):
            continue
        rows = [l.split("\t") for l in lines]
        rows = [f for f in rows if len(f) == 4 and f[0] == "traffic" and f[1] == workload]
        for x in sym:                      # the first symbol with a line wins
            for f in rows:
                if x in f[2]:
                    return float(f[3])
    return None


# ---- setup -----------------------------------------------------------------------

class Setup:
    """Device-resident workload: R replicas of keys + reps, the query
    batches of one step, and reusable argument blocks."""

    def __init__(self, name, replicas, hisa_mod, synth, device_mod, torch):
        self.name = name
        self.torch = torch
        self.h = hisa_mod
        dev = "cuda:0"
        if name in DECODE_BATCH:
            ns = DECODE_BATCH[name]
            w = synth.decode_batch(nseq=ns)
            self.desc = ("%d sequences x 32768 keys, d=64 bf16 MoG; B=128 m=64 k=2048; per step: append "
                         "the key at 32767 of every sequence (rep update) + index its query at 32767" % ns)
        elif name == "decode_varlen_x64":
            w = synth.decode_varlen()
            self.desc = ("64 sequences of mixed length (log-uniform in [4096, 131072], %d keys in all), d=64 bf16 "
                         "MoG; B=128 m=64 k=2048; per step: append every sequence's last key (rep update) + index "
                         "its query there, one launch for the batch" % int(w.seq_len.sum()))
        elif name == "chunked_prefill_32k":
            w = synth.chunked_prefill()
            self.desc = "32768 keys, all 32768 causal queries (MoG), d=64 bf16; B=128 m=64 k=2048"
        elif name == "long_context_128k":
            w = synth.long_context()
            self.desc = ("131072 keys (MoG + 64 needles), prefill chunk of 4096 queries + decode batch "
                         "of 32 at 131071; B=128 m=64 k=2048")
        elif name == "long_decode_1m":
            w = synth.long_decode_append(steps=1)
            self.desc = ("1,048,576-key cache (MoG), d=64 bf16; B=128 m=64 k=2048; per step: append 128 "
                         "keys (rep update) + index one query at the last position")
        elif name == "tiny_prefill_4k":
            w = synth.tiny_prefill()
            self.desc = "4096 i.i.d. N(0,1) keys, all 4096 causal queries, d=64 bf16; B=128 m=8 k=256"
        else:
            raise ValueError(name)
        self.w = w
        self.cache = device_mod.DeviceCache(w, device=dev)
        c = self.cache
        # decode workloads: the cache holds L-n_new keys, the step appends n_new
        self.append_src = None
        if name in DECODE_BATCH or name == "decode_varlen_x64":
            c.set_lengths(w.seq_len - 1)
            last = np.stack([w.keys[int(o) + int(L) - 1] for o, L in zip(w.seq_key_off, w.seq_len)])
            self.append_src = device_mod.to_dev(last[:, None, :], dev)
        elif name == "long_decode_1m":
            ph = w.phases[0]
            self.append_src = device_mod.to_dev(ph.append, dev)
        c.pool()
        if self.append_src is not None:
            self.seqs = [(c.seq_key_off[s], c.seq_rep_off[s], c.seq_len[s], c.seq_cap[s])
                         for s in range(c.nseq)]
            c.append(self.append_src, update_lengths=True)   # lengths the queries see
        torch.cuda.synchronize()
        self.phases = w.phases if name != "long_decode_1m" else w.phases[:1]
        self.B, self.m, self.k = w.B, w.m, w.k
        self.max_len = int(c.seq_cap.max())
        # replicas (cold-cache rotation)
        self.keys = [c.keys] + [c.keys.clone() for _ in range(replicas - 1)]
        self.reps = [c.reps] + [c.reps.clone() for _ in range(replicas - 1)]
        self.dev_mod = device_mod
        self.replicas = replicas
        self.block_only = False
        # HISA decode steps: append and index in one hisa_decode_step call
        # (False: the two calls, the form the flat indexer's step takes)
        self.fused_step = self.append_src is not None
        self.calls = {flat: self.build_calls(flat, self.m, self.k) for flat in (False, True)}
        self.q_per_step = sum(len(ph.q_pos) for ph in self.phases)

    def build_calls(self, flat, m, k, block_only=False):
        """Per phase: an IndexCall (buffers) and one argument block per
        replica of the keys and representatives."""
        c = self.cache
        calls = []
        for ph in self.phases:
            ic = self.dev_mod.IndexCall(c, ph.queries, ph.q_pos, ph.q_seq, k=k, m=m, flat=flat, scores=False,
                                        blocks=False, one_chunk_limit=16 << 30, block_only=block_only)
            per_rep = []
            for r in range(self.replicas):
                a = self.h.make_args(ic.queries, ic.q_pos, self.keys[r], k, reps=self.reps[r], q_seq=ic.q_seq,
                                     seq_key_off=c.d_key_off, seq_rep_off=c.d_rep_off, seq_len=c.d_len,
                                     max_len=ic.max_len, B=self.B, m=m, out_idx=ic.out_idx,
                                     out_scores=ic.out_scores, out_blocks=ic.out_blocks, workspace=ic.workspace)
                a.workspace_bytes = ic.args.workspace_bytes
                per_rep.append(a)
            calls.append((ic, per_rep))
        return calls

    def step(self, r, flat, stream, events=None, append_events=None):
        """One step on replica r; events: one StageEvents per phase."""
        h = self.h
        if self.append_src is not None and not flat and not self.block_only and self.fused_step:
            (ic, per_rep), = self.calls[False]
            a = per_rep[r]
            if events is not None:
                events[0].attach(a)
            else:
                a.stage_events = None
            h.hisa_decode_step(a, self.seqs, self.append_src)
            return
        if self.append_src is not None:
            if append_events is not None:
                h._hiprt().hipEventRecord(append_events[0], stream)
            h.hisa_append_keys(self.keys[r], self.reps[r], self.seqs, self.append_src, self.B,
                               self.torch.cuda.current_stream())
            if append_events is not None:
                h._hiprt().hipEventRecord(append_events[1], stream)
        for p, (ic, per_rep) in enumerate(self.calls[flat]):
            a = per_rep[r]
            if events is not None:
                events[p].attach(a)
            else:
                a.stage_events = None
            (h.hisa_flat_index if flat else h.hisa_block_index if self.block_only else h.hisa_index)(a)


class AttentionLeg:
    """The sparse attention over one decode step's indices: per replica of
    the attention keys and values, one call reading the index call's
    output buffer (HISA's or the flat indexer's)."""

    def __init__(self, S, replicas, device_mod, synth, torch):
        w = S.w
        ph = S.phases[0]
        qa, ka, va = synth.attention_inputs(w.keys.shape[0], len(ph.q_pos), seed=ATTN_SEED)
        c = S.cache
        dev = "cuda:0"
        self.scale = 1.0 / np.sqrt(synth.DA)
        q = device_mod.to_dev(qa, dev)
        kr = [device_mod.to_dev(ka, dev)]
        vr = [device_mod.to_dev(va, dev)]
        for _ in range(replicas - 1):
            kr.append(kr[0].clone())
            vr.append(vr[0].clone())
        self.replicas = replicas
        self.kk = S.k
        self.calls = {}
        for flat in (False, True):
            ic = S.calls[flat][0][0]
            self.calls[flat] = [device_mod.AttentionCall(q, kr[r], vr[r], ic.out_idx, self.scale, q_seq=ic.q_seq,
                                                         seq_key_off=c.d_key_off, seq_len=c.d_len)
                                for r in range(replicas)]
        self.nq = len(ph.q_pos)
        self.desc = ("one head, d=128, bf16 q/k/v ~ N(0,1) beside every index key; k=%d indices per query; "
                     "%d replicas of k and v (%.0f MiB each)" % (S.k, replicas, kr[0].numel() * 4 / 2 ** 20))
        torch.cuda.synchronize()

    def algorithmic_bytes(self, n_valid):
        """q row, the index row, the selected key and value rows, the output row."""
        return self.nq * (256 + 4 * self.kk + 512) + int(n_valid) * 512

    def run(self, r, flat):
        self.calls[flat][r % self.replicas].run()


class LsaLeg:
    """LSA-Flat on the workload's keys: the bucket cache of every complete
    512-key block (built once, timed), replicated like the key cache, and
    one flat-search call per replica over the step's queries."""

    def __init__(self, S, replicas, p, k, device_mod, torch):
        self.S, self.p, self.k = S, p, k
        self.torch = torch
        self.lsa = device_mod.LsaCache(S.cache)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        self.lsa.build()
        e1.record()
        torch.cuda.synchronize()
        self.build_ms = e0.elapsed_time(e1)
        self.nblk = int(self.lsa.nblk.sum())
        ph = S.phases[0]
        base = device_mod.LsaCall(self.lsa, ph.queries, ph.q_pos, ph.q_seq, p, k, buckets=False)
        self.out_idx = base.out_idx
        self.calls = []
        L = self.lsa
        for r in range(replicas):
            cen = L.centroids if r == 0 else L.centroids.clone()
            mem = L.members if r == 0 else L.members.clone()
            off = L.offs if r == 0 else L.offs.clone()
            a = S.h.make_lsa_args(base.queries, base.q_pos, cen, mem, off, L.d_blk_off, L.d_nblk, S.cache.d_len,
                                  base.max_len, p, k, q_seq=base.q_seq, out_idx=base.out_idx,
                                  workspace=base.workspace)
            self.calls.append((a, cen, mem, off))
        self.base = base
        self.replicas = replicas

    def run(self, r):
        """One decode step: the same key append as the other methods' steps
        (the search does not read the new key until its block completes),
        then the search."""
        S = self.S
        if S.append_src is not None:
            rr = r % S.replicas
            S.h.hisa_append_keys(S.keys[rr], S.reps[rr], S.seqs, S.append_src, S.B)
        S.h.hisa_lsa_index(self.calls[r % self.replicas][0])

    def time_steps(self, steps, warmup):
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.run(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        n = max(self.replicas, self.S.replicas)
        for r in range(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.run(r)
            graphs.append(g)
        for i in range(warmup):
            graphs[i % n].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            graphs[(warmup + i) % n].replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e3


def attention_kernel_ms(S, A, nsteps, torch):
    """Average duration of the attention call (both of its kernels), from
    torch events on the stream it runs on, queued behind a sleep kernel so
    the calls run back to back; inputs are one HISA step's indices."""
    S.step(0, False, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nsteps)]
    torch.cuda._sleep(int(2.0e7))
    for i in range(nsteps):
        ev[i][0].record()
        A.run(i, False)
        ev[i][1].record()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


STEPS_PER_GRAPH = 1


def capture_graphs(S, flat, torch, attn=None):
    """One HIP graph per replica holding one whole step (kernels only: no
    events, no allocation, no memset nodes), followed by the sparse
    attention over its output when attn is given.  With STEPS_PER_GRAPH > 1
    a graph holds that many consecutive steps (on consecutive replicas)."""
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                   # warm the path once outside capture
        S.step(0, flat, side.cuda_stream)
        if attn is not None:
            attn.run(0, flat)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(S.replicas):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for j in range(STEPS_PER_GRAPH):
                rr = (r + j) % S.replicas
                S.step(rr, flat, torch.cuda.current_stream().cuda_stream)
                if attn is not None:
                    attn.run(rr, flat)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def time_method(S, flat, steps, warmup, torch, attn=None):
    """Wall time of `steps` graph replays (one step each, rotating over the
    replicas), bracketed by device synchronisation."""
    graphs = capture_graphs(S, flat, torch, attn)
    spg = STEPS_PER_GRAPH
    n = max(1, steps // spg)                # replays of spg steps each, consecutive replays on fresh replicas
    for i in range(max(1, warmup // spg)):
        graphs[(i * spg) % S.replicas].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        graphs[((warmup + i) * spg) % S.replicas].replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * steps / (n * spg)


def stage_times(S, flat, nsteps, torch):
    """Average duration of every stage over `nsteps` eager steps, from the
    start / stop HIP events the library records with each stage's kernel
    dispatches (the kernels' own execution time).  A sleep kernel holds the
    GPU while the host queues the steps, so the kernels run back to back as
    in the graph-replayed steps."""
    h = S.h
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    nph = len(S.phases)
    evs = [[h.StageEvents() for _ in range(nph)] for _ in range(nsteps)]
    hr = h._hiprt()
    app = []
    if S.append_src is not None and (flat or not S.fused_step):
        for _ in range(nsteps):
            pair = []
            for _ in range(2):
                e = ctypes.c_void_p()
                hr.hipEventCreate(ctypes.byref(e))
                pair.append(e)
            app.append(pair)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2.0e7))                   # ~10 ms of spinning while the host queues
    for i in range(nsteps):
        S.step(i % S.replicas, flat, sp, evs[i], app[i] if app else None)
    torch.cuda.synchronize()
    out = {}
    for p in range(nph):
        ph = S.phases[p]
        names = dict(enumerate(STAGES_FLAT)) if flat else hisa_stage_names(len(ph.q_pos), S.max_len, S.B)
        for s_, nm in names.items():
            vals = [evs[i][p].stage_ms(s_) for i in range(nsteps)]
            out["%s/%s" % (S.phases[p].name, nm)] = float(np.mean(vals))
    if app:
        vals = []
        for a0, a1 in app:
            f = ctypes.c_float()
            hr.hipEventElapsedTime(ctypes.byref(f), a0, a1)
            vals.append(f.value)
            hr.hipEventDestroy(a0)
            hr.hipEventDestroy(a1)
        out["append"] = float(np.mean(vals))
    return out


def row_overlap(a, b):
    """Mean over rows of |A & F| / |A | F| and of |A & F| / |F| for index
    rows a (a method) and b (the flat indexer), -1 entries ignored."""
    iou, rec = [], []
    for x, y in zip(a, b):
        x = x[x >= 0]
        y = y[y >= 0]
        inter = len(np.intersect1d(x, y, assume_unique=True))
        union = len(x) + len(y) - inter
        iou.append(inter / union if union else 1.0)
        rec.append(inter / len(y) if len(y) else 1.0)
    return float(np.mean(iou)), float(np.mean(rec))


def sweep_m(S, ms, steps, warmup, torch):
    """HISA at each m (k fixed) and block-only selection at the same token
    budget (m = k/B) and at HISA's candidate set (the workload's m): time
    per step (graph replays) and overlap with the flat indexer's rows."""
    sp = torch.cuda.current_stream().cuda_stream
    nrow = 1024                                      # rows compared (evenly spaced)

    def rows_of(calls):
        out = []
        for ic, _ in calls:
            n = ic.out_idx.shape[0]
            pick = np.unique(np.linspace(0, n - 1, min(n, nrow)).astype(np.int64))
            out.append(ic.out_idx[torch.from_numpy(pick).to(ic.out_idx.device)].cpu().numpy())
        return np.concatenate(out)

    f_ms = time_method(S, True, steps, warmup, torch) / steps * 1e3
    S.step(0, True, sp)
    torch.cuda.synchronize()
    flat_rows = rows_of(S.calls[True])
    base = S.calls[False]
    points = []
    variants = [(False, m, S.k) for m in ms if m * S.B >= S.k and m * S.B <= 16384]
    variants += [(True, mb, mb * S.B) for mb in sorted({S.k // S.B, S.m}) if mb >= 3]
    for block_only, m, k in variants:
        log("sweep: %s m=%d k=%d" % ("block-only" if block_only else "hisa", m, k))
        S.calls[False] = S.build_calls(False, m, k, block_only=block_only)
        S.block_only = block_only
        ms_step = time_method(S, False, steps, warmup, torch) / steps * 1e3
        S.step(0, False, sp)
        torch.cuda.synchronize()
        iou, rec = row_overlap(rows_of(S.calls[False]), flat_rows)
        points.append({"method": "block_only" if block_only else "hisa", "m": m, "k": k, "ms_per_step": ms_step,
                       "speedup_vs_flat": f_ms / ms_step, "iou_vs_flat": iou, "recall_of_flat_topk": rec})
    S.calls[False] = base
    S.block_only = False
    return f_ms, points


def cpu_baseline(S, seconds, oracle):
    """The oracle on the same step, repeated for about `seconds`."""
    w = S.w
    B, m, k = S.B, S.m, S.k
    lens = S.cache.seq_len
    reps = np.zeros((w.total_rep_rows(B), 64), np.uint16)
    rep_off = w.seq_rep_off(B)
    for s in range(w.nseq):
        o = int(w.seq_key_off[s])
        r = oracle.pool(w.keys[o:o + int(lens[s])], B)
        reps[rep_off[s]:rep_off[s] + len(r)] = r
    # prefill steps are far beyond a few seconds of CPU work: time an evenly
    # spaced sample of at most 256 queries per phase instead
    sample = []
    for ph in S.phases:
        nq = len(ph.q_pos)
        pick = np.unique(np.linspace(0, nq - 1, min(nq, 256)).astype(np.int64))
        sample.append((ph, pick))
    nsample = sum(len(p) for _, p in sample)
    n = 0
    t0 = time.perf_counter()
    while True:
        if S.append_src is not None:                   # re-pool the blocks the append touches
            n_new = S.append_src.shape[1]
            for s in range(w.nseq):
                o = int(w.seq_key_off[s])
                L = int(lens[s])
                oracle.pool_range(w.keys[o:o + L], B, (L - n_new) // B, (L + B - 1) // B,
                                  reps[rep_off[s]:rep_off[s] + (L + B - 1) // B])
        for ph, pick in sample:
            oracle.index_batch(False, ph.queries[pick], ph.q_pos[pick], w.keys, k, reps=reps,
                               q_seq=ph.q_seq[pick], seq_key_off=w.seq_key_off, seq_rep_off=rep_off,
                               seq_len=lens, B=B, m=m)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    whole = nsample == S.q_per_step
    what = ("the whole step" if whole else "%d evenly spaced queries of the step" % nsample)
    return {"value": n * nsample / el, "unit": "queries/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": "%d repetitions of %s (%s), HISA oracle, %.1f s" % (n, what, S.desc, el)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_32k_x16", choices=WORKLOADS)
    ap.add_argument("--replicas", type=int, default=None,
                    help="key-cache copies rotated over (default: enough to exceed the 256 MB cache)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--stage-steps", type=int, default=32,
                    help="eager steps whose stages are timed with HIP events")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-attention", action="store_true", help="skip the sparse-attention leg")
    ap.add_argument("--no-lsa", action="store_true", help="skip the LSA-Flat leg")
    ap.add_argument("--steps-per-graph", type=int, default=1,
                    help="consecutive steps captured in one graph (1: one replay per step, the serving form)")
    ap.add_argument("--lsa-replicas", type=int, default=8, help="copies of the LSA bucket cache rotated over")
    ap.add_argument("--sweep-m", default=None, metavar="M1,M2,...",
                    help="instead of the default line: HISA at each m and block-only selection, time per "
                         "step and overlap with the flat indexer's rows")
    ap.add_argument("--attn-replicas", type=int, default=8,
                    help="copies of the attention keys and values rotated over")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device (a known-size reference for HBM counters)")
    args = ap.parse_args()
    global STEPS_PER_GRAPH
    STEPS_PER_GRAPH = max(1, args.steps_per_graph)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the indexer here runs on a single MI355X and has no "
              "multi-GPU path (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from long_context_sparse_hisa_amd import device, hisa, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, dtype=torch.int32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 3}), flush=True)
        return
    hisa.lib()
    # replicas rotate about 4 GiB of keys so the 256 MB MALL cannot serve
    # repeated decode steps
    default_rep = {"decode_32k_x16": 64, "decode_32k_x64": 16, "decode_32k_x256": 4, "long_decode_1m": 256,
                   "decode_varlen_x64": 16,
                   "chunked_prefill_32k": 1, "long_context_128k": 1, "tiny_prefill_4k": 1}
    R = args.replicas or default_rep[args.workload]
    log("setting up %s with %d replicas" % (args.workload, R))
    S = Setup(args.workload, R, hisa, synth, device, torch)
    if args.sweep_m:
        ms = [int(x) for x in args.sweep_m.split(",")]
        f_ms, points = sweep_m(S, ms, args.steps, args.warmup, torch)
        print(json.dumps({"metric": "HISA m-sweep: ms per step and overlap with the flat indexer's top-k rows",
                          "workload": args.workload, "description": S.desc, "n_gpus": 1, "steps": args.steps,
                          "replicas": R, "B": S.B, "k": S.k, "flat_ms_per_step": f_ms,
                          "overlap": "iou = mean |A & F| / |A | F|, recall = mean |A & F| / |F| over up to "
                                     "1024 evenly spaced rows per phase, F the flat indexer's row",
                          "points": points}), flush=True)
        return
    log("timing HISA: %d warmup + %d graph-replayed steps" % (args.warmup, args.steps))
    h_el = time_method(S, False, args.steps, args.warmup, torch)
    two_ms = None
    if S.fused_step:
        log("timing HISA as two calls (append, then index)")
        S.fused_step = False
        two_ms = time_method(S, False, args.steps, args.warmup, torch) / args.steps * 1e3
        S.fused_step = True
    log("timing flat: %d warmup + %d graph-replayed steps" % (args.warmup, args.steps))
    f_el = time_method(S, True, args.steps, args.warmup, torch)
    nst = max(4, min(args.stage_steps, S.replicas * 4))
    log("per-stage HIP-event timing over %d eager steps each" % nst)
    h_stage = stage_times(S, False, nst, torch)
    f_stage = stage_times(S, True, nst, torch)
    h_ms = h_el / args.steps * 1e3
    f_ms = f_el / args.steps * 1e3
    qps = S.q_per_step * args.steps / h_el
    fqps = S.q_per_step * args.steps / f_el

    # roofline of the dominant HISA kernel
    stage_bytes = {}
    for ph in S.phases:
        for nm, b in hisa_stage_bytes(ph.q_pos, S.B, S.m, S.k).items():
            stage_bytes["%s/%s" % (ph.name, nm)] = b
        for nm, b in flat_stage_bytes(ph.q_pos, S.k).items():
            stage_bytes["%s/%s" % (ph.name, nm)] = b
    stage_fl, stage_nq = {}, {}
    for ph in S.phases:
        for nm, f in stage_flops(ph.q_pos, S.B, S.m).items():
            stage_fl["%s/%s" % (ph.name, nm)] = f
            stage_nq["%s/%s" % (ph.name, nm)] = len(ph.q_pos)
    if S.fused_step:
        # the decode step's launch also appends: new rows written, touched
        # blocks read, their representatives written
        n_new = S.append_src.shape[1]
        blocks = sum((int(sq[2]) + n_new - 1) // S.B - int(sq[2]) // S.B + 1 for sq in S.seqs)
        app_bytes = len(S.seqs) * n_new * 128 + blocks * (S.B * 128 + 128)
        for n in list(stage_bytes):
            if n.endswith("/select_and_scores"):
                stage_bytes[n] += app_bytes
    kern = max((n for n in h_stage if n in stage_bytes), key=lambda n: h_stage[n])
    bound, achieved, peak, unit, work = stage_roofline(kern, h_stage[kern], stage_nq.get(kern, 0),
                                                       stage_fl.get(kern, 0.0), stage_bytes[kern])
    fkern = max((n for n in f_stage if n in stage_bytes), key=lambda n: f_stage[n])
    fbound, f_achieved, fpeak, funit, _ = stage_roofline(fkern, f_stage[fkern], stage_nq.get(fkern, 0),
                                                         stage_fl.get(fkern, 0.0), stage_bytes[fkern])
    # algorithmic bytes of a whole step: every stage's per-query traffic
    # (no workspace round trips) plus the append (new rows written, touched
    # blocks re-read, representatives written)
    append_rows = 0 if S.append_src is None else S.append_src.shape[0] * S.append_src.shape[1]
    h_step_bytes = sum(b for n, b in stage_bytes.items() if n.split("/")[-1] in ("block_stage", "token_ideal"))
    f_step_bytes = sum(b for n, b in stage_bytes.items() if n.split("/")[-1] in STAGES_FLAT)
    h_step_bytes += append_rows * 128 * 2
    f_step_bytes += append_rows * 128 * 2

    def per_kernel(stage):
        return {n: {"avg_ms": v, "algorithmic_bytes": stage_bytes.get(n),
                    "gbps": (stage_bytes[n] / (v * 1e-3) / 1e9) if n in stage_bytes and v > 0 else None}
                for n, v in stage.items()}

    attention = None
    if args.workload in ATTN_WORKLOADS and not args.no_attention:
        log("attention leg: inputs and %d replicas" % args.attn_replicas)
        A = AttentionLeg(S, args.attn_replicas, device, synth, torch)
        a_ms = attention_kernel_ms(S, A, max(8, nst), torch)
        n_valid = int((A.calls[False][0].idx >= 0).sum().item())
        a_bytes = A.algorithmic_bytes(n_valid)
        log("timing index + attention steps (HISA, flat)")
        ha_ms = time_method(S, False, args.steps, args.warmup, torch, A) / args.steps * 1e3
        fa_ms = time_method(S, True, args.steps, args.warmup, torch, A) / args.steps * 1e3
        a_gbps = a_bytes / (a_ms * 1e-3) / 1e9
        attention = {"description": A.desc, "kernels": "attn_partial_kernel + attn_combine_kernel",
                     "avg_call_ms": a_ms, "algorithmic_bytes": a_bytes, "gbps": a_gbps,
                     "frac_of_hbm_peak": a_gbps / HBM_PEAK_GBPS,
                     "ms_per_step_hisa_plus_attention": ha_ms, "ms_per_step_flat_plus_attention": fa_ms,
                     "speedup_vs_flat": fa_ms / ha_ms}

    lsa = None
    if args.workload in LSA_WORKLOADS and not args.no_lsa:
        p_l, k_l = LSA_WORKLOADS[args.workload]
        log("LSA-Flat leg: build and %d replicas (p=%d, k=%d)" % (args.lsa_replicas, p_l, k_l))
        Lg = LsaLeg(S, args.lsa_replicas, p_l, k_l, device, torch)
        l_ms = Lg.time_steps(args.steps, args.warmup)
        Lg.run(0)
        S.step(0, True, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        f_rows = S.calls[True][0][0].out_idx.cpu().numpy()
        l_rows = Lg.out_idx.cpu().numpy()
        S.step(0, False, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        h_rows = S.calls[False][0][0].out_idx.cpu().numpy()
        l_iou, l_rec = row_overlap(l_rows, f_rows)
        h_iou, h_rec = row_overlap(h_rows, f_rows)
        per_block_us = Lg.build_ms * 1e3 / max(Lg.nblk, 1)
        lsa = {"description": "LSA-Flat on the same keys and queries: 64 buckets per complete 512-key block "
                              "(Ward, fp64), p=%d buckets searched, k=%d keys; %d replicas of the bucket cache"
                              % (p_l, k_l, args.lsa_replicas),
               "ms_per_step": l_ms, "speedup_vs_flat": f_ms / l_ms, "vs_hisa": h_ms / l_ms,
               "build_ms": Lg.build_ms, "blocks_built": Lg.nblk, "build_us_per_block": per_block_us,
               "build_us_per_decode_step_amortized": per_block_us * S.cache.nseq / 512.0,
               "iou_vs_flat": l_iou, "recall_of_flat_topk": l_rec,
               "hisa_iou_vs_flat": h_iou, "hisa_recall_of_flat_topk": h_rec,
               "note": "a step is the same key append as HISA's and flat's steps, then the search; a sequence "
                       "completes a block every 512 decode steps, so the build adds "
                       "build_us_per_decode_step_amortized per step"}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("timing the CPU oracle for about %.0f s" % args.cpu_seconds)
        cpu = cpu_baseline(S, args.cpu_seconds, oracle)

    out = {
        "metric": "indexer queries/s + HBM GB/s at 32K/128K/1M ctx; HISA vs flat-DSA speedup",
        "value": qps,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "description": S.desc, "queries_per_step": S.q_per_step,
                   "outputs": "int32 top-k indices (the optional scores and kept-block lists are not requested)",
                   "replicas": R, "B": S.B, "m": S.m, "k": S.k},
        "roofline": {"bound": bound, "kernel": kern, "achieved": achieved, "peak": peak,
                     "unit": unit, "frac": achieved / peak,
                     "traffic": measured_traffic(os.path.dirname(os.path.abspath(__file__)), args.workload, kern,
                                                 fused_step=S.fused_step),
                     ("algorithmic_flops_per_launch" if bound == "mfma" else "algorithmic_bytes_per_launch"): work,
                     "avg_launch_ms": h_stage[kern]},
        "cpu_baseline": cpu,
        "step_bytes": h_step_bytes,
        "hbm_gbps_step": h_step_bytes / (h_ms * 1e-3) / 1e9,
        "kernels": per_kernel(h_stage),
        "flat": {"value": fqps, "unit": "queries/s", "ms_per_step": f_ms, "kernels": per_kernel(f_stage),
                 "step_bytes": f_step_bytes,
                 "hbm_gbps_step": f_step_bytes / (f_ms * 1e-3) / 1e9,
                 "dominant": {"kernel": fkern, "bound": fbound, "achieved": f_achieved, "unit": funit,
                              "frac": f_achieved / fpeak}},
        "speedup_vs_flat": f_ms / h_ms,
        "hisa_two_calls_ms_per_step": two_ms,
        "step_note": ("HISA decode steps are one hisa_decode_step call (the append in the same launch as the block "
                      "selection and token scores); hisa_two_calls_ms_per_step is the same step as append + index, "
                      "the form the flat indexer's step takes" if two_ms is not None else None),
        "attention": attention,
        "lsa_flat": lsa,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
