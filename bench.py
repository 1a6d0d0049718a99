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

Each method's steps are timed in two launch forms and the faster counts,
for HISA and flat alike: eager, the library calls queued back to back on
one stream with the host ahead of the GPU (the GPU sets the pace when it is
the slower side), and one captured HIP graph replayed per step (which wins
where a call's host work outweighs its kernels); `--launch eager|graph`
times one form only.  Per-kernel durations come
from HIP start / stop events attached to the kernel dispatches of a
separate run of eager steps (queued behind a sleep kernel so they run back
to back); the roofline object is computed from the kernel with the largest
average duration.
"""
from __future__ import annotations

import argparse
import contextlib
import ctypes
import gc
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
DECODE_FOLD_MAX_SEQS = 64       # a decode step folds its append into the first launch for this many sequences


def hisa_stage_names(nq, max_len, B):
    """Stage index -> name for one HISA call (the library's stage events)."""
    if nq < SPLIT_BELOW and (max_len + B - 1) // B <= FUSED_MAX_BLOCKS:
        return {1: "select_and_scores", 2: "token_topk"}
    return dict(enumerate(STAGES_HISA))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---- algorithmic traffic per stage ------------------------------------------------

def visible_candidates(q_pos, B, m):
    """Candidate tokens a query at t scores: every causal key when all its
    causal blocks are kept, otherwise m-1 whole earlier blocks and the
    t % B + 1 visible keys of its own block (always kept)."""
    q_pos = np.asarray(q_pos, np.int64)
    nb = q_pos // B + 1
    return np.where(nb <= m, q_pos + 1, (m - 1) * B + q_pos % B + 1)


def hisa_stage_bytes(q_pos, B, m, k):
    """Algorithmic HBM bytes of the HISA stages for queries at q_pos (d = 64:
    a key or representative row is 128 bytes): inputs read once and the
    call's required output, no workspace traffic (kept-block lists and
    candidate scores passed between kernels are not counted).  Block stage:
    the query and its causal representatives.  Token stage: the query and
    the candidate keys of its kept blocks.  Top-k: the int32 indices out."""
    q_pos = np.asarray(q_pos, np.int64)
    nb = q_pos // B + 1                                  # causal blocks
    cand = visible_candidates(q_pos, B, m)                # <= m*B candidate tokens
    block = (128 + nb * 128).sum()
    token = (128 + cand * 128).sum()
    out = len(q_pos) * k * 4
    return {
        "block_stage": float(block),
        "token_scores": float(token),
        "token_topk": float(out),
        # stage 1 and the token scores as one kernel (few queries): the
        # query once, its representatives and its candidate keys
        "select_and_scores": float(block + (cand * 128).sum()),
        # the whole path of these queries
        "token_ideal": float(block + (cand * 128).sum() + out),
    }


def stage_flops(q_pos, B, m):
    """Algorithmic flops of the contractions: 2*64 per (query, row) pair
    over the causal representatives (block stage), the visible candidates
    of the kept blocks (token stage) and every visible key (flat scores)."""
    q_pos = np.asarray(q_pos, np.int64)
    nb = q_pos // B + 1
    cand = visible_candidates(q_pos, B, m)
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
    """Flat: the scores stage reads the query and every visible key; the
    top-k stage writes the int32 indices (the score rows between them are
    workspace traffic, not counted)."""
    q_pos = np.asarray(q_pos, np.int64)
    n = q_pos + 1
    return {
        "flat_scores": float((n * 128 + 128).sum()),
        "flat_topk": float(len(n) * k * 4),
    }


# ---- measured HBM traffic ----------------------------------------------------------

# kernel symbol that carries each stage
STAGE_KERNEL = {"block_stage": ("stage1_select_kernel", "stage1_select_many_kernel", "stage1_tile_kernel",
                                "block_select_tile_kernel", "block_score"),
                "token_scores": ("select_score_kernel", "stage2_tile_kernel", "stage2_gather_kernel"),
                "token_topk": ("topk_rows_kernel", "topk_rows_many_kernel"),
                "select_and_scores": ("decode_fused_kernel", "decode_step_kernel"),
                "flat_scores": ("flat_score_kernel", "flat_score_mfma_kernel")}


def stream_ceiling(n, torch, reps=20):
    """HBM bandwidth of plain streaming kernels over n bytes, timed with HIP
    events on torch's stream (launch cost is negligible at this size): full
    reads (a sum, a maximum and a matrix-vector product over n bytes of
    float32), a device-to-device copy and an elementwise dst = src + 1 (n
    read + n written each), and a fill (n written)."""
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    mat = src.view(-1, 4096)
    vec = torch.ones(4096, dtype=torch.float32, device="cuda:0")
    out = {"bytes": n, "repeats": reps, "peak_gbps": HBM_PEAK_GBPS}
    for name, fn, moved in (("read_sum", lambda: src.sum(), n), ("read_amax", lambda: src.amax(), n),
                            ("read_gemv", lambda: torch.mv(mat, vec), n),
                            ("copy", lambda: dst.copy_(src), 2 * n),
                            ("add_one", lambda: torch.add(src, 1.0, out=dst), 2 * n),
                            ("write_fill", lambda: dst.fill_(2.0), n)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"ms": ms, "gbps": moved / ms / 1e6, "frac": moved / ms / 1e6 / HBM_PEAK_GBPS}
    return out


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
            self.seq_arr = hisa_mod.seq_array(self.seqs)      # marshalled once, reused every step
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
            h.hisa_decode_step(a, self.seq_arr, self.append_src, stream)
            return
        if self.append_src is not None:
            if append_events is not None:
                h._hiprt().hipEventRecord(append_events[0], stream)
            h.hisa_append_keys(self.keys[r], self.reps[r], self.seq_arr, self.append_src, self.B, stream)
            if append_events is not None:
                h._hiprt().hipEventRecord(append_events[1], stream)
        for p, (ic, per_rep) in enumerate(self.calls[flat]):
            a = per_rep[r]
            if events is not None:
                events[p].attach(a)
            else:
                a.stage_events = None
            (h.hisa_flat_index if flat else h.hisa_block_index if self.block_only else h.hisa_index)(a, stream)


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
            S.h.hisa_append_keys(S.keys[rr], S.reps[rr], S.seq_arr, S.append_src, S.B)
        S.h.hisa_lsa_index(self.calls[r % self.replicas][0])

    def time_steps(self, steps, warmup):
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.run(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        n = max(self.replicas, self.S.replicas)
        out = []
        if LAUNCH in ("graph", "best"):
            graphs = []
            for r in range(n):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    self.run(r)
                graphs.append(g)
            out.append(replay_timed(graphs, steps, warmup, torch, spg=1) * 1e3)
            del graphs
        if LAUNCH in ("eager", "best"):
            # as eager_timed: every replica once, the warmup, then the timed
            # steps back to back
            for r in range(n):
                self.run(r)
            torch.cuda.synchronize()
            gc.collect()
            for i in range(warmup):
                self.run(i % n)
            torch.cuda.synchronize()
            with no_gc():
                t0 = time.perf_counter()
                for i in range(steps):
                    self.run((warmup + i) % n)
                torch.cuda.synchronize()
                out.append((time.perf_counter() - t0) / steps * 1e3)
        return min(out)


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
# How timed steps are launched: "eager" (each step's calls queued back to
# back on the stream, the host running ahead of the GPU), "graph" (one
# captured HIP graph replayed per step) or "best" (both, the faster counts:
# eager wins where the GPU is the slower side, graphs where the host work
# of a call outweighs its kernels)
LAUNCH = "best"


@contextlib.contextmanager
def no_gc():
    """Python's garbage collector off inside a timed region, so that no
    collection pause lands among the timed steps (callers collect before
    their warmup, which then brings the GPU back to its steady state)."""
    gc.disable()
    try:
        yield
    finally:
        gc.enable()


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


def replay_timed(graphs, steps, warmup, torch, spg=None):
    """Seconds per replay-step over `steps` replays of the captured graphs
    (rotating, consecutive replays on fresh replicas).  Every graph is
    replayed once before the warmup and the timed region, so that no timed
    replay is a graph's first launch (whose upload and first dispatch cost
    more than a steady-state replay)."""
    n = len(graphs)
    spg = STEPS_PER_GRAPH if spg is None else spg
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    gc.collect()
    reps = max(1, steps // spg)
    for i in range(max(1, warmup // spg)):
        graphs[i % n].replay()
    torch.cuda.synchronize()
    with no_gc():
        t0 = time.perf_counter()
        for i in range(reps):
            graphs[(warmup // spg + i) % n].replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / (reps * spg)


def eager_timed(S, flat, steps, warmup, torch, attn=None):
    """Seconds per step over `steps` steps whose calls are queued back to
    back on the current stream (rotating over the replicas; the host runs
    ahead of the GPU, so the GPU sets the pace when it is the slower side).
    Every replica takes one step before the warmup and the timed region, so
    that no timed step is the first on its replica."""
    st = torch.cuda.current_stream().cuda_stream

    def one(r):
        S.step(r, flat, st)
        if attn is not None:
            attn.run(r, flat)

    for r in range(S.replicas):
        one(r)
    torch.cuda.synchronize()
    gc.collect()
    for i in range(warmup):
        one(i % S.replicas)
    torch.cuda.synchronize()
    with no_gc():
        t0 = time.perf_counter()
        for i in range(steps):
            one((warmup + i) % S.replicas)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps


def time_forms(S, flat, steps, warmup, torch, attn=None, launch=None):
    """{launch form: milliseconds per step}, rotating over the replicas,
    bracketed by device synchronisation, for the forms `launch` (default
    LAUNCH) asks for: eager steps queued back to back, one graph replay per
    step, or both."""
    mode = launch or LAUNCH
    out = {}
    for form in (("eager", "graph") if mode == "best" else (mode,)):
        if form == "graph":
            graphs = capture_graphs(S, flat, torch, attn)
            out[form] = replay_timed(graphs, steps, warmup, torch) * 1e3
            del graphs
        else:
            out[form] = eager_timed(S, flat, steps, warmup, torch, attn) * 1e3
    return out


def time_method(S, flat, steps, warmup, torch, attn=None, launch=None):
    """Milliseconds per step in the faster of the launch forms asked for."""
    return min(time_forms(S, flat, steps, warmup, torch, attn, launch).values())


def stage_times(S, flat, nsteps, torch):
    """Average duration of every stage over `nsteps` eager steps, from the
    start / stop HIP events the library records with each stage's kernel
    dispatches (the kernels' own execution time).  A sleep kernel holds the
    GPU while the host queues the steps, so the kernels run back to back as
    in the timed steps."""
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
    per step and overlap with the flat indexer's rows."""
    sp = torch.cuda.current_stream().cuda_stream
    nrow = 1024                                      # rows compared (evenly spaced)

    def rows_of(calls):
        out = []
        for ic, _ in calls:
            n = ic.out_idx.shape[0]
            pick = np.unique(np.linspace(0, n - 1, min(n, nrow)).astype(np.int64))
            out.append(ic.out_idx[torch.from_numpy(pick).to(ic.out_idx.device)].cpu().numpy())
        return np.concatenate(out)

    f_ms = time_method(S, True, steps, warmup, torch)
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
        ms_step = time_method(S, False, steps, warmup, torch)
        S.step(0, False, sp)
        torch.cuda.synchronize()
        iou, rec = row_overlap(rows_of(S.calls[False]), flat_rows)
        points.append({"method": "block_only" if block_only else "hisa", "m": m, "k": k, "ms_per_step": ms_step,
                       "speedup_vs_flat": f_ms / ms_step, "iou_vs_flat": iou, "recall_of_flat_topk": rec})
    S.calls[False] = base
    S.block_only = False
    return f_ms, points


def oracle_rate(w, lens, n_new, B, m, k, flat, seconds, oracle, max_q=256):
    """Queries per second of the oracle on the phases of workload w (keys
    of sequence s: the first lens[s] rows at w.seq_key_off[s]), repeated
    for about `seconds`.  A phase of more than max_q queries is sampled
    (evenly spaced queries).  n_new > 0: every repetition first re-pools
    the blocks the step's append touched, as the step does.  Returns
    (queries/s, repetitions, queries per repetition, whether the sample is
    the whole step, seconds)."""
    reps = None
    if not flat:
        reps = np.zeros((w.total_rep_rows(B), 64), np.uint16)
        rep_off = w.seq_rep_off(B)
        for s in range(w.nseq):
            o = int(w.seq_key_off[s])
            r = oracle.pool(w.keys[o:o + int(lens[s])], B)
            reps[rep_off[s]:rep_off[s] + len(r)] = r
    else:
        rep_off = None
    sample = []
    for ph in w.phases:
        nq = len(ph.q_pos)
        pick = np.unique(np.linspace(0, nq - 1, min(nq, max_q)).astype(np.int64))
        sample.append((ph, pick))
    nsample = sum(len(p) for _, p in sample)
    whole = nsample == sum(len(ph.q_pos) for ph in w.phases)
    n = 0
    t0 = time.perf_counter()
    while True:
        if n_new and not flat:                          # re-pool the blocks the append touches
            for s in range(w.nseq):
                o = int(w.seq_key_off[s])
                L = int(lens[s])
                oracle.pool_range(w.keys[o:o + L], B, (L - n_new) // B, (L + B - 1) // B,
                                  reps[rep_off[s]:rep_off[s] + (L + B - 1) // B])
        for ph, pick in sample:
            oracle.index_batch(flat, ph.queries[pick], ph.q_pos[pick], w.keys, k, reps=reps,
                               q_seq=ph.q_seq[pick], seq_key_off=w.seq_key_off, seq_rep_off=rep_off,
                               seq_len=lens, B=B, m=m)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return n * nsample / el, n, nsample, whole, el


def host_facts():
    """The host the oracle runs on: logical CPUs, the ones this process may
    use, the CPU model and OMP_NUM_THREADS."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"nproc": os.cpu_count(), "usable_cpus": usable, "cpu_model": model,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def cpu_baseline(S, seconds, oracle, extras=True):
    """The oracle (HISA) on the same step, repeated for about `seconds`;
    with extras also the flat oracle on the same sample and the HISA
    oracle on one core over the 4K tiny prefill."""
    n_new = 0 if S.append_src is None else int(S.append_src.shape[1])
    w = S.w
    w_ph = w.phases
    w.phases = S.phases
    try:
        v, n, nsample, whole, el = oracle_rate(w, S.cache.seq_len, n_new, S.B, S.m, S.k, False, seconds, oracle)
        what = ("the whole step" if whole else "%d evenly spaced queries of the step" % nsample)
        out = {"value": v, "unit": "queries/s", "cores": oracle.threads(), "kind": "oracle",
               "sample": "%d repetitions of %s (%s), HISA oracle, %.1f s" % (n, what, S.desc, el)}
        out.update(host_facts())
        if extras:
            fv, fn, fns, fwhole, fel = oracle_rate(w, S.cache.seq_len, 0, S.B, S.m, S.k, True,
                                                   max(1.0, seconds / 3), oracle)
            out["flat_oracle"] = {"value": fv, "unit": "queries/s", "cores": oracle.threads(),
                                  "sample": "%d repetitions of the same %d queries, %.1f s" % (fn, fns, fel)}
    finally:
        w.phases = w_ph
    if extras:
        from long_context_sparse_hisa_amd import synth
        tw = synth.tiny_prefill()
        oracle.set_threads(1)
        try:
            tv, tn, tns, _, tel = oracle_rate(tw, tw.seq_len, 0, tw.B, tw.m, tw.k, False, max(1.0, seconds / 3),
                                              oracle)
        finally:
            oracle.set_threads(out["cores"])
        out["one_core_tiny_prefill_4k"] = {
            "value": tv, "unit": "queries/s", "cores": 1,
            "sample": "%d repetitions of %d evenly spaced queries of the 4096-query causal prefill (4096 i.i.d. "
                      "N(0,1) keys, B=128 m=8 k=256), HISA oracle, %.1f s" % (tn, tns, tel)}
    return out


def measure(S, args, torch, label):
    """Time HISA and the flat indexer on setup S: timed steps (HISA's
    decode steps also as two calls), per-kernel event times, the
    roofline of each method's dominant kernel and the step's algorithmic
    bytes.  Returns the summary dict."""
    log("%s: timing HISA: %d warmup + %d steps (launch: %s)" % (label, args.warmup, args.steps, LAUNCH))
    h_forms = time_forms(S, False, args.steps, args.warmup, torch)
    h_ms = min(h_forms.values())
    two_ms = None
    if S.fused_step:
        log("%s: timing HISA as two calls (append, then index)" % label)
        S.fused_step = False
        two_ms = time_method(S, False, args.steps, args.warmup, torch)
        S.fused_step = True
    log("%s: timing flat: %d warmup + %d steps (launch: %s)" % (label, args.warmup, args.steps, LAUNCH))
    f_forms = time_forms(S, True, args.steps, args.warmup, torch)
    f_ms = min(f_forms.values())
    nst = max(4, min(args.stage_steps, S.replicas * 4))
    log("%s: per-stage HIP-event timing over %d eager steps each" % (label, nst))
    h_stage = stage_times(S, False, nst, torch)
    h_stage_two = None
    if S.fused_step:
        # the append and the index kernels apart: the two-call form
        S.fused_step = False
        h_stage_two = stage_times(S, False, nst, torch)
        S.fused_step = True
    f_stage = stage_times(S, True, nst, torch)
    qps = S.q_per_step / (h_ms * 1e-3)
    fqps = S.q_per_step / (f_ms * 1e-3)

    stage_bytes = {}
    for ph in S.phases:
        for nm, b in hisa_stage_bytes(ph.q_pos, S.B, S.m, S.k).items():
            stage_bytes["%s/%s" % (ph.name, nm)] = b
        for nm, b in flat_stage_bytes(ph.q_pos, S.k).items():
            stage_bytes["%s/%s" % (ph.name, nm)] = b
    stage_fl, stage_nq, stage_pairs = {}, {}, {}
    for ph in S.phases:
        fl = stage_flops(ph.q_pos, S.B, S.m)
        for nm, f in fl.items():
            stage_fl["%s/%s" % (ph.name, nm)] = f
            stage_nq["%s/%s" % (ph.name, nm)] = len(ph.q_pos)
        # (query, row) pairs each stage works through: causal representatives,
        # kept candidates, every visible key
        cand, vis = fl["token_scores"] / 128, fl["flat_scores"] / 128
        for nm, v in (("block_stage", fl["block_stage"] / 128), ("token_scores", cand), ("select_and_scores", cand),
                      ("token_topk", cand), ("flat_scores", vis), ("flat_topk", vis)):
            stage_pairs["%s/%s" % (ph.name, nm)] = v
    # the append: the new rows read and written, the touched blocks' other
    # rows read, their representatives written
    app_bytes = 0
    if S.append_src is not None:
        n_new = S.append_src.shape[1]
        for sq in S.seqs:
            L0 = int(sq[2])
            b0, b1 = L0 // S.B, (L0 + n_new - 1) // S.B
            old_rows = L0 - b0 * S.B                       # rows of the first touched block already there
            app_bytes += 2 * n_new * 128 + old_rows * 128 + (b1 - b0 + 1) * 128
    if S.fused_step and S.cache.nseq <= DECODE_FOLD_MAX_SEQS:
        # the decode step's first launch also runs the append (the library
        # folds it for up to 64 sequences; beyond, the append is a launch
        # of its own inside the same call)
        for n in list(stage_bytes):
            if n.endswith("/select_and_scores") or (n.endswith("/block_stage") and S.max_len // S.B > 2048):
                stage_bytes[n] += app_bytes
    kern = max((n for n in h_stage if n in stage_bytes), key=lambda n: h_stage[n])
    bound, achieved, peak, unit, work = stage_roofline(kern, h_stage[kern], stage_nq.get(kern, 0),
                                                       stage_fl.get(kern, 0.0), stage_bytes[kern])
    fkern = max((n for n in f_stage if n in stage_bytes), key=lambda n: f_stage[n])
    fbound, f_achieved, fpeak, funit, fwork = stage_roofline(fkern, f_stage[fkern], stage_nq.get(fkern, 0),
                                                             stage_fl.get(fkern, 0.0), stage_bytes[fkern])
    # algorithmic bytes of a whole step: every query's representatives,
    # candidate keys and output, plus the append
    h_step_bytes = sum(b for n, b in stage_bytes.items() if n.endswith("/token_ideal")) + app_bytes
    f_step_bytes = sum(b for n, b in stage_bytes.items() if n.split("/")[-1] in STAGES_FLAT) + app_bytes

    def per_kernel(stage):
        out = {}
        for n, v in stage.items():
            b = app_bytes if n == "append" and app_bytes else stage_bytes.get(n)
            p = stage_pairs.get(n)
            out[n] = {"avg_ms": v, "algorithmic_bytes": b, "gbps": (b / (v * 1e-3) / 1e9) if b and v > 0 else None,
                      "pairs": p, "pairs_per_s": (p / (v * 1e-3)) if p and v > 0 else None}
        return out

    return {
        "workload": S.name, "description": S.desc, "queries_per_step": S.q_per_step, "replicas": S.replicas,
        "B": S.B, "m": S.m, "k": S.k,
        "hisa": {"ms_per_step": h_ms, "launch_forms_ms_per_step": h_forms, "queries_per_s": qps,
                 "step_bytes": h_step_bytes,
                 "hbm_gbps_step": h_step_bytes / (h_ms * 1e-3) / 1e9, "kernels": per_kernel(h_stage),
                 "two_calls_ms_per_step": two_ms,
                 "two_calls_kernels": per_kernel(h_stage_two) if h_stage_two is not None else None},
        "flat": {"ms_per_step": f_ms, "launch_forms_ms_per_step": f_forms, "queries_per_s": fqps,
                 "step_bytes": f_step_bytes,
                 "hbm_gbps_step": f_step_bytes / (f_ms * 1e-3) / 1e9, "kernels": per_kernel(f_stage),
                 "dominant": {"kernel": fkern, "bound": fbound, "achieved": f_achieved, "peak": fpeak,
                              "unit": funit, "frac": f_achieved / fpeak,
                              ("algorithmic_flops_per_launch" if fbound == "mfma" else
                               "algorithmic_bytes_per_launch"): fwork, "avg_launch_ms": f_stage[fkern]}},
        "speedup_vs_flat": f_ms / h_ms,
        "roofline": {"bound": bound, "kernel": kern, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak,
                     ("algorithmic_flops_per_launch" if bound == "mfma" else "algorithmic_bytes_per_launch"): work,
                     "avg_launch_ms": h_stage[kern]},
    }


# The supplementary block-scoring shape: the last 32,768 positions of a
# 1,048,576-key MoG sequence (8,192 blocks of 128), all indexed in one call.
SUPP_L = 1 << 20
SUPP_NQ = 32768
SUPP_SEED = 13


def supplementary_block_scoring(nsteps, torch, hisa_mod, device_mod, synth):
    """Block scoring at 32,768 queries x 8,192 representatives (about 34
    GFLOP of causal pairs), a shape large enough for the matrix-core
    fraction to be read, outside the pages' configurations.  One hisa_index
    call indexes every query (B=128, m=64, k=2048); stage 0 is the
    block scores on the MFMA and the top-m select (two walks over the
    representatives, no score row in memory), timed with the library's
    stage events over `nsteps` eager calls; its fraction counts each causal
    (query, block) pair's 128 flops once, though the two walks issue them
    twice.  No flat indexer: its score rows would take
    128 GiB."""
    pos = np.arange(SUPP_L - SUPP_NQ, SUPP_L, dtype=np.int64)
    w = synth.chunked_prefill(L=SUPP_L, seed=SUPP_SEED, q_positions=pos)
    cache = device_mod.DeviceCache(w)
    cache.pool()
    ph = w.phases[0]
    ic = device_mod.IndexCall(cache, ph.queries, ph.q_pos, ph.q_seq, k=w.k, m=w.m, scores=False, blocks=False,
                              one_chunk_limit=16 << 30)
    ic.run()
    torch.cuda.synchronize()
    evs = [hisa_mod.StageEvents() for _ in range(nsteps)]
    torch.cuda._sleep(int(2.0e7))
    for e in evs:
        e.attach(ic.args)
        ic.run()
    torch.cuda.synchronize()
    ic.args.stage_events = None
    st = {nm: float(np.mean([e.stage_ms(i) for e in evs])) for i, nm in enumerate(STAGES_HISA)}
    flops = stage_flops(pos, w.B, w.m)["block_stage"]
    tflops = flops / (st["block_stage"] * 1e-3) / 1e12
    nvalid = int((ic.out_idx >= 0).sum().item())
    del ic, cache
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"label": "supplementary: not a configuration of the pages",
            "description": "%d queries at positions %d..%d of one %d-key MoG sequence (d=64 bf16; B=%d, so "
                           "8,064-8,192 causal blocks per query), m=%d, k=%d, all in one hisa_index call"
                           % (SUPP_NQ, SUPP_L - SUPP_NQ, SUPP_L - 1, SUPP_L, w.B, w.m, w.k),
            "causal_block_pairs": int((pos // w.B + 1).sum()), "block_flops": flops,
            "stage_ms": st, "call_ms": float(sum(st.values())),
            "block_stage": {"kernels": "block_select_tile_kernel (two bf16 MFMA walks over the representatives, "
                                       "no score row in memory: a per-row threshold, then the exact top-m of the "
                                       "blocks at or above it) + stage1_fixup_kernel (rows that list cannot "
                                       "certify, selected from scratch)",
                            "mfma_flops_issued": 2 * flops,
                            "achieved_tflops": tflops, "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                            "frac": tflops / MFMA_BF16_PEAK_TFLOPS},
            "valid_indices": nvalid, "steps": nsteps}


# workloads reported beside the default one, so that one run covers the
# 32K, 128K and 1M contexts and the large decode batch
CONTEXT_WORKLOADS = ("decode_32k_x256", "chunked_prefill_32k", "long_context_128k", "long_decode_1m")
DEFAULT_REPLICAS = {"decode_32k_x16": 64, "decode_32k_x64": 16, "decode_32k_x256": 4, "long_decode_1m": 256,
                    "decode_varlen_x64": 16, "chunked_prefill_32k": 1, "long_context_128k": 1,
                    "tiny_prefill_4k": 1}


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
    ap.add_argument("--no-contexts", action="store_true",
                    help="only the named workload: skip the 32K x 256, 32K prefill, 128K and 1M workloads "
                         "reported beside the default one, its warm-cache timing and the streaming peak")
    ap.add_argument("--no-supplementary", action="store_true",
                    help="skip the supplementary block-scoring shape (32768 queries x 8192 representatives)")
    ap.add_argument("--supplementary-only", action="store_true",
                    help="only the supplementary block-scoring shape")
    ap.add_argument("--launch", choices=("best", "eager", "graph"), default="best",
                    help="timed steps launched eagerly back to back, as one graph replay per step, or both with "
                         "the faster counted (default)")
    ap.add_argument("--steps-per-graph", type=int, default=1,
                    help="with --launch graph: consecutive steps captured in one graph (1: one replay per step)")
    ap.add_argument("--lsa-replicas", type=int, default=8, help="copies of the LSA bucket cache rotated over")
    ap.add_argument("--sweep-m", default=None, metavar="M1,M2,...",
                    help="instead of the default line: HISA at each m and block-only selection, time per "
                         "step and overlap with the flat indexer's rows")
    ap.add_argument("--attn-replicas", type=int, default=8,
                    help="copies of the attention keys and values rotated over")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device (a known-size reference for HBM counters)")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the warm-cache timing (one replica) of the default workload")
    ap.add_argument("--no-stream-peak", action="store_true",
                    help="skip measuring the plain streaming kernels the HBM rooflines are also compared with")
    ap.add_argument("--stream-ceiling", type=int, default=0, metavar="MIB",
                    help="only time plain streaming kernels over MIB MiB (a full read, a copy): the HBM "
                         "bandwidth simple kernels reach on this GPU, beside the 8 TB/s peak")
    args = ap.parse_args()
    global STEPS_PER_GRAPH, LAUNCH
    STEPS_PER_GRAPH = max(1, args.steps_per_graph)
    LAUNCH = args.launch
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
    if args.stream_ceiling:
        print(json.dumps(stream_ceiling(args.stream_ceiling << 20, torch)), flush=True)
        return
    hisa.lib()
    root = os.path.dirname(os.path.abspath(__file__))
    if args.supplementary_only:
        log("supplementary block-scoring shape: %d queries x %d representatives" % (SUPP_NQ, SUPP_L // 128))
        print(json.dumps(supplementary_block_scoring(max(4, min(args.stage_steps, 8)), torch, hisa, device, synth)),
              flush=True)
        return
    R = args.replicas or DEFAULT_REPLICAS[args.workload]
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
    res = measure(S, args, torch, args.workload)
    h_ms = res["hisa"]["ms_per_step"]
    f_ms = res["flat"]["ms_per_step"]
    roof = dict(res["roofline"])
    roof["traffic"] = measured_traffic(root, args.workload, roof["kernel"], fused_step=S.fused_step)

    attention = None
    if args.workload in ATTN_WORKLOADS and not args.no_attention:
        log("attention leg: inputs and %d replicas" % args.attn_replicas)
        A = AttentionLeg(S, args.attn_replicas, device, synth, torch)
        a_ms = attention_kernel_ms(S, A, max(8, min(args.stage_steps, S.replicas * 4)), torch)
        n_valid = int((A.calls[False][0].idx >= 0).sum().item())
        a_bytes = A.algorithmic_bytes(n_valid)
        log("timing index + attention steps (HISA, flat)")
        ha_ms = time_method(S, False, args.steps, args.warmup, torch, A)
        fa_ms = time_method(S, True, args.steps, args.warmup, torch, A)
        a_gbps = a_bytes / (a_ms * 1e-3) / 1e9
        attention = {"description": A.desc, "kernels": "attn_partial_kernel + attn_combine_kernel",
                     "avg_call_ms": a_ms, "algorithmic_bytes": a_bytes, "gbps": a_gbps,
                     "frac_of_hbm_peak": a_gbps / HBM_PEAK_GBPS,
                     "ms_per_step_hisa_plus_attention": ha_ms, "ms_per_step_flat_plus_attention": fa_ms,
                     "speedup_vs_flat": fa_ms / ha_ms}
        del A

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
        del Lg

    warm = None
    if args.workload == "decode_32k_x16" and R > 1 and not args.no_warm and not args.no_contexts:
        # the same steps on one copy of the key cache (64 MiB), which stays
        # in the 256 MB last-level cache from one step to the next
        log("warm-cache leg: one replica")
        S1 = Setup(args.workload, 1, hisa, synth, device, torch)
        w_h = time_method(S1, False, args.steps, args.warmup, torch)
        w_f = time_method(S1, True, args.steps, args.warmup, torch)
        warm = {"replicas": 1, "hisa_ms_per_step": w_h, "flat_ms_per_step": w_f, "speedup_vs_flat": w_f / w_h,
                "queries_per_s": res["queries_per_step"] / (w_h * 1e-3),
                "note": "one copy of the keys and representatives, resident in the last-level cache across "
                        "steps; the top-level figures are cold (replicas rotated over 4 GiB)"}
        del S1
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("timing the CPU oracle for about %.0f s" % args.cpu_seconds)
        cpu = cpu_baseline(S, args.cpu_seconds, oracle)

    contexts = None
    if args.workload == "decode_32k_x16" and not args.no_contexts:
        contexts = {args.workload: {"hisa_ms_per_step": h_ms, "flat_ms_per_step": f_ms,
                                    "speedup_vs_flat": res["speedup_vs_flat"], "see": "the top-level fields"}}
        del S
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        for name in CONTEXT_WORKLOADS:
            log("setting up %s with %d replicas" % (name, DEFAULT_REPLICAS[name]))
            S2 = Setup(name, DEFAULT_REPLICAS[name], hisa, synth, device, torch)
            r = measure(S2, args, torch, name)
            r["roofline"]["traffic"] = measured_traffic(root, name, r["roofline"]["kernel"],
                                                        fused_step=S2.fused_step)
            if not args.no_cpu_baseline:
                import oracle
                log("%s: timing the CPU oracle for about %.0f s" % (name, max(1.0, args.cpu_seconds / 3)))
                r["cpu_baseline"] = cpu_baseline(S2, max(1.0, args.cpu_seconds / 3), oracle, extras=False)
                r["cpu_baseline"]["flat_oracle"] = None
            contexts[name] = r
            del S2
            torch.cuda.synchronize()
            torch.cuda.empty_cache()

    supplementary = None
    if args.workload == "decode_32k_x16" and not args.no_contexts and not args.no_supplementary:
        log("supplementary block-scoring shape: %d queries x %d representatives" % (SUPP_NQ, SUPP_L // 128))
        supplementary = supplementary_block_scoring(max(4, min(args.stage_steps, 8)), torch, hisa, device, synth)

    stream_peak = None
    if args.workload == "decode_32k_x16" and not args.no_stream_peak and not args.no_contexts:
        # after every timed region: what plain streaming kernels reach on this
        # GPU, beside the published peak, for the HBM rooflines
        log("plain streaming kernels over 4 GiB")
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        sc = stream_ceiling(4 << 30, torch)
        torch.cuda.empty_cache()
        ref = max(sc["copy"]["gbps"], sc["add_one"]["gbps"])
        stream_peak = {"bytes": sc["bytes"], "copy_gbps": sc["copy"]["gbps"],
                       "elementwise_copy_gbps": sc["add_one"]["gbps"],
                       "read_only_gbps": max(sc["read_sum"]["gbps"], sc["read_amax"]["gbps"],
                                             sc["read_gemv"]["gbps"]),
                       "reference_gbps": ref,
                       "note": "4 GiB per operand: the runtime's copy and an element-wise dst = src + 1 (bytes read "
                               "+ written), the best of a sum, a maximum and a matrix-vector product (bytes read); "
                               "frac_of_measured_stream in the HBM rooflines is achieved / reference_gbps, the "
                               "faster of the two copies"}
        for rf in [roof] + [c.get("roofline") for c in (contexts or {}).values() if isinstance(c, dict)]:
            if rf and rf.get("unit") == "GB/s":
                rf["frac_of_measured_stream"] = rf["achieved"] / ref

    out = {
        "metric": "indexer queries/s + HBM GB/s at 32K/128K/1M ctx; HISA vs flat-DSA speedup",
        "value": res["hisa"]["queries_per_s"],
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
        "config": {"workload": args.workload, "description": res["description"],
                   "queries_per_step": res["queries_per_step"],
                   "outputs": "int32 top-k indices (the optional scores and kept-block lists are not requested)",
                   "replicas": R, "B": res["B"], "m": res["m"], "k": res["k"]},
        "roofline": roof,
        "cpu_baseline": cpu,
        "step_bytes": res["hisa"]["step_bytes"],
        "hbm_gbps_step": res["hisa"]["hbm_gbps_step"],
        "kernels": res["hisa"]["kernels"],
        "flat": dict(res["flat"], value=res["flat"]["queries_per_s"], unit="queries/s"),
        "speedup_vs_flat": res["speedup_vs_flat"],
        "hisa_launch_forms_ms_per_step": res["hisa"]["launch_forms_ms_per_step"],
        "hisa_two_calls_ms_per_step": res["hisa"]["two_calls_ms_per_step"],
        "hisa_two_calls_kernels": res["hisa"]["two_calls_kernels"],
        "step_note": ("HISA decode steps are one hisa_decode_step call (the append in the same launch as the block "
                      "selection and token scores); hisa_two_calls_ms_per_step is the same step as append + index, "
                      "the form the flat indexer's step takes"
                      if res["hisa"]["two_calls_ms_per_step"] is not None else None),
        "timing_note": {"best": "each method's steps are timed in two launch forms and the faster counts, for HISA "
                                "and flat alike (launch_forms_ms_per_step holds both): eager, the calls queued back "
                                "to back on one stream with the host ahead of the GPU, every replica taking one "
                                "untimed step first; and one captured HIP graph replayed per step, every graph "
                                "replayed once first. The garbage collector is off inside timed regions.",
                        "eager": "steps launched eagerly, back to back on one stream; every replica takes one "
                                 "untimed step before the warmup and the timed steps",
                        "graph": "one captured graph replayed per step; every graph is replayed once before the "
                                 "warmup and the timed replays"}[LAUNCH],
        "warm": warm,
        "attention": attention,
        "lsa_flat": lsa,
        "contexts": contexts,
        "supplementary_block_scoring": supplementary,
        "stream_peak": stream_peak,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
