#!/usr/bin/env python3
"""Decode benchmark of the CSA / HCA hybrid attention hot path on one MI355X.

Workload (the 1M-context configuration): an interleaved stack of 8 attention
layers, CSA (m = 4, two-path compression, Lightning Indexer with 64 heads x
128, top-1024, 128-token window, sinks) alternating with HCA (m = 128, dense,
128-token window, sinks); 64 query heads x d = 512 sharing one KV head; bf16
storage, fp32 accumulation; n_ctx = 1,000,000 tokens; batch 16.  All eight
layers' compressed caches are resident in HBM (about 2.4 GB per sequence).

One step decodes the token at position t = n_ctx - 1 of every sequence
through all 8 layers.  Per CSA layer: csa_compress writes the entry whose
block the new token completes (K, V and index keys, two-path), then the
indexer scores every visible entry and keeps the top 1024 (csa_index_topk:
one scan kernel that also selects each part's candidates, then a merge
kernel), and csa_sparse_attn attends over them plus the window.  Per HCA layer: hca_compress refreshes the
newest complete 128-token entry (K and V) and hca_dense_attn attends over all
7812 visible entries plus the window.

Metric: queries/s, a query being one token of one sequence through the whole
8-layer stack (B queries per step), plus achieved HBM GB/s of the step and
the roofline of the dominant call (csa_index_topk: its scan kernel streams
the index keys and takes about nine tenths of the call), timed with HIP
events on the stream the kernels run on.  The CPU oracle is timed on a bounded
sample of the same step (a few sequences) as a reported baseline.

Usage: python bench.py [--steps K] [--warmup W] [--batch B] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

import synthetic as syn  # noqa: E402

HBM_PEAK_GBPS = 8000.0
SEED = 5


class Stack:
    """Shapes of the 8-layer decode workload."""

    def __init__(self, B=16, n_ctx=1_000_000, layers=8, eb=2):
        self.B, self.n_ctx, self.layers = B, n_ctx, layers
        self.eb = eb  # bytes per stored element: caches, window, indexer q/k, compression inputs
        self.H, self.d = 64, 512
        self.HI, self.dI = 64, 128
        self.k, self.W = 1024, 128
        self.m_csa, self.m_hca = 4, 128
        self.L_csa = -(-n_ctx // self.m_csa)
        self.L_hca = -(-n_ctx // self.m_hca)
        self.t = n_ctx - 1
        self.nv_csa = min(self.L_csa, self.t // self.m_csa)
        self.nv_hca = min(self.L_hca, self.t // self.m_hca)
        # CSA: the block holding t is complete after t arrives; its entry is new.
        self.csa_new = self.t // self.m_csa if (self.t + 1) % self.m_csa == 0 else self.nv_csa - 1
        # HCA: the newest complete 128-token entry (visible to t).
        self.hca_new = self.nv_hca - 1
        self.scale = 1.0 / math.sqrt(self.d)

    def kinds(self):
        return ["csa" if i % 2 == 0 else "hca" for i in range(self.layers)]

    # ---- algorithmic bytes (what the method must move), per query ----------
    def index_bytes(self):
        """csa_index_topk per query: the visible indexer keys, the query's
        index heads and head weights, the selected indices written."""
        return self.nv_csa * self.dI * self.eb + self.HI * self.dI * self.eb + self.HI * 4 + self.k * 4

    def csa_bytes(self):
        b = self.index_bytes()
        e = self.eb
        b += self.k * self.d * 2 * e            # gathered compressed K and V rows
        b += self.W * self.d * 2 * e            # raw window K and V
        b += 2 * self.H * self.d * 2            # q and out (bf16)
        b += self.k * 4                         # selected indices, read by the attention
        m = self.m_csa
        b += 4 * m * (2 * self.d + self.dI) * e  # compress: x/z, A and B paths, K V I
        b += (2 * self.d + self.dI) * e         # new entries
        return b

    def hca_bytes(self):
        e = self.eb
        b = self.nv_hca * self.d * 2 * e + self.W * self.d * 2 * e + 2 * self.H * self.d * 2
        b += 2 * 2 * self.m_hca * self.d * e + 2 * self.d * e  # compress K, V
        return b

    def step_bytes(self):
        per = sum(self.csa_bytes() if k == "csa" else self.hca_bytes() for k in self.kinds())
        return per * self.B


def raw_rows(st: Stack, name, layer, p0, cnt, D, device, scale, dtype=torch.bfloat16):
    """Rows p0 .. p0+cnt-1 of a virtual raw stream [B][n_ctx][D]."""
    b = torch.arange(st.B, dtype=torch.int64, device=device).reshape(-1, 1)
    p = torch.arange(p0, p0 + cnt, dtype=torch.int64, device=device).reshape(1, -1)
    r = (b * st.n_ctx + p).reshape(-1)
    return syn.rows((st.B, st.n_ctx, D), r, SEED, syn.TID[name], dtype=dtype, device=device,
                    scale=scale, layer=layer).reshape(st.B, cnt, D)


class GpuState:
    """All device buffers of the workload, generated in place on the GPU."""

    def __init__(self, st: Stack, device="cuda"):
        """st.eb == 2: bf16 storage.  st.eb == 1: FP8 (E4M3) storage of the
        caches, the window, the indexer's q and keys and the compression
        inputs; the attention query and output stay bf16.  FP8 K/V rows are
        unit-scale codes with the K scale 1/sqrt(d) folded into the softmax
        scale (the V scale would fold into the output's consumer)."""
        import compressed_sparse_kv_compress_amd as csa
        self.csa = csa
        self.st = st
        bf = torch.bfloat16
        sto = bf if st.eb == 2 else torch.float8_e4m3fn
        B, d, dI, H = st.B, st.d, st.dI, st.H
        si = dI ** -0.5
        sd = d ** -0.5 if st.eb == 2 else 1.0          # K/V value scale
        self.ascale = st.scale if st.eb == 2 else st.scale * d ** -0.5
        dt_code = csa.CSA_BF16 if st.eb == 2 else csa.CSA_FP8
        self.layers = []
        for li, kind in enumerate(st.kinds()):
            L = st.L_csa if kind == "csa" else st.L_hca
            lay = {"kind": kind}

            def gen(shape, name, scale, dtype=bf, li=li):
                t = torch.empty(shape, dtype=dtype, device=device)
                return syn.fill_(t, SEED, syn.TID[name], scale=scale, layer=li)

            lay["kc"] = gen((B, L, d), "kc", sd, sto)
            lay["vc"] = gen((B, L, d), "vc", sd, sto)
            lay["q"] = gen((B, 1, H, d), "q", d ** -0.5)
            lay["sink"] = gen((H,), "sink", 1.0, torch.float32)
            lay["kr"] = raw_rows(st, "kr", li, st.n_ctx - st.W, st.W, d, device, sd, sto)
            lay["vr"] = raw_rows(st, "vr", li, st.n_ctx - st.W, st.W, d, device, sd, sto)
            lay["out"] = torch.empty((B, 1, H, d), dtype=bf, device=device)
            if kind == "csa":
                m = st.m_csa
                lay["ki"] = gen((B, L, dI), "kic", si, sto)
                lay["qi"] = gen((B, 1, st.HI, dI), "q_idx", si, sto)
                lay["wi"] = gen((B, 1, st.HI), "w_idx", st.HI ** -0.5, torch.float32)
                p0 = (st.csa_new - 1) * m
                for s, D, sc in (("k", d, sd), ("v", d, sd), ("idx", dI, si)):
                    xa = "k" if s == "k" else ("v" if s == "v" else "k_idx")
                    lay["raw_" + s] = (
                        raw_rows(st, xa, li, p0, 2 * m, D, device, sc, sto),
                        raw_rows(st, "z_" + s, li, p0, 2 * m, D, device, 0.5, sto),
                        raw_rows(st, "xb_" + s, li, p0, 2 * m, D, device, sc, sto),
                        raw_rows(st, "zb_" + s, li, p0, 2 * m, D, device, 0.5, sto))
                lay["p0"] = p0
                lay["idx"] = torch.empty((B, 1, st.k), dtype=torch.int32, device=device)
                lay["itk_ws"] = torch.empty(max(16, csa.csa_index_topk_workspace(B, 1, L, st.k)),
                                            dtype=torch.uint8, device=device)
                nb = csa.csa_sparse_attn_workspace(B, 1, H, d, st.k, st.W, dt_code)
            else:
                m = st.m_hca
                p0 = st.hca_new * m
                lay["raw_k"] = (raw_rows(st, "k", li, p0, m, d, device, sd, sto),
                                raw_rows(st, "z_k", li, p0, m, d, device, 0.5, sto))
                lay["raw_v"] = (raw_rows(st, "v", li, p0, m, d, device, sd, sto),
                                raw_rows(st, "z_v", li, p0, m, d, device, 0.5, sto))
                lay["p0"] = p0
                nb = csa.hca_dense_attn_workspace(B, 1, H, d, L, m, st.n_ctx, st.W, dt_code)
            lay["ws"] = torch.empty(max(nb, 16), dtype=torch.uint8, device=device)
            self.layers.append(lay)
        self.side = torch.cuda.Stream(device=device)  # default priority
        torch.cuda.synchronize()

    def step(self, ev=None, only=None, csa_layer=None):
        """One decode step through all layers.

        Compression runs on a second stream: its inputs are raw tokens of
        blocks that are already complete, so it overlaps the HBM-bound indexer
        scan.  The CSA entry written by this step is not visible to the current
        token; the HCA refresh is joined (event wait) before that layer's dense
        attention reads it.  ev: optional dict of event lists keyed by call
        name; events bracket calls (all, or the names in `only`) on the stream
        that runs them; csa_layer: bracket only that CSA layer's calls (every
        timing event costs a few microseconds of idle GPU between kernels)."""
        csa, st = self.csa, self.st
        main = torch.cuda.current_stream()
        side = self.side
        side.wait_stream(main)

        def mark(name, ci=None):
            if ev is None or (only is not None and name.replace("_end", "") not in only):
                return
            if csa_layer is not None and ci != csa_layer:
                return
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            ev.setdefault(name, []).append(e)

        joins = []
        with torch.cuda.stream(side):
            for lay in self.layers:
                if lay["kind"] == "csa":
                    m = st.m_csa
                    mark("csa_compress")
                    for s, cache in (("k", "kc"), ("v", "vc"), ("idx", "ki")):
                        xa, za, xb, zb = lay["raw_" + s]
                        L = lay[cache].shape[1]
                        csa.csa_compress(xa, za, m, x_b=xb, z_b=zb, n=st.n_ctx, p0=lay["p0"], e0=st.csa_new,
                                         e1=st.csa_new + 1, out=lay[cache][:, st.csa_new:], out_ld=L)
                    mark("csa_compress_end")
                    joins.append(None)
                else:
                    m = st.m_hca
                    mark("hca_compress")
                    for s, cache in (("k", "kc"), ("v", "vc")):
                        x, z = lay["raw_" + s]
                        L = lay[cache].shape[1]
                        csa.hca_compress(x, z, m, n=st.n_ctx, p0=lay["p0"], e0=st.hca_new,
                                         e1=st.hca_new + 1, out=lay[cache][:, st.hca_new:], out_ld=L)
                    mark("hca_compress_end")
                    done = torch.cuda.Event()
                    done.record()
                    joins.append(done)

        ci = 0
        for lay, done in zip(self.layers, joins):
            if lay["kind"] == "csa":
                m = st.m_csa
                mark("index_topk", ci)
                csa.csa_index_topk(lay["qi"], lay["ki"], m, st.k, w_idx=lay["wi"], n_ctx=st.n_ctx, idx=lay["idx"],
                                   ws=lay["itk_ws"])
                mark("index_topk_end", ci)
                ci += 1
                mark("csa_sparse_attn")
                csa.csa_sparse_attn(lay["q"], lay["kc"], lay["vc"], lay["idx"], kr=lay["kr"], vr=lay["vr"],
                                    W=st.W, sink=lay["sink"], scale=self.ascale, n_ctx=st.n_ctx, out=lay["out"],
                                    ws=lay["ws"])
                mark("csa_sparse_attn_end")
            else:
                m = st.m_hca
                main.wait_event(done)
                mark("hca_dense_attn")
                csa.hca_dense_attn(lay["q"], lay["kc"], lay["vc"], m, kr=lay["kr"], vr=lay["vr"], W=st.W,
                                   sink=lay["sink"], scale=self.ascale, n_ctx=st.n_ctx, out=lay["out"], ws=lay["ws"])
                mark("hca_dense_attn_end")
        main.wait_stream(side)


def event_means_ms(ev):
    """Average duration per call name (ms) from start/end event pairs."""
    res = {}
    for name, starts in ev.items():
        if name.endswith("_end"):
            continue
        ends = ev[name + "_end"]
        ts = [a.elapsed_time(b) for a, b in zip(starts, ends)]
        res[name] = sum(ts) / len(ts)
    return res


INDEX_TOPK_SOURCES = [os.path.join(ROOT, "compressed_sparse_kv_compress_amd", "csrc", f)
                      for f in ("index.hip", "topk.hip", "select.hpp", "common.hpp")]


def source_hash(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic(kernel_src, per_launch_units):
    """HBM bytes per csa_index_topk call (its two kernels) from the committed
    rocprofv3 counter summary, or None when it is missing or the kernels'
    sources changed since."""
    path = os.path.join(ROOT, "profiles", "index_topk_stack8_b16_counters.txt")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_src = re.search(r"^source_sha256_16:\s*(\w+)", txt, re.M)
    m_b = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt, re.M)
    m_u = re.search(r"^queries_per_launch:\s*(\d+)", txt, re.M)
    if not (m_src and m_b and m_u) or m_src.group(1) != source_hash(kernel_src):
        return None
    return float(m_b.group(1)) * per_launch_units / int(m_u.group(1))


def cpu_baseline(st: Stack, sample: int, min_seconds: float = 10.0, max_reps: int = 8):
    """Time the CPU oracle on `sample` sequences of the same decode step.

    Inputs are regenerated on the CPU from the same seeds, layer by layer (not
    timed); the oracle calls of a layer (compression of the new entries,
    indexer + top-k and sparse attention, or dense attention) are timed and
    repeated on the same inputs until the layer has had its share of
    min_seconds (at most max_reps times).  The step time is the sum over
    layers of the mean time per repetition."""
    bf = torch.bfloat16
    S = min(sample, st.B)
    sd, si = st.d ** -0.5, st.dI ** -0.5

    def full(shape, name, scale, li, rows=None, dtype=bf):
        D = shape[-1]
        if rows is None:
            return syn.make(shape, SEED, syn.TID[name], dtype=dtype, scale=scale, layer=li).double().numpy()
        return syn.rows(shape, rows, SEED, syn.TID[name], dtype=dtype, scale=scale,
                        layer=li).double().numpy().reshape(-1, D)

    sub = Stack(B=S, n_ctx=st.n_ctx, layers=st.layers)
    per_layer = min_seconds / st.layers
    step_s, total, reps_all = 0.0, 0.0, []
    for li, kind in enumerate(st.kinds()):
        t_layer, reps = _oracle_layer(st, sub, S, full, sd, si, li, kind, per_layer, max_reps)
        step_s += t_layer / reps
        total += t_layer
        reps_all.append(reps)
        print("# cpu oracle: layer %d (%s) %.2f s over %d repetition(s)" % (li, kind, t_layer, reps),
              file=sys.stderr, flush=True)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": S / step_s, "unit": "queries/s", "cores": min(S, threads), "kind": "oracle",
            "sample": "%d of %d sequences, one decode step through all %d layers, each layer's oracle calls "
                      "repeated %s times on the same inputs (%.1f s of oracle time)"
                      % (S, st.B, st.layers, "/".join(map(str, reps_all)), total)}


def _oracle_layer(st, sub, S, full, sd, si, li, kind, min_seconds, max_reps):
    """Oracle calls of one layer of the decode step for S sequences, repeated
    until min_seconds (at most max_reps times); returns (seconds, repetitions),
    input regeneration excluded."""
    import numpy as np

    import oracle
    L = st.L_csa if kind == "csa" else st.L_hca
    seq_rows = lambda b, n: np.arange(b * n, (b + 1) * n)  # noqa: E731
    q = np.stack([full((st.B, 1, st.H, st.d), "q", sd, li, rows=np.arange(b * st.H, (b + 1) * st.H))
                  for b in range(S)]).reshape(S, 1, st.H, st.d)
    sink = full((st.H,), "sink", 1.0, li, dtype=torch.float32)
    kr = np.stack([raw_rows(sub, "kr", li, st.n_ctx - st.W, st.W, st.d, "cpu", sd)[b].double().numpy()
                   for b in range(S)])
    vr = np.stack([raw_rows(sub, "vr", li, st.n_ctx - st.W, st.W, st.d, "cpu", sd)[b].double().numpy()
                   for b in range(S)])
    total, reps = 0.0, 0
    if kind == "csa":
        m = st.m_csa
        p0 = (st.csa_new - 1) * m
        raws = {}
        for s, D, sc in (("k", st.d, sd), ("v", st.d, sd), ("idx", st.dI, si)):
            xa = "k" if s == "k" else ("v" if s == "v" else "k_idx")
            raws[s] = [raw_rows(sub, nm, li, p0, 2 * m, D, "cpu", scl).double().numpy()
                       for nm, scl in ((xa, sc), ("z_" + s, 0.5), ("xb_" + s, sc), ("zb_" + s, 0.5))]
        ki = np.stack([full((st.B, L, st.dI), "kic", si, li, rows=seq_rows(b, L)) for b in range(S)])
        qi = np.stack([full((st.B, 1, st.HI, st.dI), "q_idx", si, li,
                            rows=np.arange(b * st.HI, (b + 1) * st.HI)) for b in range(S)])
        qi = qi.reshape(S, 1, st.HI, st.dI)
        wi = np.stack([full((st.B, 1, st.HI), "w_idx", st.HI ** -0.5, li, dtype=torch.float32,
                            rows=np.arange(b, b + 1)) for b in range(S)]).reshape(S, 1, st.HI)
        kc = vc = loc = None
        while reps < max_reps and (reps == 0 or total < min_seconds):
            reps += 1
            t0 = time.perf_counter()
            for s in ("k", "v", "idx"):
                xa, za, xb, zb = raws[s]
                oracle.compress(xa, za, m, x_b=xb, z_b=zb, n=st.n_ctx, p0=p0, e0=st.csa_new,
                                e1=st.csa_new + 1)
            idx, _ = oracle.index_topk(qi, ki, m, st.k, w=wi, n_ctx=st.n_ctx)
            total += time.perf_counter() - t0
            if kc is None:  # gather only the selected rows of the compressed K/V caches (not timed)
                kc = np.zeros((S, st.k, st.d))
                vc = np.zeros((S, st.k, st.d))
                loc = np.full_like(idx, -1)
                for b in range(S):
                    sel = idx[b, 0][idx[b, 0] >= 0]
                    kc[b, :len(sel)] = full((st.B, L, st.d), "kc", sd, li, rows=b * L + sel)
                    vc[b, :len(sel)] = full((st.B, L, st.d), "vc", sd, li, rows=b * L + sel)
                    loc[b, 0, :len(sel)] = np.arange(len(sel))
            t0 = time.perf_counter()
            oracle.sparse_attn(q, kc, vc, loc, kr, vr, st.W, sink=sink, n_ctx=st.n_ctx)
            total += time.perf_counter() - t0
    else:
        m = st.m_hca
        p0 = st.hca_new * m
        raws = [raw_rows(sub, nm, li, p0, m, st.d, "cpu", scl).double().numpy()
                for nm, scl in (("k", sd), ("z_k", 0.5), ("v", sd), ("z_v", 0.5))]
        kc = np.stack([full((st.B, L, st.d), "kc", sd, li, rows=seq_rows(b, L)) for b in range(S)])
        vc = np.stack([full((st.B, L, st.d), "vc", sd, li, rows=seq_rows(b, L)) for b in range(S)])
        while reps < max_reps and (reps == 0 or total < min_seconds):
            reps += 1
            t0 = time.perf_counter()
            oracle.compress(raws[0], raws[1], m, n=st.n_ctx, p0=p0, e0=st.hca_new, e1=st.hca_new + 1)
            oracle.compress(raws[2], raws[3], m, n=st.n_ctx, p0=p0, e0=st.hca_new, e1=st.hca_new + 1)
            oracle.dense_attn(q, kc, vc, m, kr, vr, st.W, sink=sink, n_ctx=st.n_ctx)
            total += time.perf_counter() - t0
    return total, reps


def prefill_sparse_attn(queries: int, reps: int = 3):
    """Prefill-chunk sparse attention (the CSA prefill shape: `queries` new
    tokens after a 262,144-token prefix, m = 4, 64 heads x 512 on one KV head,
    top-1024 + 128-token window, sinks).  The index lists are seeded uniform
    draws of 1024 visible entries per query, ascending (what the top-k of the
    seeded random indexer inputs is, statistically); inputs are generated on
    the GPU.  Returns the average call time and its MFMA / gather rates."""
    import compressed_sparse_kv_compress_amd as csa
    dev = "cuda"
    B, H, d, k, W, m = 1, 64, 512, 1024, 128, 4
    T = queries
    n_ctx = 262144 + T
    L = -(-n_ctx // m)
    R = T + W - 1
    bf = torch.bfloat16

    def gen(shape, name, scale, dtype=bf, kind="normal"):
        t = torch.empty(shape, dtype=dtype, device=dev)
        return syn.fill_(t, SEED, syn.TID[name], scale=scale, layer=0, kind=kind)

    sd = d ** -0.5
    q = gen((B, T, H, d), "q", sd)
    kc, vc = gen((B, L, d), "kc", sd), gen((B, L, d), "vc", sd)
    kr, vr = gen((B, R, d), "kr", sd), gen((B, R, d), "vr", sd)
    sink = gen((H,), "sink", 1.0, torch.float32)
    u = gen((B, T, k), "idx", 1.0, torch.float32, kind="uniform")  # seeded draws in [0, 1)
    nv = (torch.arange(n_ctx - T, n_ctx, device=dev) // m).clamp(max=L)
    idx = (u.double() * nv.view(1, T, 1)).long().sort(-1).values.int()
    out = torch.empty_like(q)
    ws = torch.empty(max(16, csa.csa_sparse_attn_workspace(B, T, H, d, k, W, csa.CSA_BF16)), dtype=torch.uint8,
                     device=dev)
    call = lambda: csa.csa_sparse_attn(q, kc, vc, idx, kr=kr, vr=vr, W=W, sink=sink, n_ctx=n_ctx,  # noqa: E731
                                       out=out, ws=ws)
    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    rows = k + W
    flop = 2 * 2 * B * T * H * rows * d
    gathered = B * T * rows * d * 2 * 2
    del q, kc, vc, kr, vr, out, ws, idx, u
    torch.cuda.empty_cache()
    return {"queries": T, "prefix": 262144, "ms_per_call": ms,
            "tflops": flop / (ms * 1e-3) / 1e12, "peak_tflops_bf16": 2500.0,
            "frac_of_bf16_peak": flop / (ms * 1e-3) / 1e12 / 2500.0,
            "gathered_GB": gathered / 1e9, "gathered_TBps": gathered / (ms * 1e-3) / 1e12,
            "note": "per query 1152 K and V rows of 1 KiB gathered (no reuse across queries beyond the window: "
                    "the index lists are independent uniform draws); flop = 4 * queries * heads * rows * d, "
                    "64 flop per gathered byte, so gather-bound: random 1 KiB gathers from the Infinity Cache "
                    "top out near 7.3 TB/s on this GPU, i.e. about 18.7% of the bf16 peak"}


def fp8_storage_step(B: int, steps: int, warmup: int):
    """The same 8-layer decode step with FP8 (E4M3) storage: reported beside
    the bf16 headline, never as it."""
    st = Stack(B=B, eb=1)
    state = GpuState(st)
    for _ in range(warmup):
        state.step()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        state.step()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    ev = {}
    for _ in range(3):
        state.step(ev)
    torch.cuda.synchronize()
    per_call = event_means_ms(ev)
    del state
    torch.cuda.empty_cache()
    idx_bytes = st.index_bytes() * st.B
    return {
        "storage": "E4M3 caches, window, indexer q/k and compression inputs; bf16 query and output",
        "ms_per_step": ms, "queries_per_s": st.B / (ms * 1e-3),
        "algorithmic_bytes_per_step": st.step_bytes(),
        "achieved_GBps": st.step_bytes() / (ms * 1e-3) / 1e9,
        "index_topk_GBps": idx_bytes / (per_call["index_topk"] * 1e-3) / 1e9,
        "per_call_ms": per_call,
        "note": "attention converts each E4M3 row to bf16 before the bf16 MFMA sequence; at B=16 the decode "
                "attention kernels are bound by their per-stage chain, not by bytes, so the gain comes "
                "from the indexer scan",
    }


def prefill_index_topk(queries: int = 4096, reps: int = 3):
    """csa_index_topk on the CSA prefill-chunk shape: the last `queries` of a
    65,536-token chunk after a 262,144-token prefix (81,920 compressed
    entries, about 82 K visible per query), 64 index heads x 128, k = 1024."""
    import compressed_sparse_kv_compress_amd as csa
    HI, dI, m, k = 64, 128, 4, 1024
    prefix, chunk = 262144, 65536
    n_ctx = prefix + chunk
    L = n_ctx // m
    ki = syn.fill_(torch.empty((1, L, dI), dtype=torch.bfloat16, device="cuda"), 4, syn.TID["kic"], scale=dI ** -0.5)
    qi = syn.fill_(torch.empty((1, queries, HI, dI), dtype=torch.bfloat16, device="cuda"), 4, syn.TID["q_idx"],
                   scale=dI ** -0.5)
    wi = syn.fill_(torch.empty((1, queries, HI), device="cuda"), 4, syn.TID["w_idx"], scale=HI ** -0.5)
    ws = torch.empty(csa.csa_index_topk_workspace(1, queries, L, k), dtype=torch.uint8, device="cuda")
    idx = torch.empty((1, queries, k), dtype=torch.int32, device="cuda")

    def call():
        csa.csa_index_topk(qi, ki, m, k, w_idx=wi, n_ctx=n_ctx, idx=idx, ws=ws)

    call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    t = torch.arange(n_ctx - queries, n_ctx, dtype=torch.float64)
    pairs = float(torch.clamp(torch.floor(t / m), max=L).sum())
    flop = pairs * HI * dI * 2
    del ki, qi, ws
    torch.cuda.empty_cache()
    return {"queries": queries, "entries": L, "ms_per_call": ms, "tflops": flop / (ms * 1e-3) / 1e12,
            "peak_tflops_bf16": 2500.0, "frac_of_bf16_peak": flop / (ms * 1e-3) / 1e12 / 2500.0,
            "visible_pairs": pairs,
            "note": "flop = 2 * visible (query, entry) pairs * index heads * index dim; scores by the 16-row "
                    "prefill kernel (each key tile read once per 16 queries), then the stand-alone top-k "
                    "(about a fifth of the time)"}


def decode_step_b1(steps: int, warmup: int):
    """The same bf16 8-layer step for one sequence (B = 1): the latency-bound
    end of the decode workload, reported beside the B = 16 headline."""
    st = Stack(B=1)
    state = GpuState(st)
    for _ in range(warmup):
        state.step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        state.step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    ev = {}
    for _ in range(3):
        state.step(ev)
    torch.cuda.synchronize()
    per_call = event_means_ms(ev)
    del state
    torch.cuda.empty_cache()
    return {"ms_per_step": ms, "tokens_per_s": 1.0 / (ms * 1e-3),
            "algorithmic_bytes_per_step": st.step_bytes(),
            "achieved_GBps": st.step_bytes() / (ms * 1e-3) / 1e9, "per_call_ms": per_call,
            "note": "one query per call: bound by launch latency and by the stand-alone top-k (with one "
                    "query row the single-pass scan-and-select plan does not apply)"}


def index_topk_mxfp4(B: int, reps: int = 20):
    """One csa_index_topk call of the CSA decode shape with q^I and k^I in
    MXFP4 (random E2M1 codes, E8M0 scales 2^-2 .. 2^2), timed over `reps`
    back-to-back calls: reported beside the bf16 headline, never as it."""
    import compressed_sparse_kv_compress_amd as csa
    st = Stack(B=B)
    L, HI, dI, k, m = st.L_csa, st.HI, st.dI, st.k, st.m_csa
    nq, nk = B * HI * dI, B * L * dI
    qb = syn.mxfp4_(torch.empty(nq // 2 + nq // 32, dtype=torch.uint8, device="cuda"), SEED, syn.TID["q_idx"], nq,
                    scale_lo=125, scale_hi=129)
    kb = syn.mxfp4_(torch.empty(nk // 2 + nk // 32, dtype=torch.uint8, device="cuda"), SEED, syn.TID["kic"], nk,
                    scale_lo=125, scale_hi=129)
    q, kk = csa.MXFP4(qb, (B, 1, HI, dI)), csa.MXFP4(kb, (B, L, dI))
    w = syn.fill_(torch.empty((B, 1, HI), device="cuda"), SEED, syn.TID["w_idx"], scale=HI ** -0.5)
    idx = torch.empty((B, 1, k), dtype=torch.int32, device="cuda")
    ws = torch.empty(csa.csa_index_topk_workspace(B, 1, L, k), dtype=torch.uint8, device="cuda")

    def call():
        csa.csa_index_topk(q, kk, m, k, w_idx=w, n_ctx=st.n_ctx, idx=idx, ws=ws)

    for _ in range(3):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    key_bytes = dI // 2 + dI // 32
    byts = B * (st.nv_csa * key_bytes + HI * key_bytes + HI * 4 + k * 4)
    del qb, kb, ws
    torch.cuda.empty_cache()
    return {"ms_per_call": ms, "algorithmic_bytes_per_call": byts, "GBps": byts / (ms * 1e-3) / 1e9,
            "keys": "16 x %d visible keys of 68 B (64 code bytes + 4 scales), k = %d" % (st.nv_csa, k),
            "note": "scan bound by its per-tile MFMA and epilogue chain (one wavefront per SIMD), not by bytes"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--batch", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=2)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle step until at least this much oracle time")
    ap.add_argument("--prefill-queries", type=int, default=16384,
                    help="queries of the prefill sparse-attention measurement (0: skip)")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8-storage step")
    ap.add_argument("--no-batch1", action="store_true", help="skip the batch-1 decode step")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="first run a plain device copy of BYTES bytes 3 times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(sharding and collectives are out of scope); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.empty(args.copy_calibration, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print("# calibration copy of %d bytes done" % args.copy_calibration, file=sys.stderr, flush=True)
    st = Stack(B=args.batch)
    t_gen = time.perf_counter()
    state = GpuState(st)
    t_gen = time.perf_counter() - t_gen
    print("# inputs generated on the GPU in %.1f s" % t_gen, file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        state.step()
    torch.cuda.synchronize()
    print("# warmup done", file=sys.stderr, flush=True)

    # Timed region: K steps; HIP events bracket one csa_index_topk call (the
    # dominant call) per step, on the stream it runs on, taking the CSA layers
    # in turn.
    ev = {}
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    n_csa = st.kinds().count("csa")
    for i in range(args.steps):
        state.step(ev, only=("index_topk",), csa_layer=i % n_csa)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = start.elapsed_time(stop) / args.steps
    idx_ms = event_means_ms(ev)["index_topk"]
    print("# timed %d steps: %.3f ms/step (wall %.3f ms/step)" % (args.steps, ms_step, 1e3 * wall / args.steps),
          file=sys.stderr, flush=True)
    # Untimed breakdown pass: every call bracketed by events.
    ev_all = {}
    for _ in range(3):
        state.step(ev_all)
    torch.cuda.synchronize()
    per_call = event_means_ms(ev_all)

    value = st.B / (ms_step * 1e-3)
    step_gbps = st.step_bytes() / (ms_step * 1e-3) / 1e9
    idx_bytes = st.index_bytes() * st.B
    idx_gbps = idx_bytes / (idx_ms * 1e-3) / 1e9
    traffic = counter_traffic(INDEX_TOPK_SOURCES, st.B)

    del state
    torch.cuda.empty_cache()
    fp8 = None
    if not args.no_fp8:
        fp8 = fp8_storage_step(args.batch, args.steps, args.warmup)
        print("# fp8 storage: %.3f ms/step" % fp8["ms_per_step"], file=sys.stderr, flush=True)
        fp8["index_topk_mxfp4"] = index_topk_mxfp4(args.batch)
        print("# mxfp4 index_topk: %.3f ms/call" % fp8["index_topk_mxfp4"]["ms_per_call"], file=sys.stderr,
              flush=True)

    b1 = None
    if args.batch != 1 and not args.no_batch1:
        b1 = decode_step_b1(args.steps, args.warmup)
        print("# batch 1: %.3f ms/step" % b1["ms_per_step"], file=sys.stderr, flush=True)

    prefill = None
    if args.prefill_queries > 0:
        prefill = prefill_sparse_attn(args.prefill_queries)
        prefill["index_topk"] = prefill_index_topk()
        print("# prefill index + top-k: %.2f ms (%.0f TFLOP/s)" % (prefill["index_topk"]["ms_per_call"],
              prefill["index_topk"]["tflops"]), file=sys.stderr, flush=True)
        print("# prefill sparse attention: %.2f ms for %d queries (%.0f TFLOP/s)"
              % (prefill["ms_per_call"], prefill["queries"], prefill["tflops"]), file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(st, args.cpu_sample, args.cpu_seconds)

    line = {
        "metric": "CSA/HCA decode queries/s at 1M ctx + achieved HBM GB/s (% peak)",
        "value": value,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)/sqrt(dim) tensors, compressed caches generated in HBM)",
        "config": {
            "workload": "csa_hca_stack8_decode_1M",
            "query": "one token of one sequence through all 8 layers",
            "batch": st.B, "n_ctx": st.n_ctx, "layers": "4 CSA (two-path m=4) + 4 HCA (m=128), alternating",
            "heads": st.H, "head_dim": st.d, "index_heads": st.HI, "index_dim": st.dI, "top_k": st.k,
            "window": st.W, "csa_entries": st.L_csa, "hca_entries": st.L_hca,
        },
        "hbm": {"algorithmic_bytes_per_step": st.step_bytes(), "achieved_GBps": step_gbps,
                "frac_of_peak": step_gbps / HBM_PEAK_GBPS},
        "roofline": {"kernel": "csa_index_topk (index_score_stream<4,true,true,0> then topk_merge_kernel)",
                     "bound": "hbm", "achieved": idx_gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": idx_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic, "avg_launch_ms": idx_ms,
                     "algorithmic_bytes_per_launch": idx_bytes},
        "per_call_ms": per_call,
        "per_call_note": "untimed pass with events around every call; compression runs on a second stream",
        "prefill_sparse_attn": prefill,
        "fp8_storage": fp8,
        "decode_batch1": b1,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
